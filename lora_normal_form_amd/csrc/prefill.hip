// MFMA prefill path (bf16 activations, fp32 accumulate, long adapter
// segments; d_in a multiple of 64, and of 256 when a row rotates or has a
// low-rank term).
//
// Two kernels per forward.
//
// k_prefill_prologue works on items of one work-group (4 waves) each:
//   shrink       t = x A' for 64 rows of a segment x 64 own ranks, and
//   VeRA shrink  u = (x A_sh) (.) d for 64 VeRA rows x 64 ranks, both over
//                one K part of 1024 on 32x32x16 bf16 MFMA, operands staged in
//                LDS by direct loads; each part writes its fp32 partial
//                tile, and the last part of a tile to arrive adds the parts
//                in part order (so every forward gives the same bits, at any
//                input scale fp32 holds) and converts the sums to bf16 for
//                the main kernel;
//   rotation     Delta = x (R - I) for 32 rotated rows x 256 columns; R is
//                block diagonal, so each 32-column MFMA block contracts over
//                one diagonal block.
//
// k_prefill_main computes one tile of 128 staged rows by 256 output columns
// per work-group of 4 waves, over the whole K dimension. A chunk (the tile's
// rows) belongs to one adapter segment: up to 128 tokens, or up to 64 tokens
// followed by their 64 Delta rows when the adapter rotates. Wave w owns
// columns 64 w .. 64 w + 63 of the tile (two 32-column MFMA blocks) for all
// 128 rows, so its accumulators are 4 row groups x 2 column blocks of
// 32x32x16 bf16 MFMA tiles.
//   K loop   stages of 64 k: the 128 rows (gathered by token from x, or the
//            Delta rows) and the tile's 256 W rows land in a 3-slot LDS ring
//            by direct buffer->LDS loads (each instruction moves 8 whole
//            128-byte row segments), two stages ahead; both MFMA operands are
//            read from LDS. The loop is unrolled at compile time so every
//            wait is exact.
//   epilogue Delta W folds into the token rows (rows 64 + r onto r, in
//            registers), the base product is scaled by s, the expand runs as
//            extra MFMA steps: A = the chunk's shrink sums (bf16, staged
//            through the ring in pieces of 64 ranks), B = the
//            adapter's B' rows, or the shared B_sh rows scaled by e (VeRA:
//            ((x A_sh) (.) d) B_sh (.) e, with e folded into B per column),
//            then b is added and the token rows are stored.
// The pages' order of operations holds: ((x R) W) (.) s + b plus the
// low-rank terms, which are not scaled by s ("The big picture",
// paper-daily.com explainer of "Scute: Exact Batched Serving for PEFT
// Adapters Beyond LoRA").

#include <algorithm>

#include "internal.h"
#include "kernels.h"

namespace scute {

namespace {

struct PfArgs {
  const uint16_t* x;       // [n][d_in] rows in batch (token) order
  const uint16_t* dx;      // [np][n_rot][d_in] Delta rows by sorted position, one block per
                           // projection (np = 1 unless a row rotates per projection)
  const uint16_t* W;       // [d_out][d_in]
  const PfChunk* chunks;   // [n_chunks]
  const int32_t* crow;     // [n_chunks][128] row sources: token, or -(Delta row) - 1
  const uint16_t* B_sh;    // [d_out][r_v]
  const uint16_t* tbf;     // [n][AW] shrink sums in bf16: RT own ranks, then r_v VeRA ranks
  float* y;                // [n][d_out]
  const int4* items;        // per work-group: column tile, chunk, K part (-1: all), exchange slot
  float* part;              // [n_split][P][32][256] f32x4 partial tiles
  int32_t* cnt;             // [n_split] arrival counters, kept at zero between forwards
  uint32_t acc_bytes, x_bytes, dx_bytes, part_bytes;  // dx_bytes: one block
  int32_t d_in, d_out, RT, AW, r_v, P;
  int32_t nst;  // 64-k stages of the whole K dimension (d_in / 64)
  int32_t n_rot;                // rows of a Delta block
  int32_t ptile[MAX_PROJ - 1];  // first column tile of projections 1.. (past the last tile if none)
};

constexpr int PK = 64;              // k per stage
constexpr int PROW = 2 * PK;        // bytes per staged row
constexpr int PSTAGE_X = 128 * PROW;  // staged rows of a stage
constexpr int PSTAGE = PSTAGE_X + 256 * PROW;  // rows, then the 256 W rows (columns)

// Staged row r of a stage (x / Delta row, or W row = output column): 8
// pieces of 16 bytes, piece p stored at position p ^ ((r >> 1) & 7) to
// spread LDS banks. One direct-to-LDS instruction fills 8 rows (lane i ->
// row i / 8, position i % 8); wave w issues instructions w, w + 4, w + 8, ..
// of each part. Rows are gathered by token through a per-lane offset; W rows
// are contiguous, so one per-lane offset plus a scalar offset per instruction
// addresses them. (Loads in the MFMA operand layout, one W row per lane,
// move half as many bytes per second on this part; register loads written
// to LDS by the waves cost more LDS time than the direct loads.)
struct PfSrc {
  rsrc_t rlo, rhi, rw;  // staged rows 0..63 (x), rows 64..127 (x or Delta), W rows
  uint32_t roff[4];     // per-lane byte offsets of this wave's 4 row pieces
  uint32_t woff;        // per-lane byte offset of its W piece in instruction 0
  uint32_t wstep;       // bytes between consecutive W instructions (32 W rows)
  int32_t kb;           // byte offset of stage 0 in every row (K part of a split tile)
};
__device__ __forceinline__ void pf_stage(uint8_t* slot, const PfSrc& src, int stage, int w) {
  const int soff = src.kb + stage * PK * 2;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(q >= 2 ? src.rhi : src.rlo,
                                             (lds_void*)(slot + (w + 4 * q) * 1024), 16,
                                             src.roff[q], soff, 0, 0);
#pragma unroll
  for (int q = 0; q < 8; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.rw, (lds_void*)(slot + PSTAGE_X + (w + 4 * q) * 1024),
                                             16, src.woff, soff + q * (int)src.wstep, 0, 0);
}
constexpr int PF_LOADS = 12;  // direct-to-LDS loads per wave and stage

// Loads 3 P .. 3 P + 2 of a stage (the 4 row pieces, then the 8 W pieces),
// so a wave can spread the next stage's loads over its MFMA steps instead of
// waiting to issue all of them before it multiplies.
template <int P>
__device__ __forceinline__ void pf_stage_part(uint8_t* slot, const PfSrc& src, int stage, int w) {
  const int soff = src.kb + stage * PK * 2;
#pragma unroll
  for (int i = 3 * P; i < 3 * P + 3; ++i) {
    if (i < 4) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(i >= 2 ? src.rhi : src.rlo,
                                               (lds_void*)(slot + (w + 4 * i) * 1024), 16,
                                               src.roff[i], soff, 0, 0);
    } else {
      const int q = i - 4;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src.rw, (lds_void*)(slot + PSTAGE_X + (w + 4 * q) * 1024),
                                               16, src.woff, soff + q * (int)src.wstep, 0, 0);
    }
  }
}

// MFMA operand of step s (k = 32 h + 8 s .. + 7 of the stage, the same
// permutation of k on both operands) for staged row r
__device__ __forceinline__ uint4 pf_frag(const uint8_t* base, int r, int s, int h) {
  const int pos = (4 * h + s) ^ ((r >> 1) & 7);
  return *reinterpret_cast<const uint4*>(base + r * PROW + 16 * pos);
}

// one stage: 4 MFMA k-steps of 16 over the 4 row groups and this wave's 2
// column blocks. The operands of steps 0 and 1 are read first and each
// later step's operands are read while the step before it multiplies;
// scheduling fences keep the steps in that order (left alone the compiler
// reads two operands at a time and waits for them right away, or chains
// MFMAs on one accumulator).
__device__ __forceinline__ void pf_read(uint4 (&av)[4], uint4 (&bv)[2], const uint8_t* slot, int s,
                                        int m, int h, int w) {
#pragma unroll
  for (int g = 0; g < 4; ++g) av[g] = pf_frag(slot, 32 * g + m, s, h);
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) bv[cb] = pf_frag(slot + PSTAGE_X, 64 * w + 32 * cb + m, s, h);
}
__device__ __forceinline__ void pf_mul(const uint4 (&av)[4], const uint4 (&bv)[2],
                                       f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[g][cb] = mfma32(av[g], bv[cb], acc[g][cb]);
}
// With LD, a quarter of stage ns's loads (into slot nxt) goes out before each
// k-step's MFMAs.
template <bool LD>
__device__ __forceinline__ void pf_mma(const uint8_t* slot, f32x16 (&acc)[4][2], int m, int h,
                                       int w, uint8_t* nxt = nullptr, const PfSrc* src = nullptr,
                                       int ns = 0) {
  uint4 av[4][4], bv[4][2];
  pf_read(av[0], bv[0], slot, 0, m, h, w);
  pf_read(av[1], bv[1], slot, 1, m, h, w);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (LD) pf_stage_part<0>(nxt, *src, ns, w);
  __builtin_amdgcn_sched_barrier(0);
  pf_mul(av[0], bv[0], acc);
  pf_read(av[2], bv[2], slot, 2, m, h, w);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (LD) pf_stage_part<1>(nxt, *src, ns, w);
  __builtin_amdgcn_sched_barrier(0);
  pf_mul(av[1], bv[1], acc);
  pf_read(av[3], bv[3], slot, 3, m, h, w);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (LD) pf_stage_part<2>(nxt, *src, ns, w);
  __builtin_amdgcn_sched_barrier(0);
  pf_mul(av[2], bv[2], acc);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (LD) pf_stage_part<3>(nxt, *src, ns, w);
  __builtin_amdgcn_sched_barrier(0);
  pf_mul(av[3], bv[3], acc);
}

// Pipeline step T (3-slot ring): wait until stage T has landed (the loads of
// stage T + 1, issued after it, may still be in flight), barrier (every
// wave's share of stage T is visible and every wave is done with stage
// T - 1), refill the slot stage T - 1 used with stage T + 2, multiply stage T.
template <int NST, int T>
__device__ __forceinline__ void pf_steps(const PfSrc& src, uint8_t* s0, uint8_t* s1, uint8_t* s2,
                                         f32x16 (&acc)[4][2], int m, int h, int w) {
  if constexpr (T < NST) {
    constexpr int TN = T + 2;
    uint8_t* cur = T % 3 == 0 ? s0 : (T % 3 == 1 ? s1 : s2);
    uint8_t* nxt = TN % 3 == 0 ? s0 : (TN % 3 == 1 ? s1 : s2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(T + 1 < NST ? PF_LOADS : 0));
    wg_barrier();
    if constexpr (TN < NST)
      pf_mma<true>(cur, acc, m, h, w, nxt, &src, TN);
    else
      pf_mma<false>(cur, acc, m, h, w);
    pf_steps<NST, T + 1>(src, s0, s1, s2, acc, m, h, w);
  }
}

// Consumer side of the producer-wave K loop: step T waits at the work-group
// barrier (the producer wave has waited for stage T's loads before it, and
// every consumer is done with stage T - 1) and multiplies stage T; the
// consumers issue no loads, so a full load queue never holds up an MFMA.
template <int NST, int T>
__device__ __forceinline__ void pf_csteps(uint8_t* s0, uint8_t* s1, uint8_t* s2,
                                          f32x16 (&acc)[4][2], int m, int h, int w) {
  if constexpr (T < NST) {
    uint8_t* cur = T % 3 == 0 ? s0 : (T % 3 == 1 ? s1 : s2);
    wg_barrier();
    pf_mma<false>(cur, acc, m, h, w);
    pf_csteps<NST, T + 1>(s0, s1, s2, acc, m, h, w);
  }
}
// Producer wave: issues every direct-to-LDS load of the tile (the four
// consumer waves' shares, `src[v]` for consumer v), two stages ahead; before
// the barrier of step T it waits for stage T (stage T + 1 may be in flight),
// after it refills the slot stage T - 1 used with stage T + 2.
constexpr int PF_STAGE_LOADS = 4 * PF_LOADS;  // loads the producer issues per stage
__device__ __forceinline__ void pf_produce(const PfSrc (&src)[4], uint8_t* s0, uint8_t* s1,
                                           uint8_t* s2, int nst) {
  issue_fence();
#pragma unroll
  for (int v = 0; v < 4; ++v) pf_stage(s0, src[v], 0, v);
  if (nst > 1) {
#pragma unroll
    for (int v = 0; v < 4; ++v) pf_stage(s1, src[v], 1, v);
  }
  issue_fence();
  for (int t = 0; t < nst; ++t) {
    if (t + 1 < nst)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(PF_STAGE_LOADS));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    wg_barrier();
    if (t + 2 < nst) {
      const int tn = t + 2;
      uint8_t* nxt = tn % 3 == 0 ? s0 : (tn % 3 == 1 ? s1 : s2);
#pragma unroll
      for (int v = 0; v < 4; ++v) pf_stage(nxt, src[v], tn, v);
    }
    issue_fence();
  }
}

// Consumer side for a stage count known only at run time: the same steps,
// three per round so every slot stays a distinct LDS object
__device__ __forceinline__ void pf_cloop(int nst, uint8_t* s0, uint8_t* s1, uint8_t* s2,
                                         f32x16 (&acc)[4][2], int m, int h, int w) {
  for (int t = 0; t < nst; t += 3) {
    wg_barrier();
    pf_mma<false>(s0, acc, m, h, w);
    if (t + 1 < nst) {
      wg_barrier();
      pf_mma<false>(s1, acc, m, h, w);
    }
    if (t + 2 < nst) {
      wg_barrier();
      pf_mma<false>(s2, acc, m, h, w);
    }
  }
}

// the K loop over NST stages: the first two stages, then the pipeline steps
template <int NST>
__device__ __forceinline__ void pf_kloop(const PfSrc& src, uint8_t* s0, uint8_t* s1, uint8_t* s2,
                                         f32x16 (&acc)[4][2], int m, int h, int w) {
  issue_fence();
  pf_stage(s0, src, 0, w);
  if (NST > 1) pf_stage(s1, src, 1, w);
  issue_fence();
  pf_steps<NST, 0>(src, s0, s1, s2, acc, m, h, w);
}

// 8 bf16 values scaled by e and rounded back to bf16
__device__ __forceinline__ uint4 scale_bf8(uint4 v, float e) {
  uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = bf2f((uint16_t)(q[i] & 0xFFFFu)) * e, hi = bf2f((uint16_t)(q[i] >> 16)) * e;
    q[i] = (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
  }
  return make_uint4(q[0], q[1], q[2], q[3]);
}

// NST: stages of the whole K dimension (a K part of a split tile covers
// NST / P of them); 0: the count a.nst, known at run time
// Five waves: waves 0..3 multiply (and run the epilogue), wave 4 issues the
// K loop's loads and leaves after the loop.
template <int NST>
__global__ void __launch_bounds__(320, 1)
k_prefill_main(PfArgs a) {
  // ring slots as separate LDS objects, so the compiler can tell the slot
  // being read from the ones the direct loads fill
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[PSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[PSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t slot2[PSTAGE];
  __shared__ int32_t tokl[128];
  __shared__ int32_t last_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31, h = lane >> 5;
  const int4 item = a.items[blockIdx.x];
  const int c = item.x, ci = item.y, kp = item.z, xslot = item.w;
  const int64_t d_in = a.d_in, d_out = a.d_out;
  const int64_t col0 = (int64_t)c * 256 + 64 * w + m;  // column block cb: col0 + 32 cb
  const PfChunk ch = a.chunks[ci];
  const GLOBAL int32_t* cr = (const GLOBAL int32_t*)(a.crow + (size_t)ci * 128);
  const int nst_all = NST > 0 ? NST : a.nst;

  // (0) the producer wave: sources of every consumer's pieces, then the loads
  if (w == 4) {
    PfSrc srcv[4];
    const bool rot = (__builtin_amdgcn_readfirstlane(ch.flags) & PF_ROT) != 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int piece = (lane & 7) ^ ((4 * v + (lane >> 4)) & 7);
      srcv[v].rlo = make_rsrc(a.x, a.x_bytes);
      srcv[v].rhi = rot ? make_rsrc(a.dx + (size_t)((c >= a.ptile[0]) + (c >= a.ptile[1]) + (c >= a.ptile[2])) *
                                                a.n_rot * d_in,
                                     a.dx_bytes)
                        : srcv[v].rlo;
      srcv[v].rw = make_rsrc(a.W + (size_t)c * 256 * d_in, (uint32_t)(256 * d_in * 2));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int32_t r = cr[8 * v + 32 * q + (lane >> 3)];
        srcv[v].roff[q] = (uint32_t)(((int64_t)(r >= 0 ? r : -r - 1) * d_in + 8 * piece) * 2);
      }
      srcv[v].woff = (uint32_t)(((int64_t)(8 * v + (lane >> 3)) * d_in + 8 * piece) * 2);
      srcv[v].wstep = (uint32_t)(32 * d_in * 2);
      srcv[v].kb = kp < 0 ? 0 : kp * (nst_all / a.P) * PK * 2;
    }
    pf_produce(srcv, slot0, slot1, slot2, kp < 0 ? nst_all : nst_all / a.P);
    return;
  }

  // (1) this lane's token-table entry
  const int32_t tokv = cr[tid & 127];
  // (2) factor vectors of this lane's columns (used after the K loop)
  float sv[2], ev[2], bv[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    sv[cb] = ldg(ch.s + col0 + 32 * cb);
    ev[cb] = ldg(ch.e + col0 + 32 * cb);
    bv[cb] = ldg(ch.b + col0 + 32 * cb);
  }
  // (4) K loop: the whole K, or one of P parts
  f32x16 acc[4][2];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[g][cb] = f32x16{};
  if constexpr (NST > 0) {
    if (kp < 0)
      pf_csteps<NST, 0>(slot0, slot1, slot2, acc, m, h, w);
    else if (a.P == 4)
      pf_csteps<NST / 4, 0>(slot0, slot1, slot2, acc, m, h, w);
    else
      pf_csteps<NST / 2, 0>(slot0, slot1, slot2, acc, m, h, w);
  } else {
    pf_cloop(kp < 0 ? nst_all : nst_all / a.P, slot0, slot1, slot2, acc, m, h, w);
  }
  lds_barrier();  // every wave is done with the ring

  // (4b) the P parts of a split tile meet: each stores its partial tile with
  //      system-coherent stores (parts may run on different XCDs), waits for
  //      them and counts its arrival; the last to arrive adds the parts in
  //      part order (so the sum does not depend on arrival order) and goes on
  //      with the epilogue
  if (kp >= 0) {
    const rsrc_t pr = make_rsrc(a.part, a.part_bytes);
    constexpr uint32_t TILE = 32u * 256u * 16u;
    const uint32_t base = (uint32_t)xslot * (uint32_t)a.P * TILE + (uint32_t)tid * 16u;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          st_sys4(pr, base + (uint32_t)kp * TILE + (uint32_t)((g * 2 + cb) * 4 + j) * 4096u,
                  f32x4{acc[g][cb][4 * j], acc[g][cb][4 * j + 1], acc[g][cb][4 * j + 2],
                        acc[g][cb][4 * j + 3]});
    wait_vm_all();
    lds_barrier();
    if (tid == 0) {
      const int old = arrive(a.cnt + xslot);
      last_flag = old == a.P - 1;
      if (old == a.P - 1) reset_counter(a.cnt + xslot);
    }
    lds_barrier();
    if (!last_flag) return;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 other[2][4][3];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int qq = 0; qq < 3; ++qq) {
            const int q = qq < kp ? qq : qq + 1;  // the other parts, in order
            other[cb][j][qq] = qq < a.P - 1
                                   ? ld_sys4(pr, base + (uint32_t)q * TILE + (uint32_t)((g * 2 + cb) * 4 + j) * 4096u)
                                   : f32x4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 own{acc[g][cb][4 * j], acc[g][cb][4 * j + 1], acc[g][cb][4 * j + 2],
                          acc[g][cb][4 * j + 3]};
          f32x4 t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // part q: this work-group's own, or other[q] / other[q - 1]
            const f32x4 lo = other[cb][j][q < 3 ? q : 2], hi = other[cb][j][q > 0 ? q - 1 : 0];
            if (q < a.P) t += q == kp ? own : (q < kp ? lo : hi);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[g][cb][4 * j + e] = t[e];
        }
    }
  }

  // (5) epilogue
  if (tid < 128) tokl[tid] = tokv;
  const int32_t flags = ch.flags;
  const bool rot = (flags & PF_ROT) != 0;
  if (rot) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      acc[0][cb] += acc[2][cb];
      acc[1][cb] += acc[3][cb];
    }
  }
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[g][cb] *= sv[cb];

  // expand pieces of 64 ranks: the own term's, then the VeRA term's
  const int rank = ch.rank;
  const int n_own = (flags & PF_OWN) ? (rank + 63) / 64 : 0;
  const int n_ver = (flags & PF_VERA) ? a.r_v / 64 : 0;
  const int ntok = rot ? 64 : 128;  // token rows of the tile
  const rsrc_t ar = make_rsrc(a.tbf, a.acc_bytes);
  for (int pc = 0; pc < n_own + n_ver; ++pc) {
    const bool own = pc < n_own;
    const int kp0 = own ? 64 * pc : 64 * (pc - n_own);
    const int len = own ? rank : a.r_v;  // ranks of the term (B row length)
    const int acol = own ? 0 : a.RT;
    uint8_t* slot = pc % 3 == 0 ? slot0 : (pc % 3 == 1 ? slot1 : slot2);
    // B operand: this lane's columns, ranks kp0 + 32 h + 8 s .. + 7
    const uint16_t* bbase = own ? ch.Bp : a.B_sh;
    uint4 bf[2][4];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int k = kp0 + 32 * h + 8 * s;
        bf[cb][s] = k < len ? ldg16(bbase + (size_t)(col0 + 32 * cb) * len + k) : make_uint4(0, 0, 0, 0);
      }
    // A operand: thread -> row tid / 2, ranks 32 (tid % 2) .. + 31 of the
    // piece (bf16 sums) into the staged layout
    {
      const int r = tid >> 1, hh = tid & 1;
      const bool rowok = r < ntok && r < ch.nx;
      const uint32_t base = (uint32_t)((((int64_t)ch.x0 + r) * a.AW + acol + kp0 + 32 * hh) * 2);
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const bool ok = rowok && kp0 + 32 * hh + 8 * pp < len;
        const u32x4 v = ok ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ar, base + 16 * pp, 0, 0))
                           : u32x4{0u, 0u, 0u, 0u};
        const int pos = (4 * hh + pp) ^ ((r >> 1) & 7);
        *reinterpret_cast<u32x4*>(slot + r * PROW + 16 * pos) = v;
      }
    }
    if (!own) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int s = 0; s < 4; ++s) bf[cb][s] = scale_bf8(bf[cb][s], ev[cb]);
    }
    lds_barrier();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (kp0 + 8 * s < len) {
        uint4 av[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) av[g] = pf_frag(slot, 32 * g + m, s, h);
#pragma unroll
        for (int g = 0; g < 4; ++g)
          if (32 * g < ntok)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) acc[g][cb] = mfma32(av[g], bf[cb][s], acc[g][cb]);
      }
    }
  }
  lds_barrier();  // token table

  // (6) + b, store the token rows: element i of group g is row
  //     32 g + 8 (i / 4) + 4 h + i % 4, column col0 + 32 cb
  const int nst_rows = min(ntok, ch.nx);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    if (32 * g < nst_rows) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 32 * g + 8 * (i >> 2) + 4 * h + (i & 3);
        if (r < nst_rows) {
          float* yr = a.y + (size_t)tokl[r] * d_out + col0;
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) *(GLOBAL float*)(yr + 32 * cb) = acc[g][cb][i] + bv[cb];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// prologue: shrinks and rotation, one item per work-group of 4 waves
// ---------------------------------------------------------------------------

struct PpArgs {
  const uint16_t* x;            // [n][d_in]
  const int32_t* perm;          // sorted position -> token
  const PfProItem* items;
  const DecVeraRow* vrows;      // [64 nvb]
  const uint16_t* A_sh;         // [r_v][d_in]
  uint16_t* dx;                 // [np][n_rot][d_in] Delta rows by sorted position (a rotation
                                // item writes block pad / n_rot)
  float* tpart;                 // [shrink tiles][KP][4 waves][16][64] fp32 partial tiles
  uint16_t* tbf;                // [n][AW] finished sums in bf16
  int32_t* tcnt;                // [shrink tiles] arrival counters
  uint32_t tpart_bytes, tbf_bytes;
  int32_t KP;                   // K parts of a shrink tile
  uint32_t x_bytes, ash_bytes;
  int32_t d_in, AW, RT, r_v;
};

// Delta = x (R - I) for up to 32 rows and 256 columns (64 per wave). With
// blocks of a multiple of 32, each 32-column MFMA block lies in one diagonal
// block and takes blk / 16 k-steps: A = the rows' x over that block, B = the
// block's (R - I)^T rows (stored transposed, so a column's k values are
// contiguous). Operands of up to 4 k-steps are loaded before they are used.
__device__ void pp_rotate(const PpArgs& a, const PfProItem& it, int w, int m, int h) {
  const int64_t d_in = a.d_in;
  const int nr = it.n, blk = it.blk, nks = blk / 16;
  const int tok = ldg(a.perm + it.p0 + min(m, nr - 1));
  const uint16_t* xrow = a.x + (size_t)tok * d_in;
  const uint16_t* xk[2];
  const uint16_t* pk[2];
  int64_t col[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int cblk = it.k + 64 * w + 32 * cb;  // first column of this MFMA block
    const int kb = cblk / blk;
    col[cb] = cblk + m;
    pk[cb] = it.ptr + ((size_t)kb * blk + (col[cb] - (int64_t)kb * blk)) * blk + 8 * h;
    xk[cb] = xrow + (size_t)kb * blk + 8 * h;
  }
  f32x16 acc[2] = {f32x16{}, f32x16{}};
  for (int s0 = 0; s0 < nks; s0 += 4) {
    uint4 xv[2][4], pv[2][4];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (s0 + j < nks) {
          xv[cb][j] = ldg16(xk[cb] + 16 * (s0 + j));
          pv[cb][j] = ldg16(pk[cb] + 16 * (s0 + j));
        }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (s0 + j < nks) acc[cb] = mfma32(xv[cb][j], pv[cb][j], acc[cb]);
  }
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 8 * (i >> 2) + 4 * h + (i & 3);
      if (row < nr) a.dx[(size_t)(it.pad + it.p0 + row) * d_in + col[cb]] = f2bf(acc[cb][i]);
    }
}

// the same for other block sizes: one column per thread, fp32 accumulate
__device__ void pp_rotate_scalar(const PpArgs& a, const PfProItem& it, int tid) {
  const int64_t d_in = a.d_in;
  const int blk = it.blk;
  const int64_t col = it.k + tid;
  const int64_t kb = col / blk, jj = col - kb * blk;
  const uint16_t* prow = it.ptr + ((size_t)kb * blk + jj) * blk;
  for (int r = 0; r < it.n; ++r) {
    const uint16_t* xr = a.x + (size_t)ldg(a.perm + it.p0 + r) * d_in + kb * blk;
    float acc = 0.f;
    for (int i = 0; i < blk; ++i) acc += bf2f(ldg(xr + i)) * bf2f(ldg(prow + i));
    a.dx[(size_t)(it.pad + it.p0 + r) * d_in + col] = f2bf(acc);
  }
}

// Shrink tile: 64 rows x 64 ranks over one K part of 1024, in 4 slices of
// 256. Each slice's rows (gathered by token) and A rows land in LDS by direct
// buffer->LDS loads (one instruction: 2 rows of 512 bytes; 16-byte piece p of
// row r stored at position p ^ (r & 31), so the 32 rows an MFMA operand read
// touches fall in distinct banks), two slices in flight in two buffers; wave
// w multiplies row block w & 1 by rank block w >> 1. Each K part stores
// its fp32 partial tile; the last part to arrive adds them in part order.
constexpr int PP_ROW = 512;                  // bytes of a staged row (256 k)
constexpr int PP_BUF = 2 * 64 * PP_ROW;      // 64 x rows, then 64 A rows
constexpr int PP_LOADS = 16;                 // direct loads per wave and slice
__device__ __forceinline__ uint4 pp_frag(const uint8_t* base, int r, int piece) {
  return *reinterpret_cast<const uint4*>(base + r * PP_ROW + 16 * (piece ^ (r & 31)));
}
__device__ __forceinline__ void pp_stage(uint8_t* buf, rsrc_t rx, rsrc_t ra, const uint32_t (&xoff)[8],
                                         const uint32_t (&aoff)[8], int soff, int w) {
#pragma unroll
  for (int q = 0; q < 8; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(buf + (w + 4 * q) * 1024), 16, xoff[q], soff, 0, 0);
#pragma unroll
  for (int q = 0; q < 8; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(buf + 64 * PP_ROW + (w + 4 * q) * 1024), 16,
                                             aoff[q], soff, 0, 0);
}
__device__ __forceinline__ void pp_mul(const uint8_t* buf, f32x16& acc, int rb, int cb, int m, int h) {
#pragma unroll
  for (int s = 0; s < 16; ++s)
    acc = mfma32(pp_frag(buf, 32 * rb + m, 2 * s + h), pp_frag(buf + 64 * PP_ROW, 32 * cb + m, 2 * s + h), acc);
}

__global__ void __launch_bounds__(256) k_prefill_prologue(PpArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t buf0[PP_BUF];
  __shared__ __attribute__((aligned(1024))) uint8_t buf1[PP_BUF];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31, h = lane >> 5;
  const PfProItem it = a.items[blockIdx.x];
  const int64_t d_in = a.d_in;
  if (it.type == PP_ROT) {
    if (it.blk % 32 == 0)
      pp_rotate(a, it, w, m, h);
    else
      pp_rotate_scalar(a, it, tid);
    return;
  }
  const bool vera = it.type == PP_VSHRINK;
  const int k0 = it.k & 0xFFFF, nk = it.k >> 16;
  const int kbase = it.blk * 1024;  // this item's K part
  // (1) sources: this lane's row in each of its 8 x and 8 A instructions
  //     (instruction j: rows 2 j, 2 j + 1)
  const int pos = lane & 31;
  uint32_t xoff[8], aoff[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int r = 2 * (w + 4 * q) + (lane >> 5);
    const int tok = vera ? a.vrows[64 * it.p0 + r].tok : ldg(a.perm + it.p0 + min(r, it.n - 1));
    xoff[q] = (uint32_t)(((int64_t)tok * d_in + 8 * (pos ^ (r & 31))) * 2);
    aoff[q] = (uint32_t)(((int64_t)(k0 + min(r, nk - 1)) * d_in + 8 * (pos ^ (r & 31))) * 2);
  }
  const rsrc_t rx = make_rsrc(a.x, a.x_bytes);
  const rsrc_t ra = vera ? make_rsrc(a.A_sh, a.ash_bytes)
                         : make_rsrc(it.ptr, (uint32_t)((int64_t)(k0 + nk) * d_in * 2));
  // slices of 256 in this part (the last part of a d_in that is not a
  // multiple of 1024 has fewer than 4)
  const int ns = min(4, (int)((d_in - kbase) / 256));
  issue_fence();
  pp_stage(buf0, rx, ra, xoff, aoff, kbase * 2, w);
  if (ns > 1) pp_stage(buf1, rx, ra, xoff, aoff, (kbase + 256) * 2, w);
  issue_fence();
  // VeRA: rows and d of this lane's outputs, fetched while the loads land
  const int rb = w & 1, cb = w >> 1;
  int32_t prow[16];
  float dsc[16];
  if (vera) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const DecVeraRow o = a.vrows[64 * it.p0 + 32 * rb + 8 * (i >> 2) + 4 * h + (i & 3)];
      prow[i] = o.p;
      dsc[i] = ldg(o.vd + k0 + 32 * cb + m);
    }
  }
  // (2) up to four slices, two buffers; each wait lets only the slice
  //     staged after the one it waits for stay in flight
  f32x16 acc = {};
  if (ns > 1)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(PP_LOADS));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  wg_barrier();
  pp_mul(buf0, acc, rb, cb, m, h);
  if (ns > 1) {
    wg_barrier();
    if (ns > 2) pp_stage(buf0, rx, ra, xoff, aoff, (kbase + 512) * 2, w);
    if (ns > 2)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(PP_LOADS));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    wg_barrier();
    pp_mul(buf1, acc, rb, cb, m, h);
    if (ns > 2) {
      wg_barrier();
      if (ns > 3) pp_stage(buf1, rx, ra, xoff, aoff, (kbase + 768) * 2, w);
      if (ns > 3)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(PP_LOADS));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      wg_barrier();
      pp_mul(buf0, acc, rb, cb, m, h);
      if (ns > 3) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        wg_barrier();
        pp_mul(buf1, acc, rb, cb, m, h);
      }
    }
  }
  const int j = 32 * cb + m;  // rank of this lane's outputs within the tile
  // (3) store this K part's partial tile (VeRA: scaled by d, which is per
  //     rank and so commutes with the K sum): element i of wave w, lane l
  //     at [tile][part][w][i][l], so every store instruction writes 256
  //     contiguous bytes; written through to memory for the last part
  const rsrc_t pr = make_rsrc(a.tpart, a.tpart_bytes);
  const uint32_t tile_off = (uint32_t)(it.pad * a.KP) * 16384u;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    st_sys1(pr, tile_off + (uint32_t)it.blk * 16384u + (uint32_t)((w * 16 + i) * 64 + lane) * 4u,
            vera ? acc[i] * dsc[i] : acc[i]);
  // (4) the last K part of the tile to arrive adds the parts in part order,
  //     then writes the tile's sums as bf16
  __shared__ int32_t last_part;
  wait_vm_all();
  lds_barrier();
  if (tid == 0) {
    const int old = arrive(a.tcnt + it.pad);
    last_part = old == a.KP - 1;
    if (old == a.KP - 1) reset_counter(a.tcnt + it.pad);
  }
  lds_barrier();
  if (!last_part) return;
  {
    float sum[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) sum[i] = 0.f;
    for (int p = 0; p < a.KP; ++p) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        v[i] = ld_sys1(pr, tile_off + (uint32_t)p * 16384u + (uint32_t)((w * 16 + i) * 64 + lane) * 4u);
#pragma unroll
      for (int i = 0; i < 16; ++i) sum[i] += v[i];
    }
    // transpose through LDS (buf0 is free: every wave is past its last
    // multiply): T[row][rank], row 32 rb + 8 (i / 4) + 4 h + i % 4, rank j
    float* T = reinterpret_cast<float*>(buf0);
#pragma unroll
    for (int i = 0; i < 16; ++i) T[(32 * rb + 8 * (i >> 2) + 4 * h + (i & 3)) * 64 + j] = sum[i];
  }
  lds_barrier();
  {
    // thread -> tile row tid / 4, ranks 16 (tid % 4) .. + 15
    const int r = tid >> 2, c16 = 16 * (tid & 3);
    int32_t row;
    if (vera)
      row = a.vrows[64 * it.p0 + r].p;
    else
      row = r < it.n ? it.p0 + r : -1;
    if (row >= 0 && c16 < nk) {
      const float* T = reinterpret_cast<const float*>(buf0) + r * 64 + c16;
      uint32_t wv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) wv[e] = pack_bf2(__float_as_uint(T[2 * e]), __float_as_uint(T[2 * e + 1]));
      uint16_t* dst = a.tbf + (size_t)row * a.AW + (vera ? a.RT : 0) + k0 + c16;
      *(GLOBAL u32x4*)dst = u32x4{wv[0], wv[1], wv[2], wv[3]};
      *(GLOBAL u32x4*)(dst + 8) = u32x4{wv[4], wv[5], wv[6], wv[7]};
    }
  }
}

}  // namespace

scute_status launch_prefill(scute_layer* L, const scute_batch* B, const void* x, const void* W,
                            float* y, hipStream_t st, int32_t* launches) {
  const PrefillPlan& P = B->pp;
  // the shrink sums of this forward and the buffer cleared for the next
  int nl = 0;
  if (P.n_pro > 0) {
    PpArgs pa{};
    pa.x = (const uint16_t*)x;
    pa.perm = B->d_perm;
    pa.items = P.pro_items;
    pa.vrows = P.vrows;
    pa.A_sh = (const uint16_t*)L->A_sh;
    pa.dx = (uint16_t*)B->delta;
    pa.tpart = P.tpart;
    pa.tpart_bytes = P.tpart_bytes;
    pa.tbf = P.tbf;
    pa.tcnt = P.tcnt;
    pa.tbf_bytes = P.tbf_bytes;
    pa.KP = (int32_t)((L->d_in + 1023) / 1024);
    pa.x_bytes = (uint32_t)((size_t)B->n * L->d_in * 2);
    pa.ash_bytes = (uint32_t)((size_t)L->r_v * L->d_in * 2);
    pa.d_in = (int32_t)L->d_in;
    pa.AW = P.AW;
    pa.RT = P.RT;
    pa.r_v = L->r_v;
    ProfScope ps(L, st, "prefill_prologue", true);
    hipExtLaunchKernelGGL(k_prefill_prologue, dim3(P.n_pro), dim3(256), 0, st, ps.ev_start(), ps.ev_stop(),
                          0, pa);
    ++nl;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "launch k_prefill_prologue");
  }
  PfArgs ma{};
  ma.x = (const uint16_t*)x;
  ma.dx = (const uint16_t*)B->delta;
  ma.W = (const uint16_t*)W;
  ma.chunks = P.chunks;
  ma.crow = P.crow;
  ma.B_sh = (const uint16_t*)L->B_sh;
  ma.tbf = P.tbf;
  ma.y = y;
  ma.acc_bytes = P.tbf_bytes;
  ma.x_bytes = (uint32_t)((size_t)B->n * L->d_in * 2);
  ma.dx_bytes = (uint32_t)((size_t)B->n_rot * L->d_in * 2);
  ma.n_rot = B->n_rot;
  for (int32_t i = 0; i + 1 < MAX_PROJ; ++i)
    ma.ptile[i] = (int32_t)((B->rproj && i + 1 < L->n_proj ? L->proj_end[i] : L->d_out) / 256);
  ma.d_in = (int32_t)L->d_in;
  ma.d_out = (int32_t)L->d_out;
  ma.RT = P.RT;
  ma.AW = P.AW;
  ma.r_v = L->r_v;
  ma.items = P.items;
  ma.part = P.part;
  ma.cnt = P.cnt;
  ma.part_bytes = P.part_bytes;
  ma.P = P.P;
  ma.nst = (int32_t)(L->d_in / 64);
  // every table the kernel dereferences must be there
  if (!ma.chunks || !ma.crow || !ma.items || !ma.x || !ma.W || !ma.y ||
      (P.P > 1 && (!ma.part || !ma.cnt)) || (B->n_rot > 0 && !ma.dx) ||
      (B->n_vera > 0 && !ma.B_sh) || (P.AW > 0 && !ma.tbf))
    return fail(SCUTE_E_STATE, "prefill path: plan tables missing");
  {
    ProfScope ps(L, st, "prefill_main", true);
    if (ma.nst == 64)  // d_in 4096: the K loop unrolled at compile time
      hipExtLaunchKernelGGL(k_prefill_main<64>, dim3(P.n_items), dim3(320), 0, st, ps.ev_start(),
                            ps.ev_stop(), 0, ma);
    else
      hipExtLaunchKernelGGL(k_prefill_main<0>, dim3(P.n_items), dim3(320), 0, st, ps.ev_start(),
                            ps.ev_stop(), 0, ma);
    ++nl;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch k_prefill_main");
  if (launches) *launches = nl;
  return SCUTE_OK;
}

}  // namespace scute
