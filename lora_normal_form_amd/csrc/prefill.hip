// MFMA prefill path (bf16 activations, fp32 accumulate, long adapter
// segments; d_in = 4096).
//
// Two kernels per forward.
//
// k_prefill_prologue works on items of one work-group (16 waves) each:
//   shrink       t = x A' for 32 rows of a segment x 32 own ranks, and
//   VeRA shrink  u = (x A_sh) (.) d for 32 VeRA rows x 32 ranks, both over the
//                whole K on 32x32x16 bf16 MFMA (16 waves, wave w sums K slice
//                w; the slices meet in LDS in a fixed order, so the sums are
//                the same on every forward and are stored once, without
//                atomics);
//   rotation     Delta = x (R - I) for 32 rotated rows x 1024 columns; R is
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
//            extra MFMA steps: A = the chunk's shrink sums (fp32 rounded to
//            bf16, staged through the ring in pieces of 64 ranks), B = the
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
  const uint16_t* dx;      // [n_rot][d_in] Delta rows by sorted position
  const uint16_t* W;       // [d_out][d_in]
  const PfChunk* chunks;   // [n_chunks]
  const int32_t* crow;     // [n_chunks][128] row sources: token, or -(Delta row) - 1
  const uint16_t* B_sh;    // [d_out][r_v]
  const float* acc;        // [n][AW] shrink sums: RT own ranks, then r_v VeRA ranks
  float* y;                // [n][d_out]
  const int4* items;        // per work-group: column tile, chunk, K part (-1: all), exchange slot
  float* part;              // [n_split][P][32][256] f32x4 partial tiles
  int32_t* cnt;             // [n_split] arrival counters, kept at zero between forwards
  uint32_t acc_bytes, x_bytes, dx_bytes, part_bytes;
  int32_t d_in, d_out, RT, AW, r_v, P;
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
__device__ __forceinline__ void pf_mma(const uint8_t* slot, f32x16 (&acc)[4][2], int m, int h,
                                       int w) {
  uint4 av[4][4], bv[4][2];
  pf_read(av[0], bv[0], slot, 0, m, h, w);
  pf_read(av[1], bv[1], slot, 1, m, h, w);
  __builtin_amdgcn_sched_barrier(0);
  pf_mul(av[0], bv[0], acc);
  pf_read(av[2], bv[2], slot, 2, m, h, w);
  __builtin_amdgcn_sched_barrier(0);
  pf_mul(av[1], bv[1], acc);
  pf_read(av[3], bv[3], slot, 3, m, h, w);
  __builtin_amdgcn_sched_barrier(0);
  pf_mul(av[2], bv[2], acc);
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
    if constexpr (TN < NST) pf_stage(nxt, src, TN, w);
    pf_mma(cur, acc, m, h, w);
    pf_steps<NST, T + 1>(src, s0, s1, s2, acc, m, h, w);
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
// NST / P of them)
template <int NST>
__global__ void __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
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

  // (1) row sources of this lane's 4 pieces per stage, its token-table entry
  const GLOBAL int32_t* cr = (const GLOBAL int32_t*)(a.crow + (size_t)ci * 128);
  int32_t srow[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) srow[q] = cr[8 * w + 32 * q + (lane >> 3)];
  const int32_t tokv = cr[tid & 127];
  // (2) factor vectors of this lane's columns (used after the K loop)
  float sv[2], ev[2], bv[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    sv[cb] = ldg(ch.s + col0 + 32 * cb);
    ev[cb] = ldg(ch.e + col0 + 32 * cb);
    bv[cb] = ldg(ch.b + col0 + 32 * cb);
  }
  // (3) sources, then the first two stages
  PfSrc src;
  {
    const int piece = (lane & 7) ^ ((4 * w + (lane >> 4)) & 7);
    const bool rot = (__builtin_amdgcn_readfirstlane(ch.flags) & PF_ROT) != 0;
    src.rlo = make_rsrc(a.x, a.x_bytes);
    src.rhi = rot ? make_rsrc(a.dx, a.dx_bytes) : src.rlo;
    src.rw = make_rsrc(a.W + (size_t)c * 256 * d_in, (uint32_t)(256 * d_in * 2));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int32_t v = srow[q];
      src.roff[q] = (uint32_t)(((int64_t)(v >= 0 ? v : -v - 1) * d_in + 8 * piece) * 2);
    }
    src.woff = (uint32_t)(((int64_t)(8 * w + (lane >> 3)) * d_in + 8 * piece) * 2);
    src.wstep = (uint32_t)(32 * d_in * 2);
    src.kb = kp < 0 ? 0 : kp * (NST / a.P) * PK * 2;
  }

  // (4) K loop: the whole K, or one of P parts
  f32x16 acc[4][2];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[g][cb] = f32x16{};
  if (kp < 0)
    pf_kloop<NST>(src, slot0, slot1, slot2, acc, m, h, w);
  else if (a.P == 4)
    pf_kloop<NST / 4>(src, slot0, slot1, slot2, acc, m, h, w);
  else
    pf_kloop<NST / 2>(src, slot0, slot1, slot2, acc, m, h, w);
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
  const rsrc_t ar = make_rsrc(a.acc, a.acc_bytes);
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
    // piece, fp32 sums rounded to bf16 into the staged layout
    {
      const int r = tid >> 1, hh = tid & 1;
      const bool rowok = r < ntok && r < ch.nx;
      const uint32_t base = (uint32_t)((((int64_t)ch.x0 + r) * a.AW + acol + kp0 + 32 * hh) * 4);
      f32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool ok = rowok && kp0 + 32 * hh + 4 * j < len;
        v[j] = ok ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ar, base + 16 * j, 0, 0))
                  : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const f32x4 lo = v[2 * pp], hi = v[2 * pp + 1];
        const uint4 pk = make_uint4(pack_bf2(__float_as_uint(lo.x), __float_as_uint(lo.y)),
                                    pack_bf2(__float_as_uint(lo.z), __float_as_uint(lo.w)),
                                    pack_bf2(__float_as_uint(hi.x), __float_as_uint(hi.y)),
                                    pack_bf2(__float_as_uint(hi.z), __float_as_uint(hi.w)));
        const int pos = (4 * hh + pp) ^ ((r >> 1) & 7);
        *reinterpret_cast<uint4*>(slot + r * PROW + 16 * pos) = pk;
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
  const uint16_t* x;         // [n][d_in]
  const int32_t* perm;       // sorted position -> token
  const PfProItem* items;
  const DecVeraRow* vrows;   // [32 nvb]
  const uint16_t* A_sh;      // [r_v][d_in]
  uint16_t* dx;              // [n_rot][d_in] Delta rows by sorted position
  float* acc;                // [n][AW] shrink sums
  int32_t d_in, AW, RT;
};

// Delta = x (R - I) for up to 32 rows and 1024 columns (64 per wave). With
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
      if (row < nr) a.dx[(size_t)(it.p0 + row) * d_in + col[cb]] = f2bf(acc[cb][i]);
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
    a.dx[(size_t)(it.p0 + r) * d_in + col] = f2bf(acc);
  }
}

// 16 waves per item: a shrink tile's K slices of 256 (one per wave) meet in
// LDS and four waves add them in slice order; a rotation item spreads its
// 1024 columns over the waves.
constexpr int PP_WAVES = 16;
__global__ void __launch_bounds__(64 * PP_WAVES) k_prefill_prologue(PpArgs a) {
  __shared__ f32x4 red[PP_WAVES][4][64];
  const PfProItem it = a.items[blockIdx.x];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31, h = lane >> 5;
  const int64_t d_in = a.d_in;
  if (it.type == PP_ROT) {
    if (it.blk % 32 == 0)
      pp_rotate(a, it, w, m, h);
    else
      pp_rotate_scalar(a, it, tid);
    return;
  }
  // shrink tile of 32 rows x 32 ranks: wave w sums K slice w (d_in = 16 x 256)
  const uint16_t* xr;
  const uint16_t* ar;
  if (it.type == PP_SHRINK) {
    const int nk = it.k >> 16;
    xr = a.x + (size_t)ldg(a.perm + it.p0 + min(m, it.n - 1)) * d_in;
    ar = it.ptr + (size_t)((it.k & 0xFFFF) + min(m, nk - 1)) * d_in;
  } else {
    xr = a.x + (size_t)a.vrows[32 * it.p0 + m].tok * d_in;
    ar = a.A_sh + (size_t)(32 * it.k + m) * d_in;
  }
  const int64_t koff = (int64_t)w * 256 + 32 * h;
  const f32x16 acc = shrink_tile(xr + koff, ar + koff);
#pragma unroll
  for (int c = 0; c < 4; ++c) red[w][c][lane] = f32x4{acc[4 * c], acc[4 * c + 1], acc[4 * c + 2], acc[4 * c + 3]};
  lds_barrier();
  if (w >= 4) return;
  // wave c adds elements 4 c .. 4 c + 3 of every lane over the slices, in
  // slice order, so every forward gives the same sums
  const int c = w;
  f32x4 sum = red[0][c][lane];
#pragma unroll
  for (int v = 1; v < PP_WAVES; ++v) sum += red[v][c][lane];
  // element 4 c + e: row 8 c + 4 h + e of the tile, rank column m
  if (it.type == PP_SHRINK) {
    const int k0 = it.k & 0xFFFF, nk = it.k >> 16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 8 * c + 4 * h + e;
      if (row < it.n && m < nk) a.acc[(size_t)(it.p0 + row) * a.AW + k0 + m] = sum[e];
    }
  } else {
    // VeRA row 32 p0 + row, rank 32 k + m; d scales each rank (it commutes
    // with the K sum)
    const int j = 32 * it.k + m;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const DecVeraRow o = a.vrows[32 * it.p0 + 8 * c + 4 * h + e];
      if (o.p >= 0) a.acc[(size_t)o.p * a.AW + a.RT + j] = sum[e] * ldg(o.vd + j);
    }
  }
}

}  // namespace

scute_status launch_prefill(scute_layer* L, const scute_batch* B, const void* x, const void* W,
                            float* y, hipStream_t st, int32_t* launches) {
  const PrefillPlan& P = B->pp;
  int nl = 0;
  if (P.n_pro > 0) {
    PpArgs pa{};
    pa.x = (const uint16_t*)x;
    pa.perm = B->d_perm;
    pa.items = P.pro_items;
    pa.vrows = P.vrows;
    pa.A_sh = (const uint16_t*)L->A_sh;
    pa.dx = (uint16_t*)B->delta;
    pa.acc = P.acc32;
    pa.d_in = (int32_t)L->d_in;
    pa.AW = P.AW;
    pa.RT = P.RT;
    ProfScope ps(L, st, "prefill_prologue");
    hipLaunchKernelGGL(k_prefill_prologue, dim3(P.n_pro), dim3(64 * PP_WAVES), 0, st, pa);
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
  ma.acc = P.acc32;
  ma.y = y;
  ma.acc_bytes = P.acc_bytes;
  ma.x_bytes = (uint32_t)((size_t)B->n * L->d_in * 2);
  ma.dx_bytes = (uint32_t)((size_t)B->n_rot * L->d_in * 2);
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
  {
    ProfScope ps(L, st, "prefill_main");
    hipLaunchKernelGGL(k_prefill_main<64>, dim3(P.n_items), dim3(256), 0, st, ma);
    ++nl;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch k_prefill_main");
  if (launches) *launches = nl;
  return SCUTE_OK;
}

}  // namespace scute
