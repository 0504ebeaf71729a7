// MFMA prefill path (bf16 activations, fp32 accumulate, long adapter
// segments; d_in = 4096).
//
// Two kernels per forward: the decode path's prologue kernel (rotation
// Delta = x (R - I) into the Delta rows, own-term and VeRA shrinks into the
// fp32 shrink sums; see decode.hip), then k_prefill_main.
//
// k_prefill_main computes one tile of 128 staged rows by 256 output columns
// per work-group of 4 waves, over the whole K dimension. A chunk (the tile's
// rows) belongs to one adapter segment: up to 128 tokens, or up to 64 tokens
// followed by their 64 Delta rows when the adapter rotates. Wave w owns
// columns 64 w .. 64 w + 63 of the tile (two 32-column MFMA blocks) for all
// 128 rows, so its accumulators are 4 row groups x 2 column blocks of
// 32x32x16 bf16 MFMA tiles.
//   K loop   the rows stream through an LDS ring of 4 stages of 64 k filled
//            by direct global->LDS loads that gather each row from x (or from
//            the Delta rows) by its token; W streams straight into registers
//            three stages ahead. The loop is unrolled at compile time with
//            every wait counting exactly the loads issued after the stage it
//            waits for.
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
  uint32_t acc_bytes;
  int32_t d_in, d_out, RT, AW, r_v;
};

constexpr int PK = 64;              // k per stage
constexpr int PROW = 2 * PK;        // bytes per staged row
constexpr int PSTAGE = 128 * PROW;  // bytes per stage

// Staged row r of a stage: 8 pieces of 16 bytes, piece p stored at position
// p ^ ((r >> 1) & 7) to spread LDS banks. One direct-to-LDS instruction
// fills 8 rows (lane i -> row i / 8, position i % 8); wave w issues
// instructions w, w + 4, w + 8, w + 12 of a stage.
__device__ __forceinline__ void pf_stage_rows(uint8_t* slot, const uint16_t* const (&src)[4],
                                              int64_t koff, int w) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    __builtin_amdgcn_global_load_lds((const void*)(src[q] + koff),
                                     (lds_void*)(slot + (w + 4 * q) * 1024), 16, 0, 0);
}

// W of one stage for this lane's two columns: 64 contiguous bytes of each W
// row (k = 32 h .. 32 h + 31 of the stage), through a buffer resource with a
// fixed per-lane offset and the stage's scalar offset. MFMA step s uses
// elements 8 s .. 8 s + 7 of each half, on both operands.
struct PfW {
  rsrc_t r;
  uint32_t voff[2];
};
__device__ __forceinline__ void pf_load_w(uint4 (&wr)[2][4], const PfW& ws, int64_t koff) {
  const int soff = (int)(koff * 2);
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      wr[cb][s] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(ws.r, ws.voff[cb] + 16 * s, soff, 0));
}

// A operand of MFMA step s for row group g from a staged tile
__device__ __forceinline__ uint4 pf_afrag(const uint8_t* slot, int g, int s, int m, int h) {
  const int r = 32 * g + m;
  const int pos = (4 * h + s) ^ ((r >> 1) & 7);
  return *reinterpret_cast<const uint4*>(slot + r * PROW + 16 * pos);
}

// one stage: 4 MFMA k-steps of 16 over the 4 row groups and 2 column
// blocks; the A operands of step s + 1 are read while step s multiplies
__device__ __forceinline__ void pf_mma(const uint8_t* slot, const uint4 (&wr)[2][4],
                                       f32x16 (&acc)[4][2], int m, int h) {
  uint4 av[2][4];
#pragma unroll
  for (int g = 0; g < 4; ++g) av[0][g] = pf_afrag(slot, g, 0, m, h);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s < 3)
#pragma unroll
      for (int g = 0; g < 4; ++g) av[(s + 1) & 1][g] = pf_afrag(slot, g, s + 1, m, h);
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) acc[g][cb] = mfma32(av[s & 1][g], wr[cb][s], acc[g][cb]);
  }
}

// Outstanding vector-memory operations allowed when step T waits for stage
// T. Issue order: W(0..2), rows(0..2), then step t issues W(t + 3) before
// its wait and rows(t + 3) after it (each only for existing stages); W(T)
// always precedes rows(T), so the wait counts what was issued after rows(T):
// 8 per W stage, 4 per rows stage.
constexpr int pf_allowed(int T, int NST) {
  int cnt = 0;
  for (int u = T + 1; u <= 2; ++u)
    if (u < NST) cnt += 4;
  const int t0 = T <= 2 ? 0 : T - 2;
  for (int t = t0; t <= T; ++t) {
    if (t + 3 < NST) cnt += 8;
    if (t < T && t + 3 < NST) cnt += 4;
  }
  return cnt;
}

template <int NST, int T>
__device__ __forceinline__ void pf_steps(const PfW& ws, const uint16_t* const (&src)[4],
                                         uint8_t* s0, uint8_t* s1, uint8_t* s2, uint8_t* s3,
                                         uint4 (&wb)[4][2][4], f32x16 (&acc)[4][2], int m, int h,
                                         int w) {
  if constexpr (T < NST) {
    constexpr int TN = T + 3;
    uint8_t* cur = T % 4 == 0 ? s0 : (T % 4 == 1 ? s1 : (T % 4 == 2 ? s2 : s3));
    uint8_t* nxt = TN % 4 == 0 ? s0 : (TN % 4 == 1 ? s1 : (TN % 4 == 2 ? s2 : s3));
    if constexpr (TN < NST) pf_load_w(wb[TN % 4], ws, (int64_t)PK * TN);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(pf_allowed(T, NST)));
    wg_barrier();
    if constexpr (TN < NST) pf_stage_rows(nxt, src, (int64_t)PK * TN, w);
    pf_mma(cur, wb[T % 4], acc, m, h);
    pf_steps<NST, T + 1>(ws, src, s0, s1, s2, s3, wb, acc, m, h, w);
  }
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

template <int NST>
__global__ void __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_prefill_main(PfArgs a) {
  // ring slots as separate LDS objects, so the compiler can tell the slot
  // being read from the ones the direct loads fill
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[PSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[PSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t slot2[PSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t slot3[PSTAGE];
  __shared__ int32_t tokl[128];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31, h = lane >> 5;
  // grid (column tile, chunk): linear work-group ids run over the column
  // tiles first, so with a multiple of 8 column tiles each XCD keeps the same
  // W columns for every chunk
  const int c = blockIdx.x, ci = blockIdx.y;
  const int64_t d_in = a.d_in, d_out = a.d_out;
  const int64_t col0 = (int64_t)c * 256 + 64 * w + m;  // column block cb: col0 + 32 cb
  const PfChunk ch = a.chunks[ci];

  // (1) row sources of this lane's 4 pieces per stage, its token-table entry
  const GLOBAL int32_t* cr = (const GLOBAL int32_t*)(a.crow + (size_t)ci * 128);
  int32_t srow[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) srow[q] = cr[8 * w + 32 * q + (lane >> 3)];
  const int32_t tokv = cr[tid & 127];
  // (2) W of the first three stages
  const PfW ws{make_rsrc(a.W, (uint32_t)(d_out * d_in * 2)),
               {(uint32_t)((col0 * d_in + 32 * h) * 2), (uint32_t)(((col0 + 32) * d_in + 32 * h) * 2)}};
  uint4 wb[4][2][4];
#pragma unroll
  for (int t = 0; t < 3; ++t)
    if (t < NST) pf_load_w(wb[t], ws, (int64_t)PK * t);
  // (3) factor vectors of this lane's columns (used after the K loop)
  float sv[2], ev[2], bv[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    sv[cb] = ldg(ch.s + col0 + 32 * cb);
    ev[cb] = ldg(ch.e + col0 + 32 * cb);
    bv[cb] = ldg(ch.b + col0 + 32 * cb);
  }
  issue_fence();
  // (4) rows of the first three stages
  const uint16_t* src[4];
  {
    const int piece = (lane & 7) ^ ((4 * w + (lane >> 4)) & 7);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int32_t v = srow[q];
      const uint16_t* base = v >= 0 ? a.x + (size_t)v * d_in : a.dx + (size_t)(-v - 1) * d_in;
      src[q] = base + 8 * piece;
    }
  }
  pf_stage_rows(slot0, src, 0, w);
  if (NST > 1) pf_stage_rows(slot1, src, PK, w);
  if (NST > 2) pf_stage_rows(slot2, src, 2 * PK, w);
  issue_fence();

  // (5) K loop
  f32x16 acc[4][2];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[g][cb] = f32x16{};
  pf_steps<NST, 0>(ws, src, slot0, slot1, slot2, slot3, wb, acc, m, h, w);

  // (6) epilogue. Slots 0..2 were last read before the final step's
  //     barrier, so the expand may stage into them now.
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
        for (int g = 0; g < 4; ++g) av[g] = pf_afrag(slot, g, s, m, h);
#pragma unroll
        for (int g = 0; g < 4; ++g)
          if (32 * g < ntok)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) acc[g][cb] = mfma32(av[g], bf[cb][s], acc[g][cb]);
      }
    }
  }
  lds_barrier();  // token table

  // (7) + b, store the token rows: element i of group g is row
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

}  // namespace

scute_status launch_prefill(scute_layer* L, const scute_batch* B, const void* x, const void* W,
                            float* y, hipStream_t st, int32_t* launches) {
  const PrefillPlan& P = B->pp;
  // the shrink sums of this forward and the buffer cleared for the next
  float* acc = P.acc32[P.fwd & 1];
  float* acc_next = P.acc32[(P.fwd + 1) & 1];
  ++P.fwd;
  int nl = 0;
  if (P.n_pro > 0) {
    ProArgs pa{};
    pa.x = (const uint16_t*)x;
    pa.perm = B->d_perm;
    pa.items = P.pro_items;
    pa.n_items = P.n_pro;
    pa.vrows = P.vrows;
    pa.A_sh = (const uint16_t*)L->A_sh;
    pa.xs = (uint16_t*)B->delta;  // rotation items write Delta row p at row p
    pa.acc = acc;
    pa.acc_next = acc_next;
    pa.acc_words = P.acc_bytes / 4;
    pa.M_pad = 0;
    pa.AW = P.AW;
    pa.RT = P.RT;
    pa.d_in = (int32_t)L->d_in;
    const int grid = std::max(1, std::min(8192, pa.n_items));
    ProfScope ps(L, st, "decode_prologue");
    launch_prologue(pa, grid, st);
    ++nl;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "launch k_decode_prologue");
  }
  PfArgs ma{};
  ma.x = (const uint16_t*)x;
  ma.dx = (const uint16_t*)B->delta;
  ma.W = (const uint16_t*)W;
  ma.chunks = P.chunks;
  ma.crow = P.crow;
  ma.B_sh = (const uint16_t*)L->B_sh;
  ma.acc = acc;
  ma.y = y;
  ma.acc_bytes = P.acc_bytes;
  ma.d_in = (int32_t)L->d_in;
  ma.d_out = (int32_t)L->d_out;
  ma.RT = P.RT;
  ma.AW = P.AW;
  ma.r_v = L->r_v;
  {
    ProfScope ps(L, st, "prefill_main");
    hipLaunchKernelGGL(k_prefill_main<64>, dim3(P.C, P.n_chunks), dim3(256), 0, st, ma);
    ++nl;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch k_prefill_main");
  if (launches) *launches = nl;
  return SCUTE_OK;
}

}  // namespace scute
