// MFMA decode path (bf16 activations, fp32 accumulate, up to 256 rows).
//
// Two kernels per forward.
//
// k_decode_prologue works on small items, one per wave:
//   gather      copy the batch's x rows into sorted order, so the main
//               kernel stages rows at affine addresses;
//   rotation    delta = x (R - I) for up to 4 rotated rows and 64 columns
//               (R is block-diagonal, so a column needs one block of x),
//               stored after the sorted x rows;
//   own shrink  t = x A' for up to 4 rows x 4 ranks over a K part of 1024;
//   VeRA shrink u = (x A_sh) (.) d for 32 VeRA rows x 32 ranks over a K
//               slice of 256, on four 16x16x32 MFMA tiles.
// Rotation runs before the shared GEMM and the shared VeRA pair is read once
// per step for the whole batch ("Where is the cheapest place to compute the
// remaining slots?", paper-daily.com explainer of "Scute: Exact Batched
// Serving for PEFT Adapters Beyond LoRA"). The K parts of a shrink add into
// an fp32 buffer with float atomics (no waiting on each other); the buffers
// alternate between forwards and each prologue clears the other one.
//
// k_decode_main computes, per work-group of 4 waves, 64 output columns over
// one of S slices of K for all rows of the batch:
//   base     x W and delta W on 32x32x16 bf16 MFMA: x / delta rows staged in
//            LDS by direct global->LDS loads through a ring of 64-k stages,
//            W streamed into registers (through a per-wave LDS block that
//            turns whole-row loads into the MFMA layout where LDS allows);
//   epilogue the accumulators move to an LDS tile. Row-wise passes (16
//            threads per row, so each row's factor vectors are read through
//            a row-uniform pointer with coalesced 16-byte accesses) fold
//            delta W into the rotated rows and scale by s; the expand adds
//            the own low-rank product t B' (not scaled by s: "The big
//            picture", s multiplies the base output only) and forms the
//            VeRA product u B_sh, which the last pass scales by e and adds
//            with b.
// With S > 1 the slices of a tile meet through a workspace written and read
// with system-coherent accesses; the last slice to arrive adds the slices in
// slice order and writes y.

#include <algorithm>

#include "internal.h"
#include "kernels.h"

namespace scute {



// ---------------------------------------------------------------------------
// prologue
// ---------------------------------------------------------------------------

// delta rows for one rotated item (<= 4 rows, one 64-column chunk): lane
// handles output column col of block kb = col / blk; the block's (R - I)^T
// row for that column and the rows' x block are contiguous, read in CH-wide
// vector batches (blk a multiple of CH)
template <int CH>
__device__ __forceinline__ void rotate_rows(const uint16_t* Pt, int32_t blk,
                                            const uint16_t* const (&xr)[4], int64_t col,
                                            float (&acc)[4]) {
  const int64_t kb = col / blk, jj = col - kb * blk;
  const uint16_t* prow = Pt + ((size_t)kb * blk + jj) * blk;
  for (int32_t i0 = 0; i0 < blk; i0 += CH) {
    uint4 pv[CH / 8], xv[4][CH / 8];
#pragma unroll
    for (int q = 0; q < CH / 8; ++q) pv[q] = ldg16(prow + i0 + 8 * q);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < CH / 8; ++q) xv[r][q] = ldg16(xr[r] + kb * blk + i0 + 8 * q);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < CH / 8; ++q) acc[r] = dot8(xv[r][q], pv[q], acc[r]);
  }
}

// One wave per work-group, so consecutive items (the heavy VeRA-shrink items
// come first) land on different compute units.
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 2)))
k_decode_prologue(ProArgs a) {
  const int lane = threadIdx.x;
  const int64_t d_in = a.d_in;
  {
    f32x4* z = reinterpret_cast<f32x4*>(a.acc_next);
    for (uint32_t i = blockIdx.x * 64 + lane; i < a.acc_words / 4; i += gridDim.x * 64)
      z[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int it = blockIdx.x; it < a.n_items; it += gridDim.x) {
    if (it < a.n_vitems) {
      // VeRA shrink block: 32 VeRA rows x 32 ranks of A_sh over one K slice
      // of 256 (one round of loads), scaled by d (per rank, so it commutes
      // with the K sum) and added into the row's VeRA slots. The block
      // follows from the item index, so its row records load at once.
      const int32_t per_kv = a.nvb * a.njb;
      const int32_t kv = it / per_kv, vb = (it - kv * per_kv) / a.njb;
      const int32_t jb = it - kv * per_kv - vb * a.njb;
      // 16x16x32 MFMA tiles (2 x 2 of them): lane (i, g) = (lane % 16,
      // lane / 16) holds row i of a 16-row block, k 8 g .. 8 g + 7 of each
      // 32-k step. Step ks takes the 64-byte half (ks % 2) of the 128-byte
      // chunk ks / 2 on both operands, so one load instruction covers 16 rows
      // x 64 contiguous bytes.
      const int i16 = lane & 15, g = lane >> 4;
      const DecVeraRow v0 = a.vrows[32 * vb + i16], v1 = a.vrows[32 * vb + 16 + i16];
      const int64_t kof = (int64_t)kv * 256 + 8 * g;
      const uint16_t* xr[2] = {a.x + (size_t)v0.tok * d_in + kof, a.x + (size_t)v1.tok * d_in + kof};
      const uint16_t* ar[2] = {a.A_sh + (size_t)(32 * jb + i16) * d_in + kof,
                               a.A_sh + (size_t)(32 * jb + 16 + i16) * d_in + kof};
      // output (bi, bj) element t: VeRA row 32 vb + 16 bi + 4 g + t,
      // rank 32 jb + 16 bj + i16
      float dsc[2][4][2];
      int32_t prow[2][4];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const DecVeraRow o = a.vrows[32 * vb + 16 * bi + 4 * g + t];
          prow[bi][t] = o.p;
#pragma unroll
          for (int bj = 0; bj < 2; ++bj) dsc[bi][t][bj] = ldg(o.vd + 32 * jb + 16 * bj + i16);
        }
      uint4 xa[2][8], wa[2][8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int off = 64 * (ks >> 1) + 32 * (ks & 1);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          xa[b][ks] = ldg16(xr[b] + off);
          wa[b][ks] = ldg16(ar[b] + off);
        }
      }
      f32x4 c[2][2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) c[bi][bj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
          for (int bj = 0; bj < 2; ++bj)
            c[bi][bj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_frag(xa[bi][ks]), as_frag(wa[bj][ks]),
                                                               c[bi][bj], 0, 0, 0);
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (prow[bi][t] >= 0) {
#pragma unroll
            for (int bj = 0; bj < 2; ++bj)
              atomicAdd(a.acc + (size_t)prow[bi][t] * a.AW + a.RT + 32 * jb + 16 * bj + i16,
                        c[bi][bj][t] * dsc[bi][t][bj]);
          }
      continue;
    }
    const DecProItem item = a.items[it];
    if (item.type == PRO_GATHER) {
      // one x row (d_in <= 8192: at most 16 16-byte pieces per lane)
      const uint16_t* src = a.x + (size_t)item.tok[0] * d_in;
      uint16_t* dst = a.xs + (size_t)item.p0 * d_in;
      u32x4 v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t c = (int64_t)lane * 8 + 512 * q;
        if (c < d_in) v[q] = *(const GLOBAL u32x4*)(src + c);
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t c = (int64_t)lane * 8 + 512 * q;
        if (c < d_in) *(GLOBAL u32x4*)(dst + c) = v[q];
      }
    } else if (item.type == PRO_ROT) {
      // delta[p][col] = sum_i x[tok p][kb blk + i] (R - I)[kb][i][col - kb blk]
      const int64_t col = (int64_t)item.k + lane;
      const int32_t blk = item.blk;
      const uint16_t* xr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) xr[r] = a.x + (size_t)item.tok[r] * d_in;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      if (col < d_in) {
        if (blk % 32 == 0) {
          rotate_rows<32>(item.ptr, blk, xr, col, acc);
        } else if (blk % 8 == 0) {
          rotate_rows<8>(item.ptr, blk, xr, col, acc);
        } else {
          const int64_t kb = col / blk, jj = col - kb * blk;
          const uint16_t* prow = item.ptr + ((size_t)kb * blk + jj) * blk;
          for (int32_t i = 0; i < blk; ++i) {
            const float pv = bf2f(ldg(prow + i));
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += bf2f(ldg(xr[r] + kb * blk + i)) * pv;
          }
        }
        uint16_t* drow = a.xs + (size_t)(a.M_pad + item.p0) * d_in + col;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (r < item.n) drow[(size_t)r * d_in] = f2bf(acc[r]);
      }
    } else if (item.type == PRO_SHRINK) {
      // own-term shrink t = x A' for up to 4 rows x 4 ranks over one K part
      // of 1024, added into the row's own-rank slots
      const int32_t len = item.n, k0 = item.k & 0xFFFF, nk = item.k >> 16;
      const int64_t cbeg = (int64_t)item.blk * 1024;
      const uint16_t* ar[4];
      const uint16_t* xr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) ar[j] = item.ptr + (size_t)(k0 + min(j, nk - 1)) * d_in + cbeg;
#pragma unroll
      for (int r = 0; r < 4; ++r) xr[r] = a.x + (size_t)item.tok[r] * d_in + cbeg;
      float acc[4][4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[r][j] = 0.f;
      {
        uint4 av[2][4], xv[2][4];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int64_t c = (int64_t)lane * 8 + 512 * cc;
          const bool ok = cbeg + c < d_in;
#pragma unroll
          for (int j = 0; j < 4; ++j) av[cc][j] = ok ? ldg16(ar[j] + c) : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) xv[cc][r] = ok ? ldg16(xr[r] + c) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[r][j] = dot8(xv[cc][r], av[cc][j], acc[r][j]);
      }
      float mine = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = wave_sum(acc[r][j]);
          if (lane == 4 * r + j) mine = v;
        }
      const int r = lane >> 2, j = lane & 3;
      if (lane < 16 && r < len && j < nk)
        atomicAdd(a.acc + (size_t)(item.p0 + r) * a.AW + k0 + j, mine);
    }
  }
}

// ---------------------------------------------------------------------------
// main GEMM + epilogue
// ---------------------------------------------------------------------------

struct MainArgs {
  const uint16_t* xs;               // [M_pad + 32 g_rot np][d_in] sorted x rows, then delta
                                    // rows, one block of 32 g_rot rows per projection
  const uint16_t* W;
  const DecRow* rows;               // [M_pad]
  const DecStep* steps;             // expand steps by slice and row group
  const int32_t* goff;              // [2 S MG + 1] step ranges, below
  const float* acc;                 // [M_pad][AW] shrink sums: RT own ranks, then r_v VeRA ranks
  const uint16_t* B_sh;             // [d_out][r_v] (dense VeRA expand)
  const float* zeros;               // [d_out]
  float* part;                      // [S][C][M_pad][64] split-K partial tiles (S > 1)
  int32_t* cnt;                     // [C] arrival counters, kept at zero between forwards
  float* y;
  uint32_t acc_bytes, part_bytes;
  // slice k, row group g (q = k MG + g): own steps [goff[2q], goff[2q+1]),
  // VeRA steps [goff[2q+1], goff[2q+2])
  int32_t MG;
  int32_t g_rot, d_in, d_out, k_chunk, S, C, RT, AW;
  int32_t gv0, gv1, r_v;            // dense VeRA expand over row groups [gv0, gv1) (gv1 > gv0)
  int32_t ptile[MAX_PROJ - 1];      // first column tile of projections 1.. (C past the last)
};

// Tile of the main kernel: 64 output columns (two 32-column MFMA blocks) by
// one of S slices of K; the 4 waves of a work-group are (column block cb,
// K half kp). The x / delta rows of each K half stream through an LDS ring
// of R stages of 64 k; W streams into registers (see WSrc).
constexpr int SK = 64;                 // k per stage
constexpr int SROW = 2 * SK;           // bytes per staged row
template <int MGT>
struct DecCfg {
  static constexpr int R = MGT <= 6 ? 3 : 2;        // ring depth
  static constexpr int STAGE = 32 * MGT * SROW;     // bytes per stage per K half
  // loads each wave issues per stage: 4 W + 2 MGT direct-to-LDS
  static constexpr int PER_STAGE = 4 + 2 * MGT;
  // outstanding loads allowed when waiting for stage t (see the loop)
  static constexpr int WAIT = (R - 2) * PER_STAGE + 4;
  // W loads whole rows per instruction and passes through a 4 KB LDS block
  // per wave when that block fits beside the ring and the row records (with
  // the 3-deep ring only: with 2 slots, as on the FFN-up shape, it measured
  // slower)
  static constexpr bool WLDS = R == 3 && R * 2 * STAGE + 4 * 4096 + 32 * MGT * 32 + 1024 <= 160 * 1024;
};



// Staged rows: 32 MGT rows (x rows of the sorted batch, then delta rows) of
// SROW bytes; the 16-byte piece index is XOR-swizzled by (row >> 1) & 7 to
// spread LDS banks. One direct-to-LDS instruction fills 8 rows (lane i ->
// row i / 8, slot i % 8); the two waves of a K half split the 4 MGT
// instructions of a stage (wave cb issues instructions cb + 2 q).
template <int MGT>
__device__ __forceinline__ void stage_rows(uint8_t* stage, const uint16_t* const (&src)[2 * MGT],
                                           int64_t koff, int cb) {
#pragma unroll
  for (int q = 0; q < 2 * MGT; ++q)
    __builtin_amdgcn_global_load_lds((const void*)(src[q] + koff),
                                     (lds_void*)(stage + (cb + 2 * q) * 1024), 16, 0, 0);
}

// W of one stage for one wave: 32 W rows (the wave's columns) x 128 bytes
// (64 k), addressed by a fixed per-lane buffer offset plus the stage's
// scalar offset. Two lane layouts:
//  - direct (rstep = 16 bytes): lane (m, h) loads the 64 contiguous bytes of its
//    own row m that it multiplies (pieces 4h .. 4h+3); each instruction then
//    touches 32 rows;
//  - through LDS (rstep = 8 rows): instruction s, lane l loads row
//    8 s + l / 8, piece (l % 8) ^ (l / 8), so one instruction covers 8 whole
//    rows; the wave writes the four registers to its LDS block in lane order
//    (row r's piece p lands in slot p ^ (r % 8)) and reads back the
//    direct layout, bank-conflict free.
struct WSrc {
  rsrc_t r;
  uint32_t voff, rstep;
  uint8_t* wsw;  // the wave's 4 KB LDS block (through-LDS layout)
};
__device__ __forceinline__ void load_w(uint4 (&wr)[4], const WSrc& ws, int64_t koff) {
  const int soff = (int)(koff * 2);
#pragma unroll
  for (int s = 0; s < 4; ++s)
    wr[s] = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(ws.r, ws.voff + s * ws.rstep, soff, 0));
}

// one stage: 4 MFMA k-steps of 16 over every staged row group
template <int MGT>
__device__ __forceinline__ void mma_stage(const uint8_t* stage, const uint4 (&wl)[4], const WSrc& ws,
                                          f32x16 (&acc)[MGT], int m, int h) {
  uint4 wr[4];
  if constexpr (DecCfg<MGT>::WLDS) {
    // through the wave's LDS block: the wave's own writes and reads, in order
#pragma unroll
    for (int s = 0; s < 4; ++s) *reinterpret_cast<uint4*>(ws.wsw + s * 1024 + (32 * h + m) * 16) = wl[s];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      wr[s] = *reinterpret_cast<const uint4*>(ws.wsw + m * 128 + 16 * ((4 * h + s) ^ (m & 7)));
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) wr[s] = wl[s];
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 av[MGT];
#pragma unroll
    for (int g = 0; g < MGT; ++g) {
      const int r = 32 * g + m;
      const int piece = (4 * h + s) ^ ((r >> 1) & 7);
      av[g] = *reinterpret_cast<const uint4*>(stage + r * SROW + 16 * piece);
    }
#pragma unroll
    for (int g = 0; g < MGT; ++g) acc[g] = mfma32(av[g], wr[s], acc[g]);
  }
}

// pipeline step t: issue W(t+R-1), wait for stage t, barrier, issue the rows
// of stage t+R-1 into the slot stage t-1 used, multiply stage t
template <int MGT>
__device__ __forceinline__ void kstep(int t, int nst, const WSrc& wrow,
                                      const uint16_t* const (&src)[2 * MGT], uint8_t* cur,
                                      uint8_t* nxt, uint4 (&wc)[4], uint4 (&wn)[4],
                                      f32x16 (&acc)[MGT], int m, int h, int cb, int kp) {
  constexpr int R = DecCfg<MGT>::R;
  const int64_t kn = (int64_t)SK * min(t + R - 1, nst - 1);
  load_w(wn, wrow, kn);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(DecCfg<MGT>::WAIT));
  wg_barrier();
  stage_rows<MGT>(nxt + kp * DecCfg<MGT>::STAGE, src, kn, cb);
  mma_stage<MGT>(cur + kp * DecCfg<MGT>::STAGE, wc, wrow, acc, m, h);
}

// The same step with the stage index T known at compile time: W is
// prefetched LW stages ahead into a ring of LW + 1 register sets (W is the
// stream from HBM, so it runs further ahead than the LDS rows), stages past
// the last are not prefetched, and the wait counts exactly the loads issued
// after stage T's rows (R = 3: the next stage's rows and W issued by the
// previous step; this step's W). Expands to the steps T .. NST-1. Step 1
// also runs `early` after its barrier (NE loads, counted at step 2).
template <int MGT, int NST, int LW, int T, int NE, typename Early>
__device__ __forceinline__ void ksteps_static(const WSrc& wrow, const uint16_t* const (&src)[2 * MGT],
                                              uint8_t* s0, uint8_t* s1, uint8_t* s2,
                                              uint4 (&wb)[LW + 1][4], f32x16 (&acc)[MGT], int m,
                                              int h, int cb, int kp, Early& early) {
  if constexpr (T < NST) {
    using Cfg = DecCfg<MGT>;
    constexpr int R = Cfg::R;
    constexpr int TN = T + R - 1;   // rows this step prefetches
    constexpr int TW = T + LW;      // W this step prefetches
    constexpr int allowed = (R == 3 && T + 1 < NST ? 2 * MGT : 0) +
                            (R == 3 && T - 1 + LW < NST ? 4 : 0) + (TW < NST ? 4 : 0) +
                            (R == 3 && T == 2 ? NE : 0);
    uint8_t* cur = T % R == 0 ? s0 : (T % R == 1 ? s1 : s2);
    uint8_t* nxt = TN % R == 0 ? s0 : (TN % R == 1 ? s1 : s2);
    if constexpr (TW < NST) load_w(wb[TW % (LW + 1)], wrow, (int64_t)SK * TW);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(allowed));
    wg_barrier();
    if constexpr (T == 1) {
      issue_fence();
      early();
      issue_fence();
    }
    if constexpr (TN < NST) stage_rows<MGT>(nxt + kp * Cfg::STAGE, src, (int64_t)SK * TN, cb);
    mma_stage<MGT>(cur + kp * Cfg::STAGE, wb[T % (LW + 1)], wrow, acc, m, h);
    ksteps_static<MGT, NST, LW, T + 1, NE>(wrow, src, s0, s1, s2, wb, acc, m, h, cb, kp, early);
  }
}

// Expand steps of one wave, 64 at a time: lane j holds the descriptor of
// step base + j (zeros past the list), read by every lane with readlane.
struct StepWin {
  u32x4 d;
  uint32_t plo, phi;
  int base;
};
__device__ __forceinline__ void load_win(const DecStep* steps, StepWin& w, int base, int end,
                                         int lane) {
  w.base = base;
  w.d = u32x4{0u, 0u, 0u, 0u};
  w.plo = w.phi = 0u;
  if (base + lane < end) {
    const GLOBAL u32x4* p = (const GLOBAL u32x4*)(steps + base + lane);
    w.d = p[0];
    const u32x4 q = p[1];
    w.plo = q.x;
    w.phi = q.y;
  }
}
struct StepDesc {
  int gk, kk, rank, lo, hi;
  const uint16_t* bp;
};
__device__ __forceinline__ StepDesc step_at(const StepWin& w, int j) {
  StepDesc d;
  d.gk = __builtin_amdgcn_readlane((int)w.d.x, j);
  d.kk = __builtin_amdgcn_readlane((int)w.d.y, j);
  d.rank = __builtin_amdgcn_readlane((int)w.d.z, j);
  const int lohi = __builtin_amdgcn_readlane((int)w.d.w, j);
  d.lo = lohi & 0xFFFF;
  d.hi = lohi >> 16;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)w.plo, j);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)w.phi, j);
  d.bp = (const uint16_t*)(((uint64_t)hi << 32) | lo);
  return d;
}

// Operands of one 16-rank expand step for lane (m, h) and both 32-column
// blocks of the tile: A = row 32 g + m's 8 shrink sums of ranks kk + 8 h ..
// (fp32 as stored), B = 8 bf16 of B' (or B_sh) row ncol (+ 32) from rank
// kk + 8 h. Loads go through buffer resources, so nothing past an operand
// is read (ranks past the term's rank read zeros or are zeroed below).
struct StepOps {
  uint4 a0, a1, b0, b1;
  int32_t ok;  // lane's row inside the step's rows and ranks inside the term
};
__device__ __forceinline__ StepOps load_step(const MainArgs& a, const StepDesc& d, int g,
                                             int64_t ncol, int m, int h) {
  StepOps o;
  const int kk = d.kk + 8 * h;
  const int row = 32 * g + m;
  const int acol = (d.gk & STEP_VERA) ? a.RT : 0;
  const rsrc_t ar = make_rsrc(a.acc, a.acc_bytes);
  const rsrc_t br = make_rsrc(d.bp, (uint32_t)(a.d_out * d.rank * 2));
  const uint32_t ao = (uint32_t)(((int64_t)row * a.AW + acol + kk) * 4);
  o.a0 = ldb16(ar, ao);
  o.a1 = ldb16(ar, ao + 16);
  o.b0 = ldb16(br, (uint32_t)((ncol * d.rank + kk) * 2));
  o.b1 = ldb16(br, (uint32_t)(((ncol + 32) * d.rank + kk) * 2));
  o.ok = kk < d.rank && row >= d.lo && row < d.hi;
  return o;
}
__device__ __forceinline__ void mma_step(const StepOps& o, f32x16& c0, f32x16& c1) {
  const uint4 av = o.ok ? make_uint4(pack_bf2(o.a0.x, o.a0.y), pack_bf2(o.a0.z, o.a0.w),
                                     pack_bf2(o.a1.x, o.a1.y), pack_bf2(o.a1.z, o.a1.w))
                        : make_uint4(0, 0, 0, 0);
  c0 = mfma32(av, o.b0, c0);
  c1 = mfma32(av, o.b1, c1);
}
// Up to NB steps' operands, loaded together (one memory round trip per
// batch); the window must hold the descriptors of steps [s, s + NB) that
// exist (those below e1).
template <int NB>
struct StepBatch {
  StepOps o[NB];
};
template <int NB>
__device__ __forceinline__ void load_batch(const MainArgs& a, const StepWin& w, int s, int e1,
                                           int g, int64_t ncol, int m, int h, StepBatch<NB>& b) {
#pragma unroll
  for (int j = 0; j < NB; ++j)
    if (s + j < e1) b.o[j] = load_step(a, step_at(w, s + j - w.base), g, ncol, m, h);
}
// The expand of one row group in this slice: steps [e0, ev) are own steps
// (summed into o0 / o1), [ev, e1) VeRA steps (into v0 / v1), for column
// blocks 0 / 1. `b` holds the first batch already when `loaded`; the window
// `w` starts at e0.
template <int NB>
__device__ __forceinline__ void expand_group(const MainArgs& a, StepWin& w, StepBatch<NB>& b,
                                             bool loaded, int e0, int ev, int e1, int g,
                                             int64_t ncol, int m, int h, int lane, f32x16& o0,
                                             f32x16& o1, f32x16& v0, f32x16& v1) {
  for (int s = e0; s < e1; s += NB) {
    if (s != e0 || !loaded) {
      if (s + NB > w.base + 64 && e1 > w.base + 64) load_win(a.steps, w, s, e1, lane);
      load_batch(a, w, s, e1, g, ncol, m, h, b);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int st = s + j;
      if (st < e1) {
        if (st < ev)
          mma_step(b.o[j], o0, o1);
        else
          mma_step(b.o[j], v0, v1);
      }
    }
  }
}

// Dense VeRA expand of one slice: the VeRA rows' products u B_sh over the
// slice's share [16 ks0, 16 ks1) of the r_v ranks, for row groups
// [gv0, gv1) (rows there without a VeRA term have zero sums). In chunks of up
// to 128 ranks, the work-group stages the rows' sums as bf16 in V's LDS
// buffer (rows of 16 pieces of 16 bytes, piece p of row r at p ^ (r & 15), so
// the MFMA reads of 16 rows hit 16 different bank groups) and each wave
// multiplies its groups (K half kp takes every other group) in registers,
// with its column's B_sh pieces for every rank step loaded once up front.
// The products go to V after every wave is done reading the staged sums.
template <int MGT>
__device__ __forceinline__ void dense_vera(const MainArgs& a, float* V, int32_t* vflag, int kc,
                                           int cb, int kp, int tid, int m, int h, int64_t ncol) {
  constexpr int MAXG = (MGT + 1) / 2;  // groups per wave
  const int nks = a.r_v / 16;
  const int ks0 = kc * nks / a.S, ks1 = (kc + 1) * nks / a.S, nk = ks1 - ks0;
  if (nk <= 0) return;  // uniform over the work-group
  const int rows = 32 * (a.gv1 - a.gv0);
  uint8_t* U = reinterpret_cast<uint8_t*>(V);
  // this lane's B_sh pieces: rank 16 (ks0 + ks) + 8 h .. + 7 of column ncol
  uint4 b[16];
  {
    const rsrc_t br = make_rsrc(a.B_sh, (uint32_t)((size_t)a.d_out * a.r_v * 2));
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      if (ks < nk) b[ks] = ldb16(br, (uint32_t)((ncol * a.r_v + 16 * (ks0 + ks) + 8 * h) * 2));
  }
  const rsrc_t ar = make_rsrc(a.acc, a.acc_bytes);
  f32x16 vacc[MAXG];
#pragma unroll
  for (int q = 0; q < MAXG; ++q) vacc[q] = f32x16{};
#pragma unroll
  for (int ch = 0; ch < 2; ++ch) {
    const int k0 = 8 * ch, kn = min(8, nk - k0);
    if (kn <= 0) break;  // uniform
    if (ch > 0) lds_barrier();  // every wave is done with the previous chunk
    // stage piece p (8 ranks) of row r: 2 kn pieces per row, at most 16 per thread
    const int pr = 2 * kn, pieces = rows * pr;
    u32x4 raw[16][2];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int pi = tid + 256 * q;
      if (pi < pieces) {
        const int r = pi / pr, p = pi - r * pr;
        const uint32_t off = (uint32_t)((((int64_t)(32 * a.gv0 + r) * a.AW) + a.RT +
                                         16 * (ks0 + k0) + 8 * p) * 4);
        raw[q][0] = __builtin_bit_cast(u32x4, ldb16(ar, off));
        raw[q][1] = __builtin_bit_cast(u32x4, ldb16(ar, off + 16));
      }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int pi = tid + 256 * q;
      if (pi < pieces) {
        const int r = pi / pr, p = pi - r * pr;
        const u32x4 v0 = raw[q][0], v1 = raw[q][1];
        const u32x4 o = u32x4{pack_bf2(v0.x, v0.y), pack_bf2(v0.z, v0.w), pack_bf2(v1.x, v1.y),
                              pack_bf2(v1.z, v1.w)};
        *reinterpret_cast<u32x4*>(U + (16 * r + (p ^ (r & 15))) * 16) = o;
      }
    }
    lds_barrier();
#pragma unroll
    for (int q = 0; q < MAXG; ++q) {
      const int g = a.gv0 + kp + 2 * q;
      if (g < a.gv1) {
        const int r = 32 * (g - a.gv0) + m;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          if (ks < kn) {
            const uint4 av =
                *reinterpret_cast<const uint4*>(U + (16 * r + ((2 * ks + h) ^ (r & 15))) * 16);
            vacc[q] = mfma32(av, b[k0 + ks], vacc[q]);
          }
        }
      }
    }
  }
  lds_barrier();  // every wave is done with the staged sums
#pragma unroll
  for (int q = 0; q < MAXG; ++q) {
    const int g = a.gv0 + kp + 2 * q;
    if (g < a.gv1) {
      float* Vg = V + 32 * g * 64 + cb * 32 + m;
#pragma unroll
      for (int i = 0; i < 16; ++i) Vg[(8 * (i >> 2) + 4 * h + (i & 3)) * 64] = vacc[q][i];
      if (tid == 0 || tid == 64 || tid == 128 || tid == 192) vflag[g] = 1;
    }
  }
}

// Row record in LDS: [0] = (s, e) pointers, [1] = (b pointer, token, flags)
__device__ __forceinline__ const float* rec_ptr(u32x4 v, int hi) {
  const uint64_t p = hi ? ((uint64_t)v.w << 32 | v.z) : ((uint64_t)v.y << 32 | v.x);
  return (const float*)p;
}

// MGT = staged row groups = x row groups + g_rot delta groups; NST = 64-k
// stages per K half when known at compile time (the K loop is then fully
// unrolled, which keeps the compiler's tracking of the in-flight LDS fills
// exact), 0 for a runtime count
template <int MGT, int NST>
__global__ void __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_decode_main(MainArgs a) {
  using Cfg = DecCfg<MGT>;
  constexpr int R = Cfg::R;
  // ring slots as separate LDS objects so the compiler can tell the slot
  // being read from the ones the direct loads fill; after the K loop slot0
  // holds the row tile T and slot1 the VeRA tile V ([32 MGT][64] fp32 each)
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[2 * Cfg::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[2 * Cfg::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t slot2[R == 3 ? 2 * Cfg::STAGE : 16];
  __shared__ u32x4 rec[32 * MGT][2];   // row records of the x rows
  __shared__ int32_t vflag[MGT];       // V holds the group's VeRA product
  __shared__ int32_t last_flag;
  __shared__ __attribute__((aligned(1024))) uint8_t wst[Cfg::WLDS ? 4 * 4096 : 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int m = lane & 31, h = lane >> 5;
  const int cb = wave & 1, kp = wave >> 1;
  const int mgx = MGT - a.g_rot;  // x row groups
  const int Mx = 32 * mgx;

  // grid (tile, slice): work-groups are dispatched round-robin over the 8
  // XCDs in linear order slice * C + tile, so with C a multiple of 8 the S
  // slices of a tile share one XCD and its L2
  const int c = blockIdx.x, kc = blockIdx.y;

  const int64_t ncol = (int64_t)c * 64 + cb * 32 + m;
  const int kw = a.k_chunk / 2;  // K per half
  const int64_t kbase = (int64_t)kc * a.k_chunk + (int64_t)kp * kw;
  const int nst = NST > 0 ? NST : kw / SK;
  const rsrc_t wr_rsrc = make_rsrc(a.W, (uint32_t)((size_t)a.d_out * a.d_in * 2));
  const WSrc wrow =
      Cfg::WLDS ? WSrc{wr_rsrc,
                       (uint32_t)((((size_t)c * 64 + cb * 32 + (lane >> 3)) * a.d_in + kbase) * 2 +
                                  16 * ((lane & 7) ^ (lane >> 3))),
                       (uint32_t)(8 * a.d_in * 2), wst + (Cfg::WLDS ? wave * 4096 : 0)}
                : WSrc{wr_rsrc, (uint32_t)(((size_t)ncol * a.d_in + kbase + 32 * h) * 2), 16u, wst};

  // (0) record of the row this thread keeps for the epilogue
  // (branch-free, so the compiler can fetch the kernel arguments at once)
  const GLOBAL u32x4* rp = (const GLOBAL u32x4*)(a.rows + min(tid, Mx - 1));
  const u32x4 rec0 = rp[0], rec1 = rp[1];
  // (1) W of the first LW = R - 1 stages (with NST known, stages past the
  //     last are not loaded)
  constexpr int LW = R - 1;
  constexpr bool pre1 = R == 3 && NST != 1;
  uint4 wb[LW + 1][4];
  load_w(wb[0], wrow, 0);
  if constexpr (NST > 0) {
#pragma unroll
    for (int t = 1; t < LW; ++t)
      if (t < NST) load_w(wb[t], wrow, (int64_t)SK * t);
  } else if constexpr (pre1) {
    load_w(wb[1], wrow, (int64_t)SK * min(1, nst - 1));
  }
  // (2) row sources: staged row r (x rows, then delta rows) is row r of xs,
  //     the delta rows taken from this tile's projection's block
  const uint16_t* src[2 * MGT];
  {
    const int piece = (lane & 7) ^ ((4 * cb + (lane >> 4)) & 7);
    const int dsh = 32 * a.g_rot * ((c >= a.ptile[0]) + (c >= a.ptile[1]) + (c >= a.ptile[2]));
#pragma unroll
    for (int q = 0; q < 2 * MGT; ++q) {
      const int r = 8 * (cb + 2 * q) + (lane >> 3);
      src[q] = a.xs + (size_t)(r + (r >= Mx ? dsh : 0)) * a.d_in + kbase + 8 * piece;
    }
  }
  stage_rows<MGT>(slot0 + kp * Cfg::STAGE, src, 0, cb);
  if constexpr (pre1) stage_rows<MGT>(slot1 + kp * Cfg::STAGE, src, (int64_t)SK * min(1, nst - 1), cb);
  // (3) the expand steps of this wave's first row group (row group `wave`
  //     of the x rows): its step range and first 64 descriptors load now
  int g_e0 = 0, g_ev = 0, g_e1 = 0;
  if (wave < mgx) {
    const int q = 2 * (kc * a.MG + wave);
    g_e0 = uni(a.goff[q]);
    g_ev = uni(a.goff[q + 1]);
    g_e1 = uni(a.goff[q + 2]);
  }
  StepWin win;
  load_win(a.steps, win, g_e0, g_e1, lane);

  f32x16 acc[MGT];
#pragma unroll
  for (int g = 0; g < MGT; ++g) acc[g] = f32x16{};

  // epilogue layout: 16 threads per row, a float4 of the tile's 64 columns
  // each; every row's s vector loads during the K loop (step 1, once the row
  // records are in LDS), so the first row pass does not wait for it
  const int q4 = tid & 15, rr = tid >> 4;  // float4 of the row, row within 16
  const int nj = 2 * mgx;                  // passes of 16 rows over the x rows
  const int64_t cbase = (int64_t)c * 64 + 4 * q4;
  f32x4 s4[2 * MGT];
  auto issue_s = [&]() {
    // the s pointers (first 8 bytes of each record) read together, then the
    // vectors, so the LDS reads overlap
    const float* sp[2 * MGT];
#pragma unroll
    for (int j = 0; j < 2 * MGT; ++j) {
      const int r = rr + 16 * min(j, nj - 1);
      sp[j] = *reinterpret_cast<const float* const*>(&rec[r][0]);
    }
#pragma unroll
    for (int j = 0; j < 2 * MGT; ++j) s4[j] = ldg4(sp[j] + cbase);
  };
  constexpr bool s_early = NST >= 2;

  // stage 0 (peeled: the row records go to LDS after its barrier)
  {
    constexpr bool pre = NST == 0 || R - 1 < NST;   // rows of stage R-1
    constexpr bool prew = NST == 0 || LW < NST;     // W of stage LW
    const int64_t kn = (int64_t)SK * min(R - 1, nst - 1);
    if constexpr (prew) load_w(wb[LW], wrow, (int64_t)SK * min(LW, nst - 1));
    // issued after the rows of stage 0: (R == 3: rows of stage 1) and W of
    // stage LW
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((pre1 ? 2 * MGT : 0) + (prew ? 4 : 0)));
    wg_barrier();
    if (tid < Mx) {
      rec[tid][0] = rec0;
      rec[tid][1] = rec1;
    }
    if (tid < MGT) vflag[tid] = 0;
    if constexpr (pre) stage_rows<MGT>((R == 3 ? slot2 : slot1) + kp * Cfg::STAGE, src, kn, cb);
    mma_stage<MGT>(slot0 + kp * Cfg::STAGE, wb[0], wrow, acc, m, h);
  }
  // remaining stages; stage t lives in ring slot t % R and W registers
  // wb[t % R], named statically in both forms of the loop
  if constexpr (NST > 0) {
    ksteps_static<MGT, NST, LW, 1, s_early ? 2 * MGT : 0>(wrow, src, slot0, slot1, slot2, wb, acc, m,
                                                        h, cb, kp, issue_s);
  } else if constexpr (R == 3) {
#pragma unroll 1
    for (int t = 1; t < nst; t += 3) {
      kstep<MGT>(t, nst, wrow, src, slot1, slot0, wb[1], wb[0], acc, m, h, cb, kp);
      if (t + 1 >= nst) break;
      kstep<MGT>(t + 1, nst, wrow, src, slot2, slot1, wb[2], wb[1], acc, m, h, cb, kp);
      if (t + 2 >= nst) break;
      kstep<MGT>(t + 2, nst, wrow, src, slot0, slot2, wb[0], wb[2], acc, m, h, cb, kp);
    }
  } else {
#pragma unroll 1
    for (int t = 1; t < nst; t += 2) {
      kstep<MGT>(t, nst, wrow, src, slot1, slot0, wb[1], wb[0], acc, m, h, cb, kp);
      if (t + 1 >= nst) break;
      kstep<MGT>(t + 1, nst, wrow, src, slot0, slot1, wb[0], wb[1], acc, m, h, cb, kp);
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // clamped tail prefetches
  wg_barrier();

  // ---- epilogue ---------------------------------------------------------------
  // the first expand batch's operands and the rows' factor vectors are in
  // flight while the K halves meet
  // (the e and b vectors first: their row records come from LDS, and with
  // the batch's registers not yet taken the reads overlap)
  if constexpr (!s_early) issue_s();
  constexpr bool early_f = MGT <= 6;       // register room to fetch e and b here too
  f32x4 e4[2 * MGT], b4[2 * MGT];
  if constexpr (early_f) {
    u32x4 re[2 * MGT], rb[2 * MGT];
#pragma unroll
    for (int j = 0; j < 2 * MGT; ++j) {
      const int r = rr + 16 * min(j, nj - 1);
      re[j] = rec[r][0];
      rb[j] = rec[r][1];
    }
#pragma unroll
    for (int j = 0; j < 2 * MGT; ++j) {
      e4[j] = ldg4(rec_ptr(re[j], 1) + cbase);
      b4[j] = ldg4((kc == 0 ? rec_ptr(rb[j], 0) : a.zeros) + cbase);
    }
  }
  const int64_t ncol0 = (int64_t)c * 64 + m;
  constexpr int NB = MGT <= 5 ? 8 : 4;  // register room
  StepBatch<NB> sb;
  load_batch(a, win, g_e0, g_e1, wave, ncol0, m, h, sb);

  // (a) K halves meet in T [32 MGT rows][64 columns]; accumulator element i
  //     of group g is row 32 g + 8 (i / 4) + 4 h + i % 4, column cb 32 + m
  float* T = reinterpret_cast<float*>(slot0);
  float* V = reinterpret_cast<float*>(slot1);
  {
    float* Tk = kp == 0 ? V : T;  // K half 0 -> V, K half 1 -> T
#pragma unroll
    for (int g = 0; g < MGT; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        Tk[(32 * g + 8 * (i >> 2) + 4 * h + (i & 3)) * 64 + cb * 32 + m] = acc[g][i];
  }
  lds_barrier();  // other waves read these LDS writes next

  // (b) row pass 1: fold delta W into the rotated rows (delta row r belongs
  //     to sorted row r; delta rows past n_rot are zero) and scale by s
  f32x4* T4 = reinterpret_cast<f32x4*>(T);
  f32x4* V4 = reinterpret_cast<f32x4*>(V);
  {
    f32x4 v[2 * MGT], dv[2 * MGT];
#pragma unroll
    for (int j = 0; j < 2 * MGT; ++j) {
      const int r = rr + 16 * min(j, nj - 1);
      v[j] = T4[r * 16 + q4] + V4[r * 16 + q4];
      dv[j] = j < 2 * a.g_rot ? T4[(Mx + r) * 16 + q4] + V4[(Mx + r) * 16 + q4]
                              : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < 2 * MGT; ++j)
      if (j < nj) T4[(rr + 16 * j) * 16 + q4] = (v[j] + dv[j]) * s4[j];
  }
  lds_barrier();

  // (c) expand: wave w takes row groups w, w + 4, .. of the x rows and both
  //     column blocks. A group's own steps (A rows zero outside each step's
  //     segment) sum in registers and are added into T's rows of the group
  //     (every read before any write); its VeRA steps sum into V's rows of
  //     the group. No two waves touch the same rows.
  for (int g = wave; g < mgx; g += 4) {
    int e0 = g_e0, ev = g_ev, e1 = g_e1;
    if (g != wave) {
      const int q = 2 * (kc * a.MG + g);
      e0 = uni(a.goff[q]);
      ev = uni(a.goff[q + 1]);
      e1 = uni(a.goff[q + 2]);
      load_win(a.steps, win, e0, e1, lane);
    }
    if (e1 <= e0) continue;
    f32x16 o0 = {}, o1 = {}, v0 = {}, v1 = {};
    expand_group(a, win, sb, g == wave, e0, ev, e1, g, ncol0, m, h, lane, o0, o1, v0, v1);
    if (ev > e0) {
      float* Tg = T + 32 * g * 64 + m;
      float old[32];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        old[i] = Tg[(8 * (i >> 2) + 4 * h + (i & 3)) * 64];
        old[16 + i] = Tg[(8 * (i >> 2) + 4 * h + (i & 3)) * 64 + 32];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        Tg[(8 * (i >> 2) + 4 * h + (i & 3)) * 64] = old[i] + o0[i];
        Tg[(8 * (i >> 2) + 4 * h + (i & 3)) * 64 + 32] = old[16 + i] + o1[i];
      }
    }
    if (e1 > ev) {
      float* Vg = V + 32 * g * 64 + m;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        Vg[(8 * (i >> 2) + 4 * h + (i & 3)) * 64] = v0[i];
        Vg[(8 * (i >> 2) + 4 * h + (i & 3)) * 64 + 32] = v1[i];
      }
      if (lane == 0) vflag[g] = 1;
    }
  }
  if (a.gv1 > a.gv0) dense_vera<MGT>(a, V, vflag, kc, cb, kp, tid, m, h, ncol);
  lds_barrier();

  // (d) row pass 2: this slice's tile = T + (V (.) e) + b (b on slice 0 only)
  f32x4 out[2 * MGT];
  {
    if constexpr (!early_f) {
      // (records read together first, so the LDS reads overlap)
      u32x4 re[2 * MGT], rb[2 * MGT];
#pragma unroll
      for (int j = 0; j < 2 * MGT; ++j) {
        const int r = rr + 16 * min(j, nj - 1);
        re[j] = rec[r][0];
        rb[j] = rec[r][1];
      }
#pragma unroll
      for (int j = 0; j < 2 * MGT; ++j) {
        e4[j] = ldg4(rec_ptr(re[j], 1) + cbase);
        b4[j] = ldg4((kc == 0 ? rec_ptr(rb[j], 0) : a.zeros) + cbase);
      }
    }
#pragma unroll
    for (int j = 0; j < 2 * MGT; ++j) {
      const int r = rr + 16 * min(j, nj - 1);
      f32x4 u = V4[r * 16 + q4];
      if (!vflag[min(j, nj - 1) >> 1]) u = f32x4{0.f, 0.f, 0.f, 0.f};
      out[j] = T4[r * 16 + q4] + u * e4[j] + b4[j];
    }
  }

  if (a.S == 1) {
#pragma unroll
    for (int j = 0; j < 2 * MGT; ++j) {
      if (j < nj) {
        const int tk = (int)rec[rr + 16 * j][1].z;
        if (tk >= 0) stg4(a.y + (size_t)tk * a.d_out + cbase, out[j]);
      }
    }
    return;
  }

  // (e) S slices of the tile meet: store this slice's tile, wait for the
  //     stores, count arrivals; the last slice to arrive adds every slice's
  //     tile in slice order (slices past S read as zero) and writes y
  const rsrc_t pr = make_rsrc(a.part, a.part_bytes);
  const uint32_t slice_bytes = (uint32_t)a.C * (uint32_t)Mx * 256u;
  const uint32_t tile = (uint32_t)c * (uint32_t)Mx * 256u + (uint32_t)q4 * 16u;
#pragma unroll
  for (int j = 0; j < 2 * MGT; ++j)
    if (j < nj) st_sys4(pr, (uint32_t)kc * slice_bytes + tile + (uint32_t)(rr + 16 * j) * 256u, out[j]);
  wait_vm_all();
  wg_barrier();
  if (tid == 0) {
    const int old = arrive(a.cnt + c);
    last_flag = old == a.S - 1;
    if (old == a.S - 1) reset_counter(a.cnt + c);
  }
  lds_barrier();  // last_flag is read by every wave
  if (!last_flag) return;
  f32x4 tot[2 * MGT];
#pragma unroll
  for (int j = 0; j < 2 * MGT; ++j) tot[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int j = 0; j < 2 * MGT; ++j) {
      const int r = rr + 16 * min(j, nj - 1);
      tot[j] += ld_sys4(pr, (uint32_t)s * slice_bytes + tile + (uint32_t)r * 256u);
    }
#pragma unroll
  for (int j = 0; j < 2 * MGT; ++j) {
    if (j < nj) {
      const int tk = (int)rec[rr + 16 * j][1].z;
      if (tk >= 0) stg4(a.y + (size_t)tk * a.d_out + cbase, tot[j]);
    }
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------

void launch_prologue(const ProArgs& pa, int grid, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  hipExtLaunchKernelGGL(k_decode_prologue, dim3(grid), dim3(64), 0, st, e0, e1, 0, pa);
}

template <int MGT>
static void launch_main(const MainArgs& a, dim3 grid, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  switch (a.k_chunk / 2 / SK) {
    case 8: hipExtLaunchKernelGGL((k_decode_main<MGT, 8>), grid, dim3(256), 0, st, e0, e1, 0, a); break;
    case 32: hipExtLaunchKernelGGL((k_decode_main<MGT, 32>), grid, dim3(256), 0, st, e0, e1, 0, a); break;
    default: hipExtLaunchKernelGGL((k_decode_main<MGT, 0>), grid, dim3(256), 0, st, e0, e1, 0, a); break;
  }
}

scute_status launch_decode(scute_layer* L, const scute_batch* B, const void* x, const void* W,
                           float* y, hipStream_t st, int32_t* launches) {
  const DecodePlan& D = B->dp;
  // the shrink sums of this forward and the buffer cleared for the next
  float* acc = D.acc32[D.fwd & 1];
  float* acc_next = D.acc32[(D.fwd + 1) & 1];
  int nl = 0;
  if (D.route) {  // route variant: the rotation as a pass of its own
    scute_status rs = launch_route_rotate(L, B, x, st, &nl);
    if (rs != SCUTE_OK) return rs;
  }
  {
    ProArgs pa{};
    pa.x = (const uint16_t*)x;
    pa.items = D.pro_items;
    pa.n_items = D.n_pro;
    pa.n_vitems = D.n_vitems;
    pa.nvb = D.nvb;
    pa.njb = D.njb;
    pa.vrows = D.vrows;
    pa.A_sh = (const uint16_t*)L->A_sh;
    pa.xs = D.xs;
    pa.acc = acc;
    pa.acc_next = acc_next;
    pa.acc_words = D.acc_bytes / 4;
    pa.M_pad = D.M_pad;
    pa.AW = D.AW;
    pa.RT = D.RT;
    pa.d_in = (int32_t)L->d_in;
    const int grid = std::max(1, std::min(8192, pa.n_items));
    ProfScope ps(L, st, "decode_prologue", true);
    launch_prologue(pa, grid, st, ps.ev_start(), ps.ev_stop());
    ++nl;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "launch k_decode_prologue");
    // the prologue cleared acc_next: only now may the next forward use it
    ++D.fwd;
  }
  MainArgs ma{};
  ma.xs = D.xs;
  ma.W = (const uint16_t*)W;
  ma.rows = D.rows;
  ma.steps = D.steps;
  ma.acc = acc;
  ma.zeros = D.zeros;
  ma.part = D.part;
  ma.cnt = D.cnt;
  ma.y = y;
  ma.acc_bytes = D.acc_bytes;
  ma.part_bytes = D.part_bytes;
  ma.goff = D.goff;
  ma.MG = D.MG;
  ma.g_rot = D.g_rot;
  ma.d_in = (int32_t)L->d_in;
  ma.d_out = (int32_t)L->d_out;
  ma.k_chunk = D.k_chunk;
  ma.S = D.S;
  ma.C = D.C;
  ma.RT = D.RT;
  ma.AW = D.AW;
  ma.B_sh = (const uint16_t*)L->B_sh;
  ma.gv0 = D.gv0;
  ma.gv1 = D.gv1;
  ma.r_v = L->r_v;
  for (int32_t i = 0; i + 1 < MAX_PROJ; ++i) ma.ptile[i] = D.ptile[i];
  const dim3 grid(D.C, D.S);
  ProfScope ps(L, st, "decode_main", true);
  switch (D.MG + D.g_rot) {
    case 1: launch_main<1>(ma, grid, st, ps.ev_start(), ps.ev_stop()); break;
    case 3: launch_main<3>(ma, grid, st, ps.ev_start(), ps.ev_stop()); break;
    case 4: launch_main<4>(ma, grid, st, ps.ev_start(), ps.ev_stop()); break;
    case 5: launch_main<5>(ma, grid, st, ps.ev_start(), ps.ev_stop()); break;
    case 6: launch_main<6>(ma, grid, st, ps.ev_start(), ps.ev_stop()); break;
    case 7: launch_main<7>(ma, grid, st, ps.ev_start(), ps.ev_stop()); break;
    case 8: launch_main<8>(ma, grid, st, ps.ev_start(), ps.ev_stop()); break;
    case 9: launch_main<9>(ma, grid, st, ps.ev_start(), ps.ev_stop()); break;
    default: return fail(SCUTE_E_UNSUPPORTED, "decode path: unsupported staged row groups");
  }
  ++nl;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch k_decode_main");
  if (D.route) {  // route variant: the passes after the GEMM
    scute_status rs = launch_route_passes(L, B, y, acc, st, &nl);
    if (rs != SCUTE_OK) return rs;
  }
  if (launches) *launches = nl;
  return SCUTE_OK;
}

}  // namespace scute
