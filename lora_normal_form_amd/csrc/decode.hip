// MFMA decode path (bf16 activations, fp32 accumulate, up to 256 rows).
//
// Two kernels per forward:
//   k_decode_prologue: zero y (when the GEMM splits K), OFT rotation
//     delta = x (R - I), own-term shrink t = x A', VeRA shrink over the whole
//     batch u = (x A_sh) (.) d. Rotation runs before the shared GEMM and the
//     shared VeRA pair is read once per step ("Where is the cheapest place to
//     compute the remaining slots?", paper-daily.com explainer of "Scute:
//     Exact Batched Serving for PEFT Adapters Beyond LoRA").
//   k_decode_main: the shared GEMM y = (x W + delta W) (.) s + b for the whole
//     batch on 32x32x16 bf16 MFMA, then the expand in the epilogue: the own
//     low-rank update t B' and the VeRA term (u B_sh) (.) e, added unscaled
//     by s ("The big picture": s multiplies the base output, the low-rank sum
//     is added after).
//
// Layout of the main kernel. A work-group of 4 waves owns 128 output columns
// (32 per wave) and one of S slices of the K dimension; its partial product
// for all rows (row groups of 32) is scaled by s and added into y with float
// atomics (y zeroed by the prologue) when S > 1, stored directly when S = 1.
// W is the MFMA B operand, streamed from HBM straight into registers: each
// lane loads 64 contiguous bytes of one W row per 128-wide K block (two 32-k
// halves of a 64-k sub-block); the MFMA's k index is permuted consistently on
// both operands so the contraction is unchanged. x (and delta) rows are the
// A operand, staged in LDS with direct global->LDS loads, 256-byte rows with
// the 16-byte chunk index XOR-swizzled by the row to spread LDS banks.

#include <algorithm>

#include "internal.h"

namespace scute {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

namespace {

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f2bf(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}
__device__ __forceinline__ bf16x8 as_frag(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_frag(a), as_frag(b), c, 0, 0, 0);
}
// Pointers read from tables are generic to the compiler; loads through these
// helpers name the global address space so they become global (not flat)
// loads and need no wait on the LDS counter.
#define GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ T ldg(const T* p) {
  return *(const GLOBAL T*)p;
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  const u32x4 v = *(const GLOBAL u32x4*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ldg16_stream(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load((const GLOBAL u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float dot8(uint4 a, uint4 b) {
  const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s += __uint_as_float(av[i] << 16) * __uint_as_float(bv[i] << 16);
    s += __uint_as_float(av[i] & 0xFFFF0000u) * __uint_as_float(bv[i] & 0xFFFF0000u);
  }
  return s;
}
// Exchange of partial results between work-groups on any XCD without
// whole-cache maintenance: the exchanged values are written and read with
// system-scope relaxed atomic stores and loads (sc0 sc1: written through to
// memory and read from memory, past the per-XCD L2). Being ordinary
// compiler-visible memory operations, their results are waited for by the
// compiler. A writer waits for its stores to complete before announcing them
// with an atomic on a counter; a reader issues its loads only after the
// atomic that saw every announcement has returned.
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ int arrive(int32_t* cnt) {
  return __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void reset_counter(int32_t* cnt) {
  __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

enum : int32_t { PRO_ROT = 0, PRO_SHRINK = 1, PRO_VSHRINK = 2 };
enum : int32_t { EXP_OWN = 0, EXP_VERA = 1 };

}  // namespace

// ---------------------------------------------------------------------------
// prologue
// ---------------------------------------------------------------------------

struct ProArgs {
  const uint16_t* x;
  const int32_t* perm;         // sorted position -> token
  const int32_t* row_adapter;  // sorted position -> adapter
  const int32_t* vera_pos;     // VeRA row index -> sorted position
  const SlotEntry* table;
  const uint16_t* A_sh;        // [r_v][d_in]
  float* y;                    // zeroed when zero_y
  int64_t y_vec4;              // n * d_out / 4
  int32_t zero_y;
  const int4* items;
  int32_t n_items;
  uint16_t* tb;                // [M_pad][RT]
  int32_t RT;
  uint16_t* ub;                // [M_pad][r_v]
  int32_t r_v;
  uint16_t* delta;             // [32 g_rot][d_in]
  float* vpart;                // [SV][nvb * njb][1024]
  int32_t* vcnt;               // [nvb * njb]
  int32_t nvb, njb, SV, n_vera;
  int32_t d_in;
  const int4* sgroups;         // own-term shrink groups (first row, rows, first rank, ranks)
  float* spart;                // [KQ][n_sgroups][16] partial dot products
  int32_t* scnt;               // [n_sgroups] arrival counters (kept at zero)
  int32_t n_sgroups, KQ;
};

// delta rows for one rotated segment chunk (<= R rows, one 64-column chunk):
// lane handles output column col = c0 + lane of block kb = col / blk; the
// block's (R - I)^T row for that column and the rows' x block are contiguous,
// read in CH-wide vector batches (blk a multiple of CH)
template <int CH, int R>
__device__ __forceinline__ void rotate_rows(const ProArgs& a, const uint16_t* Pt, int32_t blk,
                                            const uint16_t* const (&xr)[R], int32_t nr,
                                            int64_t col, float (&acc)[R]) {
  const int64_t kb = col / blk, jj = col - kb * blk;
  const uint16_t* prow = Pt + ((size_t)kb * blk + jj) * blk;
  for (int32_t i0 = 0; i0 < blk; i0 += CH) {
    uint4 pv[CH / 8], xv[R][CH / 8];
#pragma unroll
    for (int q = 0; q < CH / 8; ++q) pv[q] = ldg16(prow + i0 + 8 * q);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int q = 0; q < CH / 8; ++q) xv[r][q] = ldg16(xr[r] + kb * blk + i0 + 8 * q);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int q = 0; q < CH / 8; ++q) acc[r] += dot8(xv[r][q], pv[q]);
  }
  (void)nr;
}

__global__ void __launch_bounds__(256) k_decode_prologue(ProArgs a) {
  const int lane = threadIdx.x & 63;
  if (a.zero_y) {
    float4* y4 = reinterpret_cast<float4*>(a.y);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < a.y_vec4;
         i += (int64_t)gridDim.x * 256)
      y4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int64_t d_in = a.d_in;
  for (int it = blockIdx.x * 4 + (threadIdx.x >> 6); it < a.n_items; it += gridDim.x * 4) {
    const int4 item = a.items[it];
    if (item.x == PRO_ROT) {
      // delta[p][col] = sum_i x[tok p][kb*blk + i] (R - I)[kb][i][col - kb*blk]
      // item: (first sorted row, rows <= 4, first of 64 columns)
      const int32_t p0 = item.y, len = item.z;
      const int64_t col = (int64_t)item.w + lane;
      const SlotEntry E = a.table[a.row_adapter[p0]];
      const int32_t blk = E.blk;
      const uint16_t* Pt = (const uint16_t*)E.P;
      const uint16_t* xr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) xr[r] = a.x + (size_t)a.perm[p0 + min(r, len - 1)] * d_in;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      if (col < d_in) {
        if (blk % 32 == 0) {
          rotate_rows<32, 4>(a, Pt, blk, xr, len, col, acc);
        } else if (blk % 8 == 0) {
          rotate_rows<8, 4>(a, Pt, blk, xr, len, col, acc);
        } else {
          const int64_t kb = col / blk, jj = col - kb * blk;
          const uint16_t* prow = Pt + ((size_t)kb * blk + jj) * blk;
          for (int32_t i = 0; i < blk; ++i) {
            const float pv = bf2f(ldg(prow + i));
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += bf2f(ldg(xr[r] + kb * blk + i)) * pv;
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (r < len) a.delta[(size_t)(p0 + r) * d_in + col] = f2bf(acc[r]);
      }
    } else if (item.x == PRO_SHRINK) {
      // own-term shrink t = x A' for up to 4 rows x 4 ranks over one K part
      // of 1024; the K parts meet through a small partial buffer, the last
      // to arrive sums them in K order and writes tb (bf16).
      // item: (group index, first row | rows << 16, first rank | ranks << 16 ...)
      const int32_t grp = item.y;
      const int4 gd = a.sgroups[grp];  // (first row, rows, first rank, ranks)
      const int32_t p0 = gd.x, len = gd.y, k0 = gd.z, nk = gd.w, kq = item.z;
      const SlotEntry E = a.table[a.row_adapter[p0]];
      const uint16_t* A = (const uint16_t*)E.A;
      const int64_t cbeg = (int64_t)kq * 1024;
      const uint16_t* ar[4];
      const uint16_t* xr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) ar[j] = A + (size_t)(k0 + min(j, nk - 1)) * d_in + cbeg;
#pragma unroll
      for (int r = 0; r < 4; ++r) xr[r] = a.x + (size_t)a.perm[p0 + min(r, len - 1)] * d_in + cbeg;
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
            for (int j = 0; j < 4; ++j) acc[r][j] += dot8(xv[cc][r], av[cc][j]);
      }
      float* part = a.spart + ((size_t)kq * a.n_sgroups + grp) * 16;
      float mine = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = wave_sum(acc[r][j]);
          if (lane == 4 * r + j) mine = v;
        }
      if (lane < 16) st_coh(part + lane, mine);
      wait_vm_all();
      int32_t old = 0;
      if (lane == 0) old = arrive(&a.scnt[grp]);
      old = __shfl(old, 0, 64);
      if (old == a.KQ - 1) {
        if (lane < 16) {
          float tot = 0.f;
          for (int32_t q = 0; q < a.KQ; ++q)
            tot += q == kq ? mine : ld_coh(a.spart + ((size_t)q * a.n_sgroups + grp) * 16 + lane);
          const int r = lane >> 2, j = lane & 3;
          if (r < len && j < nk) a.tb[(size_t)(p0 + r) * a.RT + k0 + j] = f2bf(tot);
        }
        if (lane == 0) reset_counter(&a.scnt[grp]);
      }
    } else {
      // VeRA shrink block: 32 VeRA rows x 32 rows of A_sh over one K slice of
      // 512 (two rounds of loads), partial sums combined by the last of the
      // SV slices to arrive
      const int32_t vb = item.y, jb = item.z, kv = item.w;
      const int m = lane & 31, h = lane >> 5;
      const int32_t vr = 32 * vb + m;
      const int32_t vp = vr < a.n_vera ? a.vera_pos[vr] : a.vera_pos[0];
      const uint16_t* xr = a.x + (size_t)a.perm[vp] * d_in + (int64_t)kv * 512 + 32 * h;
      const uint16_t* ar = a.A_sh + (size_t)(32 * jb + m) * d_in + (int64_t)kv * 512 + 32 * h;
      f32x16 acc = {};
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint4 xa[16], wa[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          xa[q] = ldg16(xr + 256 * half + 64 * (q >> 2) + 8 * (q & 3));
          wa[q] = ldg16(ar + 256 * half + 64 * (q >> 2) + 8 * (q & 3));
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) acc = mfma32(xa[q], wa[q], acc);
      }
      const int32_t blkid = vb * a.njb + jb;
      float* part = a.vpart + ((size_t)kv * a.nvb * a.njb + blkid) * 1024;
#pragma unroll
      for (int i = 0; i < 16; ++i) st_coh(part + 64 * i + lane, acc[i]);
      wait_vm_all();
      int32_t old = 0;
      if (lane == 0) old = arrive(&a.vcnt[blkid]);
      old = __shfl(old, 0, 64);
      if (old == a.SV - 1) {
        float tot[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) tot[i] = 0.f;
#pragma unroll 1
        for (int32_t q = 0; q < a.SV; ++q) {
          if (q == kv) {
#pragma unroll
            for (int i = 0; i < 16; ++i) tot[i] += acc[i];
            continue;
          }
          const float* pq = a.vpart + ((size_t)q * a.nvb * a.njb + blkid) * 1024 + lane;
          float pv[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) pv[i] = ld_coh(pq + 64 * i);
#pragma unroll
          for (int i = 0; i < 16; ++i) tot[i] += pv[i];
        }
        // acc element i: VeRA row 8(i/4) + 4h + i%4, A_sh row 32 jb + m
        const int32_t j = 32 * jb + m;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int32_t row = 32 * vb + 8 * (i >> 2) + 4 * h + (i & 3);
          if (row < a.n_vera) {
            const int32_t p = a.vera_pos[row];
            const float* vd = a.table[a.row_adapter[p]].vd;
            a.ub[(size_t)p * a.r_v + j] = f2bf(tot[i] * ldg(vd + j));
          }
        }
        if (lane == 0) reset_counter(&a.vcnt[blkid]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// main GEMM + epilogue
// ---------------------------------------------------------------------------

struct MainArgs {
  const uint16_t* x;
  const uint16_t* W;
  const uint16_t* delta;     // [32 g_rot][d_in]
  const int32_t* row_tok;    // [M_pad], -1 past n
  const float* const* row_s; // [256] per sorted row: live s, VeRA e, shift b (or null)
  const float* const* row_ve;
  const float* const* row_b;
  const int4* items;         // expand items grouped by K slice
  const uint16_t* const* item_ptr;  // per item: B' of its adapter (own) or B_sh (VeRA)
  const int32_t* item_off;   // [S + 1]
  const uint16_t* tb;        // [M_pad][RT] own-term shrink (bf16)
  const uint16_t* ub;        // [M_pad][r_v] VeRA shrink (bf16), zero rows elsewhere
  const float* ones;         // [d_out] of 1.0 (factor of rows without s or VeRA e)
  float* part;               // split-K partials [S][C][2][mgx][16][64] (S > 1)
  int32_t* cnt;              // [C] arrival counters, kept at zero between forwards
  float* y;
  int32_t n, g_rot, d_in, d_out, k_chunk, S, C, RT, r_v;
};

// Tile of the main kernel: 64 output columns (two 32-column MFMA blocks) by
// one of S slices of K; the 4 waves of a work-group are (column block cb,
// K half kp). The x / delta rows of each K half stream through an LDS ring
// of R stages of 64 k; W streams straight into registers. The S slices of a
// tile meet through a small workspace: the last slice to arrive adds the
// others' partial products in slice order and writes y once.
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
};

// s_waitcnt immediate (gfx9 encoding) waiting until at most `n` vector
// memory operations are outstanding; export and LDS counters unconstrained
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Work-group barrier that orders LDS traffic without waiting for outstanding
// global loads (the LDS-filling loads are awaited explicitly with s_waitcnt
// before it; LDS reads are consumed before it in program order).
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

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

__device__ __forceinline__ void load_w(uint4 (&wr)[4], const uint16_t* wrow, int64_t koff) {
#pragma unroll
  for (int s = 0; s < 4; ++s) wr[s] = ldg16(wrow + koff + 8 * s);
}

// one stage: 4 MFMA k-steps of 16 over every staged row group
template <int MGT>
__device__ __forceinline__ void mma_stage(const uint8_t* stage, const uint4 (&wr)[4],
                                          f32x16 (&acc)[MGT], int m, int h) {
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
template <int MGT, int J>
__device__ __forceinline__ void kstep(int t, int nst, const uint16_t* wrow,
                                      const uint16_t* const (&src)[2 * MGT], uint8_t* cur,
                                      uint8_t* nxt, uint4 (&wc)[4], uint4 (&wn)[4],
                                      f32x16 (&acc)[MGT], int m, int h, int cb, int kp) {
  constexpr int R = DecCfg<MGT>::R;
  const int64_t kn = (int64_t)SK * min(t + R - 1, nst - 1);
  load_w(wn, wrow, kn);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(DecCfg<MGT>::WAIT));
  wg_barrier();
  stage_rows<MGT>(nxt + kp * DecCfg<MGT>::STAGE, src, kn, cb);
  mma_stage<MGT>(cur + kp * DecCfg<MGT>::STAGE, wc, acc, m, h);
}

// MGT = staged row groups = ceil(n / 32) x groups + g_rot delta groups
template <int MGT>
__global__ void __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_decode_main(MainArgs a) {
  using Cfg = DecCfg<MGT>;
  constexpr int R = Cfg::R;
  // ring slots as separate LDS objects so the compiler can tell the slot
  // being read from the ones the direct loads fill
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[2 * Cfg::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[2 * Cfg::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t slot2[R == 3 ? 2 * Cfg::STAGE : 16];
  // per sorted row: pointers to live s, VeRA e and b (null if none)
  __shared__ __attribute__((aligned(1024))) const float* lrow[3][256];
  __shared__ int32_t last_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 31, h = lane >> 5;
  const int cb = wave & 1, kp = wave >> 1;
  const int mgx = MGT - a.g_rot;  // x row groups

  // XCD-aware tile order: work-groups are dispatched round-robin over the 8
  // XCDs, so consecutive work indices (the S slices of one tile) are placed
  // on one XCD, where the combine finds their partials in one L2
  const int G = gridDim.x, bid = blockIdx.x;
  const int w = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int c = w / a.S, kc = w - c * a.S;

  const int64_t ncol = (int64_t)c * 64 + cb * 32 + m;
  const int kw = a.k_chunk / 2;  // K per half
  const int64_t kbase = (int64_t)kc * a.k_chunk + (int64_t)kp * kw;
  const int nst = kw / SK;
  const uint16_t* wrow = a.W + (size_t)ncol * a.d_in + kbase + 32 * h;

  // (1) token of each staged row this lane fills (rows 8 (cb + 2q) + lane/8)
  int32_t tok[2 * MGT];
#pragma unroll
  for (int q = 0; q < 2 * MGT; ++q) {
    const int r = 8 * (cb + 2 * q) + (lane >> 3);
    tok[q] = r < 32 * mgx ? ldg(a.row_tok + r) : 0;
  }
  // (2) W of the first R-1 stages (in flight while the tokens arrive)
  uint4 w0[4], w1[4], w2[4];
  load_w(w0, wrow, 0);
  if constexpr (R == 3) load_w(w1, wrow, (int64_t)SK * min(1, nst - 1));
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * (R - 1)));
  // (3) row sources; rows past n read token 0 (finite, never written out)
  const uint16_t* src[2 * MGT];
  {
    const int piece = (lane & 7) ^ ((4 * cb + (lane >> 4)) & 7);
#pragma unroll
    for (int q = 0; q < 2 * MGT; ++q) {
      const int r = 8 * (cb + 2 * q) + (lane >> 3);
      const uint16_t* base =
          r < 32 * mgx ? a.x + (size_t)(tok[q] < 0 ? 0 : tok[q]) * a.d_in
                       : a.delta + (size_t)(r - 32 * mgx) * a.d_in;
      src[q] = base + kbase + 8 * piece;
    }
  }
  stage_rows<MGT>(slot0 + kp * Cfg::STAGE, src, 0, cb);
  if constexpr (R == 3) stage_rows<MGT>(slot1 + kp * Cfg::STAGE, src, (int64_t)SK * min(1, nst - 1), cb);
  // (4) row tables: 3 x 256 pointers = 6 KB; every wave issues two 1 KB loads
  //     (instructions 6 and 7 repeat 4 and 5)
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int j0 = wave + 4 * jj;
    const int j = j0 < 6 ? j0 : j0 - 2;
    const float* const* tab = j < 2 ? a.row_s : (j < 4 ? a.row_ve : a.row_b);
    __builtin_amdgcn_global_load_lds((const void*)(tab + 128 * (j & 1) + 2 * lane),
                                     (lds_void*)(&lrow[j >> 1][128 * (j & 1)]), 16, 0, 0);
  }

  f32x16 acc[MGT];
#pragma unroll
  for (int g = 0; g < MGT; ++g) acc[g] = f32x16{};
  float fv[MGT][16];
  uint32_t ms[MGT], mv[MGT];

  // stage 0 (peeled: after its barrier the row tables are in LDS and the
  // per-row factors are prefetched for the epilogue)
  {
    const int64_t kn = (int64_t)SK * min(R - 1, nst - 1);
    if constexpr (R == 3) load_w(w2, wrow, kn); else load_w(w1, wrow, kn);
    // issued after the rows of stage 0: (R == 3: rows of stage 1), the two
    // row-table loads, and W of stage R-1
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(R == 3 ? 2 * MGT + 6 : Cfg::WAIT));
    wg_barrier();
    stage_rows<MGT>((R == 3 ? slot2 : slot1) + kp * Cfg::STAGE, src, kn, cb);
#pragma unroll
    for (int g = 0; g < MGT; ++g) {
      ms[g] = mv[g] = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int p = 32 * g + 8 * (i >> 2) + 4 * h + (i & 3);
        const bool live = g < mgx && kp == 0;
        const float* sp = live ? lrow[0][p] : nullptr;
        const float* vp = live ? lrow[1][p] : nullptr;
        const float* fp = (live && sp) ? sp : ((live && vp) ? vp : a.ones);
        fv[g][i] = ldg(fp + ncol);
        if (live && sp) ms[g] |= 1u << i;
        if (live && vp) mv[g] |= 1u << i;
      }
    }
    mma_stage<MGT>(slot0 + kp * Cfg::STAGE, w0, acc, m, h);
  }
  // remaining stages, unrolled by the ring depth so slots and W registers are
  // named statically
  if constexpr (R == 3) {
#pragma unroll 1
    for (int t = 1; t < nst; t += 3) {
      kstep<MGT, 1>(t, nst, wrow, src, slot1, slot0, w1, w0, acc, m, h, cb, kp);
      if (t + 1 >= nst) break;
      kstep<MGT, 2>(t + 1, nst, wrow, src, slot2, slot1, w2, w1, acc, m, h, cb, kp);
      if (t + 2 >= nst) break;
      kstep<MGT, 0>(t + 2, nst, wrow, src, slot0, slot2, w0, w2, acc, m, h, cb, kp);
    }
  } else {
#pragma unroll 1
    for (int t = 1; t < nst; t += 2) {
      kstep<MGT, 1>(t, nst, wrow, src, slot1, slot0, w1, w0, acc, m, h, cb, kp);
      if (t + 1 >= nst) break;
      kstep<MGT, 0>(t + 1, nst, wrow, src, slot0, slot1, w0, w1, acc, m, h, cb, kp);
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // clamped tail prefetches
  wg_barrier();

  // ---- K halves meet: half 1 hands its product to half 0 through LDS -------
  float* red = reinterpret_cast<float*>(slot0);  // [cb][g][16][64]
  if (kp == 1) {
#pragma unroll
    for (int g = 0; g < MGT; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[((cb * MGT + g) * 16 + i) * 64 + lane] = acc[g][i];
  }
  wg_barrier();
  if (kp == 0) {
#pragma unroll
    for (int g = 0; g < MGT; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[g][i] += red[((cb * MGT + g) * 16 + i) * 64 + lane];
  }

  if (kp == 0) {
    // rotated rows: group mgx + g holds delta W of x group g; fold it in
#pragma unroll
    for (int j = 1; j < MGT; ++j)
#pragma unroll
      for (int g = 0; g < j; ++g)
        if (j - g == mgx && g < a.g_rot) acc[g] += acc[j];

    // ---- epilogue ----------------------------------------------------------
    // accumulator element i of group g: row 32 g + 8 (i / 4) + 4 h + i % 4,
    // column ncol; this lane's A-operand row in group g is 32 g + m
    // (a) s of each row's adapter multiplies this slice's base product
#pragma unroll
    for (int g = 0; g < MGT; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (ms[g] & (1u << i)) acc[g][i] *= fv[g][i];

    // (b) expand items of this K slice (<= 4 MFMA steps each), four at a time
    const int it0 = a.item_off[kc], it1 = a.item_off[kc + 1];
#pragma unroll 1
    for (int ib = it0; ib < it1; ib += 4) {
      uint4 av[4][4], bv[4][4];
      int4 itm[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int it = min(ib + q, it1 - 1);
        itm[q] = a.items[it];
        const uint16_t* bp = a.item_ptr[it];
        const int type = itm[q].x & 0xFF, gi = itm[q].x >> 8;
        const int pa = 32 * gi + m;
        const int nstp = itm[q].z & 0xFF;  // 16-rank steps
        const int rank = itm[q].z >> 8;    // own: B' row length; VeRA: r_v
        const int lo = itm[q].w & 0xFFFF, hi = itm[q].w >> 16;
        const bool rowok = (ib + q < it1) && pa >= lo && pa < hi;
        const uint16_t* arow =
            type == EXP_OWN ? a.tb + (size_t)pa * a.RT : a.ub + (size_t)pa * a.r_v;
        const uint16_t* brow = bp + (size_t)ncol * rank;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int kk = itm[q].y + 16 * st + 8 * h;
          const bool ok = st < nstp && kk < rank;
          bv[q][st] = ok ? ldg16(brow + kk) : make_uint4(0, 0, 0, 0);
          av[q][st] = (ok && rowok) ? ldg16(arow + kk) : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (ib + q >= it1) break;
        const int type = itm[q].x & 0xFF, gi = itm[q].x >> 8;
        f32x16 t2 = {};
#pragma unroll
        for (int st = 0; st < 4; ++st) t2 = mfma32(av[q][st], bv[q][st], t2);
#pragma unroll
        for (int g = 0; g < MGT; ++g) {
          if (g != gi) continue;
          if (type == EXP_OWN) {
            acc[g] += t2;  // the own low-rank update is not scaled by s
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              if (!(mv[g] & (1u << i))) continue;
              float e = fv[g][i];
              if (ms[g] & (1u << i)) {  // row with both s and a VeRA term
                const int p = 32 * g + 8 * (i >> 2) + 4 * h + (i & 3);
                e = ldg(lrow[1][p] + ncol);
              }
              acc[g][i] += e * t2[i];
            }
          }
        }
      }
    }
  }

  // ---- S slices of the tile meet ---------------------------------------------
  bool writer = true;
  if (a.S > 1) {
    // partial of this slice -> workspace [slice][tile][cb][g][16][lane]
    // through memory, wait for the stores, count arrivals; the last slice to
    // arrive adds all slices in slice order (deterministic) and writes y
    const size_t stride = (size_t)mgx * 16 * 64;
    if (kp == 0) {
      float* mine = a.part + (((size_t)kc * a.C + c) * 2 + cb) * stride + lane;
#pragma unroll
      for (int g = 0; g < MGT; ++g) {
        if (g >= mgx) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) st_coh(mine + g * 1024 + 64 * i, acc[g][i]);
      }
    }
    wait_vm_all();
    wg_barrier();
    if (tid == 0) {
      const int old = arrive(a.cnt + c);
      last_flag = old == a.S - 1;
      if (old == a.S - 1) reset_counter(a.cnt + c);
    }
    wg_barrier();
    writer = last_flag != 0;
    if (writer) {
      if (kp == 0) {
        float tot[MGT][16];
#pragma unroll
        for (int g = 0; g < MGT; ++g)
#pragma unroll
          for (int i = 0; i < 16; ++i) tot[g][i] = 0.f;
#pragma unroll 1
        for (int q = 0; q < a.S; ++q) {
          if (q == kc) {
#pragma unroll
            for (int g = 0; g < MGT; ++g)
#pragma unroll
              for (int i = 0; i < 16; ++i) tot[g][i] += acc[g][i];
          } else {
            const float* pq = a.part + (((size_t)q * a.C + c) * 2 + cb) * stride + lane;
#pragma unroll
            for (int g = 0; g < MGT; ++g) {
              if (g >= mgx) continue;
#pragma unroll
              for (int i = 0; i < 16; ++i) tot[g][i] += ld_coh(pq + g * 1024 + 64 * i);
            }
          }
        }
#pragma unroll
        for (int g = 0; g < MGT; ++g)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[g][i] = tot[g][i];
      }
    }
  }

  // ---- shift b and y ---------------------------------------------------------
  if (writer && kp == 0) {
#pragma unroll
    for (int g = 0; g < MGT; ++g) {
      if (g >= mgx) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int p = 32 * g + 8 * (i >> 2) + 4 * h + (i & 3);
        if (p >= a.n) continue;
        float v = acc[g][i];
        const float* bp = lrow[2][p];
        if (bp) v += ldg(bp + ncol);
        a.y[(size_t)a.row_tok[p] * a.d_out + ncol] = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------

template <int MGT>
static void launch_main(const MainArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL(k_decode_main<MGT>, dim3(grid), dim3(256), 0, st, a);
}

scute_status launch_decode(scute_layer* L, const scute_batch* B, const void* x, const void* W,
                           float* y, hipStream_t st, int32_t* launches) {
  const DecodePlan& D = B->dp;
  ProArgs pa{};
  pa.x = (const uint16_t*)x;
  pa.perm = B->d_perm;
  pa.row_adapter = B->d_row_adapter;
  pa.vera_pos = B->d_vera_pos;
  pa.table = L->table_dev;
  pa.A_sh = (const uint16_t*)L->A_sh;
  pa.y = y;
  pa.y_vec4 = (int64_t)B->n * L->d_out / 4;
  pa.zero_y = 0;
  pa.items = D.pro_items;
  pa.n_items = D.n_pro;
  pa.tb = D.tb;
  pa.RT = D.RT;
  pa.ub = D.ub;
  pa.r_v = L->r_v;
  pa.delta = D.delta;
  pa.vpart = D.vpart;
  pa.vcnt = D.vcnt;
  pa.nvb = D.nvb;
  pa.njb = D.njb;
  pa.SV = D.SV;
  pa.n_vera = B->n_vera;
  pa.sgroups = D.sgroups;
  pa.spart = D.spart;
  pa.scnt = D.scnt;
  pa.n_sgroups = D.n_sgroups;
  pa.KQ = D.KQ;
  pa.d_in = (int32_t)L->d_in;
  int nl = 0;
  if (pa.zero_y || pa.n_items > 0) {
    int grid = std::max(1, std::min(2048, (pa.n_items + 3) / 4));
    if (pa.zero_y) grid = std::max(grid, 256);
    ProfScope ps(L, st, "decode_prologue");
    hipLaunchKernelGGL(k_decode_prologue, dim3(grid), dim3(256), 0, st, pa);
    ++nl;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "launch k_decode_prologue");
  }
  MainArgs ma{};
  ma.x = (const uint16_t*)x;
  ma.W = (const uint16_t*)W;
  ma.delta = D.delta;
  ma.row_tok = D.row_tok;
  ma.row_s = D.row_s;
  ma.row_b = D.row_b;
  ma.row_ve = D.row_ve;
  ma.items = D.exp_items;
  ma.item_ptr = D.exp_ptr;
  ma.item_off = D.exp_off;
  ma.tb = D.tb;
  ma.ub = D.ub;
  ma.ones = D.ones;
  ma.part = D.part;
  ma.cnt = D.cnt;
  ma.C = D.C;
  ma.y = y;
  ma.n = B->n;
  ma.g_rot = D.g_rot;
  ma.d_in = (int32_t)L->d_in;
  ma.d_out = (int32_t)L->d_out;
  ma.k_chunk = D.k_chunk;
  ma.S = D.S;
  ma.RT = D.RT;
  ma.r_v = L->r_v;
  const int grid = D.C * D.S;
  ProfScope ps(L, st, "decode_main");
  switch (D.MG + D.g_rot) {
    case 1: launch_main<1>(ma, grid, st); break;
    case 3: launch_main<3>(ma, grid, st); break;
    case 4: launch_main<4>(ma, grid, st); break;
    case 5: launch_main<5>(ma, grid, st); break;
    case 6: launch_main<6>(ma, grid, st); break;
    case 7: launch_main<7>(ma, grid, st); break;
    case 8: launch_main<8>(ma, grid, st); break;
    case 9: launch_main<9>(ma, grid, st); break;
    default: return fail(SCUTE_E_UNSUPPORTED, "decode path: too many staged row groups");
  }
  ++nl;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch k_decode_main");
  if (launches) *launches = nl;
  return SCUTE_OK;
}

}  // namespace scute
