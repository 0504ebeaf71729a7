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
__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg16_stream(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
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
  int32_t nvb, njb, SV, KV, n_vera;
  int32_t d_in;
};

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
      // delta[p][col] = sum_i x[tok p][kb*blk + i] P[kb][i][col - kb*blk]
      const int32_t p0 = item.y, len = item.z, c0 = item.w;
      const SlotEntry E = a.table[a.row_adapter[p0]];
      const int32_t blk = E.blk;
      const uint16_t* P = (const uint16_t*)E.P;
      for (int32_t r0 = 0; r0 < len; r0 += 4) {
        const int32_t nr = min(4, len - r0);
        const uint16_t* xr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          xr[r] = a.x + (size_t)a.perm[p0 + r0 + min(r, nr - 1)] * d_in;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t col = (int64_t)c0 + lane + 64 * j;
          if (col >= d_in) continue;
          const int64_t kb = col / blk, jj = col - kb * blk;
          const uint16_t* Pc = P + (size_t)kb * blk * blk + jj;
          float acc[4] = {0.f, 0.f, 0.f, 0.f};
          for (int32_t i = 0; i < blk; ++i) {
            const float pv = bf2f(Pc[(size_t)i * blk]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += bf2f(xr[r][kb * blk + i]) * pv;
          }
          for (int r = 0; r < nr; ++r) a.delta[(size_t)(p0 + r0 + r) * d_in + col] = f2bf(acc[r]);
        }
      }
    } else if (item.x == PRO_SHRINK) {
      // tb[p][k] = x[tok p] . A'[k]
      const int32_t p0 = item.y, len = item.z, k = item.w;
      const SlotEntry E = a.table[a.row_adapter[p0]];
      const uint16_t* Ak = (const uint16_t*)E.A + (size_t)k * d_in;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const uint16_t* xr[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) xr[r] = a.x + (size_t)a.perm[p0 + min(r, len - 1)] * d_in;
      for (int64_t c = (int64_t)lane * 8; c < d_in; c += 512) {
        const uint4 av = ldg16(Ak + c);
#pragma unroll
        for (int r = 0; r < 8; ++r)
          if (r < len) acc[r] += dot8(ldg16(xr[r] + c), av);
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        if (r >= len) break;
        const float s = wave_sum(acc[r]);
        if (lane == 0) a.tb[(size_t)(p0 + r) * a.RT + k] = f2bf(s);
      }
    } else {
      // VeRA shrink block: 32 VeRA rows x 32 rows of A_sh over one K slice,
      // partial sums combined by the last of the SV slices to arrive
      const int32_t vb = item.y, jb = item.z, kv = item.w;
      const int m = lane & 31, h = lane >> 5;
      const int32_t vr = 32 * vb + m;
      const int32_t vp = vr < a.n_vera ? a.vera_pos[vr] : a.vera_pos[0];
      const uint16_t* xr = a.x + (size_t)a.perm[vp] * d_in;
      const uint16_t* ar = a.A_sh + (size_t)(32 * jb + m) * d_in;
      f32x16 acc = {};
      const int64_t kbeg = (int64_t)kv * a.KV;
      for (int64_t k0 = kbeg; k0 < kbeg + a.KV; k0 += 64) {
        const int64_t ko = k0 + 32 * h;
        uint4 xa[4], wa[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          xa[s] = ldg16(xr + ko + 8 * s);
          wa[s] = ldg16(ar + ko + 8 * s);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma32(xa[s], wa[s], acc);
      }
      const int32_t blkid = vb * a.njb + jb;
      float* part = a.vpart + ((size_t)kv * a.nvb * a.njb + blkid) * 1024;
#pragma unroll
      for (int i = 0; i < 16; ++i) part[i * 64 + lane] = acc[i];
      __threadfence();
      int32_t old = 0;
      if (lane == 0) old = atomicAdd(&a.vcnt[blkid], 1);
      old = __shfl(old, 0, 64);
      if (old == a.SV - 1) {
        __threadfence();
        float tot[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) tot[i] = 0.f;
        for (int32_t q = 0; q < a.SV; ++q) {
          const float* pq = a.vpart + ((size_t)q * a.nvb * a.njb + blkid) * 1024;
#pragma unroll
          for (int i = 0; i < 16; ++i) tot[i] += __builtin_nontemporal_load(pq + i * 64 + lane);
        }
        // acc element i: VeRA row 8(i/4) + 4h + i%4, A_sh row 32 jb + m
        const int32_t j = 32 * jb + m;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int32_t row = 32 * vb + 8 * (i >> 2) + 4 * h + (i & 3);
          if (row < a.n_vera) {
            const int32_t p = a.vera_pos[row];
            const float* vd = a.table[a.row_adapter[p]].vd;
            a.ub[(size_t)p * a.r_v + j] = f2bf(tot[i] * vd[j]);
          }
        }
        if (lane == 0) atomicExch(&a.vcnt[blkid], 0);
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
  const float* const* row_s;
  const float* const* row_b;
  const float* const* row_ve;
  const SlotEntry* table;
  const int4* items;
  const int32_t* item_off;   // [S + 1]
  const uint16_t* tb;
  const uint16_t* ub;
  const uint16_t* B_sh;      // [d_out][r_v]
  float* y;
  int32_t n, g_rot, d_in, d_out, k_chunk, S, RT, r_v;
};

constexpr int KBLK = 128;     // K per block
constexpr int ROW_BYTES = 2 * KBLK;

// s_waitcnt immediate (gfx9 encoding) waiting until at most `n` vector
// memory operations are outstanding; export and LDS counters unconstrained
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Work-group barrier that orders LDS traffic without waiting for the
// outstanding W prefetch (the LDS-filling loads are awaited explicitly with
// s_waitcnt before it; LDS reads are consumed before it in program order).
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Staged A-operand rows: MGT groups of 32 rows (x rows of the sorted batch,
// then rows of delta for the rotated groups), ROW_BYTES per row, the 16-byte
// chunk index XOR-swizzled by (row & 15). Each wave fills 4 rows per 1 KB
// direct-to-LDS load (lane i -> row i / 16, slot i % 16); wave w fills rows
// 4w + 16 q + [0, 4) for q < 2 MGT.
template <int MGT>
__device__ __forceinline__ void stage_rows(uint8_t* buf, const uint16_t* const (&src)[2 * MGT],
                                           int64_t k0) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < 2 * MGT; ++q)
    __builtin_amdgcn_global_load_lds((const void*)(src[q] + k0),
                                     (lds_void*)(buf + (4 * wave + 16 * q) * ROW_BYTES), 16, 0, 0);
}

template <int MGT>
__device__ __forceinline__ void mma_block(const uint8_t* cur, const uint4 (&wr)[8],
                                          f32x16 (&acc)[MGT], int m, int h) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int chunk = 8 * half + 4 * h + s;  // 16-byte chunk of the 256-byte row
      uint4 av[MGT];
#pragma unroll
      for (int g = 0; g < MGT; ++g) {
        const int r = 32 * g + m;
        av[g] = *reinterpret_cast<const uint4*>(cur + r * ROW_BYTES + 16 * (chunk ^ (r & 15)));
      }
#pragma unroll
      for (int g = 0; g < MGT; ++g) acc[g] = mfma32(av[g], wr[4 * half + s], acc[g]);
    }
  }
}

__device__ __forceinline__ void load_w(uint4 (&wr)[8], const uint16_t* wrow, int64_t k0) {
#pragma unroll
  for (int s = 0; s < 8; ++s) wr[s] = ldg16_stream(wrow + k0 + 64 * (s >> 2) + 8 * (s & 3));
}

// MGT = staged row groups = ceil(n / 32) x groups + g_rot delta groups
template <int MGT>
__global__ void __launch_bounds__(256, 1) k_decode_main(MainArgs a) {
  // two separate LDS objects so the compiler can tell the buffer being read
  // from the one the direct loads fill
  __shared__ __attribute__((aligned(1024))) uint8_t lbuf0[32 * MGT * ROW_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t lbuf1[32 * MGT * ROW_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 31, h = lane >> 5;
  const int mgx = MGT - a.g_rot;  // x row groups

  // XCD-aware tile order: work-groups are dispatched round-robin over the 8
  // XCDs, so consecutive work indices (the S slices of one column tile) are
  // placed on one XCD, where their atomics meet in one L2
  const int G = gridDim.x, bid = blockIdx.x;
  const int w = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int c = w / a.S, kc = w - c * a.S;

  uint8_t* buf0 = lbuf0;
  uint8_t* buf1 = lbuf1;

  const int64_t ncol = (int64_t)c * 128 + wave * 32 + m;
  const uint16_t* wrow = a.W + (size_t)ncol * a.d_in + 32 * h;
  const int64_t kbeg = (int64_t)kc * a.k_chunk;
  const int nblk = a.k_chunk / KBLK;

  // per-lane source rows of the staging loads; rows past n read token 0's
  // row (finite values in rows that are never written out)
  const uint16_t* src[2 * MGT];
  {
    const int rl = 4 * wave + (lane >> 4);
    const int chunk = (lane & 15) ^ (rl & 15);
#pragma unroll
    for (int q = 0; q < 2 * MGT; ++q) {
      const int r = rl + 16 * q;
      const uint16_t* base;
      if (r < 32 * mgx) {
        const int32_t tok = a.row_tok[r];
        base = a.x + (size_t)(tok < 0 ? 0 : tok) * a.d_in;
      } else {
        base = a.delta + (size_t)(r - 32 * mgx) * a.d_in;
      }
      src[q] = base + 8 * chunk;
    }
  }

  f32x16 acc[MGT];
#pragma unroll
  for (int g = 0; g < MGT; ++g) acc[g] = f32x16{};

  // Pipeline: W for block b+1 streams into registers and the rows for block
  // b+1 stream into the other LDS buffer while block b is multiplied. Issue
  // order per block: W(b+1), barrier, rows(b+1); waiting until only the 8 W
  // loads of block b+1 are outstanding guarantees rows(b) and W(b) landed.
  // The K slice has an even number of blocks; the loop body handles two, so
  // the W ping-pong registers and LDS buffers alternate without copies. The
  // last prefetch re-reads the final block (harmless, keeps the body
  // branch-free) and is drained before the epilogue.
  uint4 wa[8], wb[8];
  load_w(wa, wrow, kbeg);
  stage_rows<MGT>(buf0, src, kbeg);
  const int npair = nblk / 2;
  for (int bp = 0; bp < npair; ++bp) {
    const int64_t k1 = kbeg + (int64_t)(2 * bp + 1) * KBLK;
    const int64_t k2 = kbeg + (int64_t)min(2 * bp + 2, nblk - 1) * KBLK;
    load_w(wb, wrow, k1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
    wg_barrier();
    stage_rows<MGT>(buf1, src, k1);
    mma_block<MGT>(buf0, wa, acc, m, h);
    load_w(wa, wrow, k2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
    wg_barrier();
    stage_rows<MGT>(buf0, src, k2);
    mma_block<MGT>(buf1, wb, acc, m, h);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // rotated rows: group mgx + g holds delta W of x group g; fold it in
#pragma unroll
  for (int j = 1; j < MGT; ++j) {
#pragma unroll
    for (int g = 0; g < j; ++g)
      if (j - g == mgx && g < a.g_rot) acc[g] += acc[j];
  }

  // ---- epilogue --------------------------------------------------------------
  // accumulator element i of group g: row 32 g + 8 (i / 4) + 4 h + i % 4,
  // column ncol
  // (1) s of each row's adapter multiplies the base product (this slice's part)
#pragma unroll
  for (int g = 0; g < MGT; ++g) {
    if (g >= mgx) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int p = 32 * g + 8 * (i >> 2) + 4 * h + (i & 3);
      const float* sp = a.row_s[p];
      if (sp) acc[g][i] *= sp[ncol];
    }
  }
  // (2) expand items of this K slice: own low-rank terms and VeRA terms
  for (int it = a.item_off[kc]; it < a.item_off[kc + 1]; ++it) {
    const int4 item = a.items[it];
    const int type = item.x & 0xFF, gi = item.x >> 8;
    const int lo = item.w & 0xFFFF, hi = item.w >> 16;
    const int pa = 32 * gi + m;  // A-operand row of this lane
    if (type == EXP_OWN) {
      const SlotEntry& E = a.table[item.y];
      const int rank = E.rank;
      const int kk = item.z + 8 * h;
      uint4 av = make_uint4(0, 0, 0, 0), bv = make_uint4(0, 0, 0, 0);
      if (kk < rank) {
        bv = ldg16((const uint16_t*)E.B + (size_t)ncol * rank + kk);
        if (pa >= lo && pa < hi) av = ldg16(a.tb + (size_t)pa * a.RT + kk);
      }
#pragma unroll
      for (int g = 0; g < MGT; ++g)
        if (g == gi) acc[g] = mfma32(av, bv, acc[g]);
    } else {
      const bool vrow = a.row_ve[pa] != nullptr;
      f32x16 t2 = {};
      for (int k0 = 0; k0 < a.r_v; k0 += 16) {
        const int kk = k0 + 8 * h;
        const uint4 bv = ldg16(a.B_sh + (size_t)ncol * a.r_v + kk);
        const uint4 av = vrow ? ldg16(a.ub + (size_t)pa * a.r_v + kk) : make_uint4(0, 0, 0, 0);
        t2 = mfma32(av, bv, t2);
      }
#pragma unroll
      for (int g = 0; g < MGT; ++g) {
        if (g != gi) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int p = 32 * g + 8 * (i >> 2) + 4 * h + (i & 3);
          const float* ve = a.row_ve[p];
          if (ve) acc[g][i] += ve[ncol] * t2[i];
        }
      }
    }
  }
  // (3) shift b (once: slice 0) and write out
#pragma unroll
  for (int g = 0; g < MGT; ++g) {
    if (g >= mgx) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int p = 32 * g + 8 * (i >> 2) + 4 * h + (i & 3);
      if (p >= a.n) continue;
      float v = acc[g][i];
      if (kc == 0) {
        const float* bp = a.row_b[p];
        if (bp) v += bp[ncol];
      }
      float* dst = a.y + (size_t)a.row_tok[p] * a.d_out + ncol;
      if (a.S > 1)
        unsafeAtomicAdd(dst, v);
      else
        *dst = v;
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
  pa.zero_y = D.S > 1;
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
  pa.KV = D.KV;
  pa.n_vera = B->n_vera;
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
  ma.table = L->table_dev;
  ma.items = D.exp_items;
  ma.item_off = D.exp_off;
  ma.tb = D.tb;
  ma.ub = D.ub;
  ma.B_sh = (const uint16_t*)L->B_sh;
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
    case 2: launch_main<2>(ma, grid, st); break;
    case 3: launch_main<3>(ma, grid, st); break;
    case 4: launch_main<4>(ma, grid, st); break;
    case 5: launch_main<5>(ma, grid, st); break;
    case 6: launch_main<6>(ma, grid, st); break;
    case 7: launch_main<7>(ma, grid, st); break;
    case 8: launch_main<8>(ma, grid, st); break;
    case 9: launch_main<9>(ma, grid, st); break;
    case 10: launch_main<10>(ma, grid, st); break;
    default: return fail(SCUTE_E_UNSUPPORTED, "decode path: too many staged row groups");
  }
  ++nl;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch k_decode_main");
  if (launches) *launches = nl;
  return SCUTE_OK;
}

}  // namespace scute
