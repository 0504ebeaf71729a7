// The forward pass: OFT rotation, shrink, base GEMM with the s / b
// epilogue, expand and the shared VeRA term.
//
// Order of steps ("How does Scute plug into vLLM?" and "Where is the
// cheapest place to compute the remaining slots?", paper-daily.com explainer
// of "Scute: Exact Batched Serving for PEFT Adapters Beyond LoRA"): rows
// are rotated first, and the rotated rows then share the GEMM; the base GEMM runs
// once for the whole batch; the own low-rank term is shrunk and expanded per
// adapter; s multiplies the base output and the low-rank update is added
// unscaled; the shared VeRA term is computed for every VeRA row of the batch
// with the shared pair read once per step.
//
// Rotation: x R = x + x (R - I). The library stores P = R - I and computes
// delta = x P in fp32, rounded once to the activation dtype, then feeds both
// x and delta through the same W. Rounding only the small delta keeps the
// rotation's effect accurate in bf16, where rounding x R itself would not.
//
// This file holds the generic kernels: correct for every shape the ABI
// accepts, in fp32 or bf16, with fp32 accumulation.

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "internal.h"

namespace scute {

__device__ __forceinline__ float ldf(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ldf(const uint16_t* p, size_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}
__device__ __forceinline__ void stf(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void stf(uint16_t* p, size_t i, float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even (finite inputs)
  p[i] = (uint16_t)(u >> 16);
}

// Row p's x row: perm[p] in a planned batch, p itself when the batch is
// taken in token order (perm null).
__device__ __forceinline__ int32_t src_row(const int32_t* perm, int32_t p) { return perm ? perm[p] : p; }
// Row p's adapter: its id, -1 (base path only), or -2 for an id that is out
// of range or not loaded (ids of a planned batch are checked on the host, so
// only a batch taken in token order from device memory can hold one).
__device__ __forceinline__ int32_t row_id(const int32_t* ra, int32_t p, const SlotEntry* table, int32_t na) {
  const int32_t a = ra[p];
  if (a == -1) return -1;
  if (a < 0 || a >= na || !(table[a].flags & F_LOADED)) return -2;
  return a;
}

// ---------------------------------------------------------------------------
// rotation: delta[z][p][col] = sum_i x[perm[p]][kb*blk + i] * P_z[kb][i][col - kb*blk],
// P stored transposed per block; rows without a rotation get zero. z is the
// projection (grid z): an adapter that rotates per projection (F_RPROJ)
// keeps P_z after P_0, one with a single rotation uses it for every z
// grid (ceil(d_in / 256), rows, projections)
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) k_rotate_ref(const T* __restrict__ x,
                                                    const int32_t* __restrict__ perm,
                                                    const int32_t* __restrict__ row_adapter,
                                                    const SlotEntry* __restrict__ table, int32_t na,
                                                    int64_t d_in, int32_t n_rot, T* __restrict__ delta) {
  const int32_t p = blockIdx.y, z = blockIdx.z;
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (col >= d_in) return;
  const size_t o = ((size_t)z * n_rot + p) * d_in + col;
  const int32_t a = row_id(row_adapter, p, table, na);
  if (a < 0 || !(table[a].flags & F_R)) {
    stf(delta, o, 0.f);
    return;
  }
  const SlotEntry E = table[a];
  const int32_t blk = E.blk;
  const int64_t kb = col / blk, jj = col - kb * blk;
  const T* xr = x + (size_t)src_row(perm, p) * d_in + kb * blk;
  const T* Pz = (const T*)E.P + ((E.flags & F_RPROJ) ? (size_t)z * d_in * blk : 0);
  const T* Pt = Pz + ((size_t)kb * blk + jj) * blk;  // (R - I)^T row jj
  float acc = 0.f;
  for (int32_t i = 0; i < blk; ++i) acc += ldf(xr, i) * ldf(Pt, i);
  stf(delta, o, acc);
}

__device__ __forceinline__ float block_sum_256(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  if (threadIdx.x == 0) s = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return s;
}

// ---------------------------------------------------------------------------
// own-term shrink: t[p][k] = x[perm[p]] . A'[k]   (0 for k >= rank)
// grid (max_rank, n), 256 threads reduce over d_in
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) k_shrink_ref(const T* __restrict__ x,
                                                    const int32_t* __restrict__ perm,
                                                    const int32_t* __restrict__ row_adapter,
                                                    const SlotEntry* __restrict__ table, int32_t na,
                                                    int64_t d_in, int32_t max_rank,
                                                    float* __restrict__ t) {
  __shared__ float red[4];
  const int32_t p = blockIdx.y, k = blockIdx.x;
  const int32_t a = row_id(row_adapter, p, table, na);
  bool live = false;
  SlotEntry E{};
  if (a >= 0) {
    E = table[a];
    live = (E.flags & F_TERM) && k < E.rank;
  }
  if (!live) {
    if (threadIdx.x == 0) t[(size_t)p * max_rank + k] = 0.f;
    return;
  }
  const T* xr = x + (size_t)src_row(perm, p) * d_in;
  const T* Ar = (const T*)E.A + (size_t)k * d_in;
  float acc = 0.f;
  for (int64_t i = threadIdx.x; i < d_in; i += 256) acc += ldf(xr, i) * ldf(Ar, i);
  acc = block_sum_256(acc, red);
  if (threadIdx.x == 0) t[(size_t)p * max_rank + k] = acc;
}

// ---------------------------------------------------------------------------
// VeRA shrink over the whole batch: u[p][k] = d_a[k] * (x[perm[p]] . A_sh[k])
// for every VeRA row p = vera_pos[v]; grid (r_v, n_vera); with vera_pos
// null, grid (r_v, rows) and rows without a VeRA term are skipped
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) k_vera_shrink_ref(const T* __restrict__ x,
                                                         const int32_t* __restrict__ perm,
                                                         const int32_t* __restrict__ row_adapter,
                                                         const int32_t* __restrict__ vera_pos,
                                                         const SlotEntry* __restrict__ table, int32_t na,
                                                         const T* __restrict__ A_sh, int64_t d_in,
                                                         int32_t r_v, float* __restrict__ u) {
  __shared__ float red[4];
  const int32_t k = blockIdx.x;
  const int32_t p = vera_pos ? vera_pos[blockIdx.y] : (int32_t)blockIdx.y;
  const int32_t a = row_id(row_adapter, p, table, na);
  if (a < 0 || !(table[a].flags & F_VERA)) return;  // uniform over the block
  const SlotEntry E = table[a];
  const T* xr = x + (size_t)src_row(perm, p) * d_in;
  const T* Ar = A_sh + (size_t)k * d_in;
  float acc = 0.f;
  for (int64_t i = threadIdx.x; i < d_in; i += 256) acc += ldf(xr, i) * ldf(Ar, i);
  acc = block_sum_256(acc, red);
  if (threadIdx.x == 0) u[(size_t)p * r_v + k] = acc * E.vd[k];
}

// ---------------------------------------------------------------------------
// base GEMM with epilogue, 32x32 output tile per block, LDS-staged operands:
//   y[perm[p]][j] = (x[perm[p]] . W[j] + [p < n_rot] delta[p] . W[j]) * s[j] + b[j]
// grid (ceil(d_out/32), ceil(n/32)), 256 threads, 4 outputs per thread; a
// row with an unusable adapter id gets NaN
// ---------------------------------------------------------------------------
// first column of projections 1, 2, 3 (d_out past the last)
struct ProjStarts {
  int64_t c[MAX_PROJ - 1];
};

static ProjStarts proj_starts(const scute_layer* L, bool rproj) {
  ProjStarts ps;
  for (int32_t i = 0; i + 1 < MAX_PROJ; ++i) ps.c[i] = rproj && i + 1 < L->n_proj ? L->proj_end[i] : L->d_out;
  return ps;
}

template <typename T>
__global__ void __launch_bounds__(256) k_gemm_ref(const T* __restrict__ x, const T* __restrict__ W,
                                                  const T* __restrict__ delta,
                                                  const int32_t* __restrict__ perm,
                                                  const int32_t* __restrict__ row_adapter,
                                                  const SlotEntry* __restrict__ table, int32_t na,
                                                  int32_t n, int32_t n_rot, int64_t d_in, int64_t d_out,
                                                  ProjStarts ps, float* __restrict__ y) {
  // 128 k per round: every thread's 32 loads of a round are in flight
  // together, so a round costs one memory round trip
  constexpr int KR = 128;
  // rows padded to 132 floats: 16-byte aligned for the float4 reads below,
  // and 8 consecutive rows start in 8 different 4-bank groups
  __shared__ __attribute__((aligned(16))) float xs[32][KR + 4];
  __shared__ __attribute__((aligned(16))) float ws[32][KR + 4];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int32_t p0 = blockIdx.y * 32;
  const int64_t j0 = (int64_t)blockIdx.x * 32;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const int passes = (p0 < n_rot) ? 2 : 1;
  // this block's projection picks the delta block (projection starts are
  // multiples of 64, so the 32 columns lie in one projection)
  const T* dz = delta + (size_t)((j0 >= ps.c[0]) + (j0 >= ps.c[1]) + (j0 >= ps.c[2])) * n_rot * d_in;
  for (int pass = 0; pass < passes; ++pass) {
    for (int64_t k0 = 0; k0 < d_in; k0 += KR) {
      for (int q = 0; q < 4; ++q) {
        const int r = ty + 8 * q;
        const int32_t p = p0 + r;
        const int64_t j = j0 + r;
        const bool xrow = pass == 0 ? p < n : p < n_rot;
        const T* xsrc = pass == 0 ? (p < n ? x + (size_t)src_row(perm, p) * d_in : x)
                                  : dz + (size_t)min(p, max(n_rot - 1, 0)) * d_in;
#pragma unroll
        for (int cq = 0; cq < KR / 32; ++cq) {
          const int64_t kk = k0 + 32 * cq + tx;
          xs[r][32 * cq + tx] = (xrow && kk < d_in) ? ldf(xsrc, kk) : 0.f;
          ws[r][32 * cq + tx] = (j < d_out && kk < d_in) ? ldf(W, (size_t)j * d_in + kk) : 0.f;
        }
      }
      __syncthreads();
      // 4 k per step: one float4 of W and one of each of the 4 rows (16 FMAs
      // per 5 LDS reads)
#pragma unroll 4
      for (int kk = 0; kk < KR; kk += 4) {
        const float4 wv = *reinterpret_cast<const float4*>(&ws[tx][kk]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 xv = *reinterpret_cast<const float4*>(&xs[ty + 8 * q][kk]);
          acc[q] += xv.x * wv.x;
          acc[q] += xv.y * wv.y;
          acc[q] += xv.z * wv.z;
          acc[q] += xv.w * wv.w;
        }
      }
      __syncthreads();
    }
  }
  const int64_t j = j0 + tx;
  if (j >= d_out) return;
  for (int q = 0; q < 4; ++q) {
    const int32_t p = p0 + ty + 8 * q;
    if (p >= n) continue;
    float v = acc[q];
    const int32_t a = row_id(row_adapter, p, table, na);
    if (a >= 0) {
      const SlotEntry E = table[a];
      if (E.flags & F_S) v *= E.s[j];
      if (E.flags & F_B) v += E.b[j];
    } else if (a == -2) {
      v = __builtin_nanf("");
    }
    y[(size_t)src_row(perm, p) * d_out + j] = v;
  }
}

// ---------------------------------------------------------------------------
// expand: y[perm[p]][j] += t[p] . B'[j] + e_a[j] * (u[p] . B_sh[j])
// grid (ceil(d_out/256), n)
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) k_expand_ref(const float* __restrict__ t,
                                                    const float* __restrict__ u,
                                                    const T* __restrict__ B_sh,
                                                    const int32_t* __restrict__ perm,
                                                    const int32_t* __restrict__ row_adapter,
                                                    const SlotEntry* __restrict__ table, int32_t na,
                                                    int32_t max_rank, int32_t r_v, int64_t d_out,
                                                    float* __restrict__ y) {
  const int32_t p = blockIdx.y;
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= d_out) return;
  const int32_t a = row_id(row_adapter, p, table, na);
  if (a < 0) return;
  const SlotEntry E = table[a];
  float v = 0.f;
  if (E.flags & F_TERM) {
    const T* Bj = (const T*)E.B + (size_t)j * E.rank;
    const float* tp = t + (size_t)p * max_rank;
    for (int32_t k = 0; k < E.rank; ++k) v += tp[k] * ldf(Bj, k);
  }
  if (E.flags & F_VERA) {
    const T* Bj = B_sh + (size_t)j * r_v;
    const float* up = u + (size_t)p * r_v;
    float w = 0.f;
    for (int32_t k = 0; k < r_v; ++k) w += up[k] * ldf(Bj, k);
    v += E.ve[j] * w;
  }
  if (E.flags & (F_TERM | F_VERA)) y[(size_t)src_row(perm, p) * d_out + j] += v;
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------

static inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

template <typename T>
static scute_status launch_ref(scute_layer* L, const scute_batch* B, const T* x, const T* W,
                               float* y, hipStream_t st, int32_t* launches) {
  const int32_t n = B->n;
  const int64_t d_in = L->d_in, d_out = L->d_out;
  int32_t nl = 0;
  if (B->n_rot > 0) {
    ProfScope ps(L, st, "rotate");
    const unsigned npz = B->rproj ? (unsigned)L->n_proj : 1u;
    hipLaunchKernelGGL(k_rotate_ref<T>, dim3(cdiv(d_in, 256), B->n_rot, npz), dim3(256), 0, st, x,
                       B->d_perm, B->d_row_adapter, L->table_dev, L->max_adapters, d_in, B->n_rot,
                       (T*)B->delta);
    ++nl;
  }
  if (B->max_rank > 0) {
    ProfScope ps(L, st, "shrink");
    hipLaunchKernelGGL(k_shrink_ref<T>, dim3(B->max_rank, n), dim3(256), 0, st, x, B->d_perm,
                       B->d_row_adapter, L->table_dev, L->max_adapters, d_in, B->max_rank, B->t);
    ++nl;
  }
  if (B->n_vera > 0) {
    ProfScope ps(L, st, "vera_shrink");
    hipLaunchKernelGGL(k_vera_shrink_ref<T>, dim3(L->r_v, B->n_vera), dim3(256), 0, st, x,
                       B->d_perm, B->d_row_adapter, B->d_vera_pos, L->table_dev, L->max_adapters,
                       (const T*)L->A_sh, d_in, L->r_v, B->u);
    ++nl;
  }
  {
    ProfScope ps(L, st, "gemm");
    hipLaunchKernelGGL(k_gemm_ref<T>, dim3(cdiv(d_out, 32), cdiv(n, 32)), dim3(256), 0, st, x, W,
                       (const T*)B->delta, B->d_perm, B->d_row_adapter, L->table_dev, L->max_adapters,
                       n, B->n_rot, d_in, d_out, proj_starts(L, B->rproj), y);
    ++nl;
  }
  if (B->max_rank > 0 || B->n_vera > 0) {
    ProfScope ps(L, st, "expand");
    hipLaunchKernelGGL(k_expand_ref<T>, dim3(cdiv(d_out, 256), n), dim3(256), 0, st, B->t, B->u,
                       (const T*)L->B_sh, B->d_perm, B->d_row_adapter, L->table_dev, L->max_adapters,
                       B->max_rank, L->r_v, d_out, y);
    ++nl;
  }
  SCUTE_HIP_CHECK(hipGetLastError());
  if (launches) *launches = nl;
  return SCUTE_OK;
}

int32_t forward_launch_count(const scute_layer* L, const scute_batch* B) {
  (void)L;
  if (B->n == 0) return 0;
  if (B->fp.enabled) return (B->fp.n_rot_items > 0) + 1;  // rotation + fused main
  if (B->dp.enabled) return 2 + decode_route_launches(B);  // prologue (gather, rotation, shrinks) + main
  if (B->pp.enabled) return (B->pp.n_pro > 0) + 1;  // prologue (rotation, shrinks) + main
  return (B->n_rot > 0) + (B->max_rank > 0) + (B->n_vera > 0) + 1 +
         (B->max_rank > 0 || B->n_vera > 0);
}

// SCUTE_TRACE=1 in the environment (read once): one line per forward on
// stderr with the path, the batch's shape and the launches it made
static bool trace_on() {
  static const bool on = [] {
    const char* v = getenv("SCUTE_TRACE");
    return v && *v && *v != '0';
  }();
  return on;
}

static scute_status launch_path(scute_layer* L, const scute_batch* B, const void* x, const void* W, float* y,
                                hipStream_t st, int32_t* launches) {
  if (B->fp.enabled) return launch_fdecode(L, B, x, W, y, st, launches);
  if (B->dp.enabled) return launch_decode(L, B, x, W, y, st, launches);
  if (B->pp.enabled) return launch_prefill(L, B, x, W, y, st, launches);
  if (L->act == SCUTE_BF16)
    return launch_ref<uint16_t>(L, B, (const uint16_t*)x, (const uint16_t*)W, y, st, launches);
  return launch_ref<float>(L, B, (const float*)x, (const float*)W, y, st, launches);
}

scute_status launch_forward(scute_layer* L, const scute_batch* B, const void* x, const void* W,
                            float* y, hipStream_t st, int32_t* launches) {
  int32_t nl = 0;
  const scute_status s = launch_path(L, B, x, W, y, st, &nl);
  if (launches) *launches = nl;
  if (trace_on()) {
    const char* path = B->fp.enabled ? "fused-decode" : B->dp.enabled ? "decode" : B->pp.enabled ? "prefill" : "generic";
    fprintf(stderr,
            "scute: forward layer=%p plan=%p path=%s n=%d d_in=%lld d_out=%lld segments=%d rot_rows=%d "
            "vera_rows=%d max_rank=%d route=0x%x launches=%d status=%d\n",
            (const void*)L, (const void*)B, path, B->n, (long long)L->d_in, (long long)L->d_out, B->nseg(),
            B->n_rot, B->n_vera, B->max_rank, B->dp.route, nl, (int)s);
  }
  return s;
}

}  // namespace scute

using namespace scute;

extern "C" scute_status scute_layer_forward(scute_layer* L, const scute_batch* B, const void* x,
                                            const void* W, float* y, void* stream) {
  if (!L || !B) return fail(SCUTE_E_INVALID, "scute_layer_forward: null layer or plan");
  if (B->layer != L) return fail(SCUTE_E_STATE, "scute_layer_forward: plan belongs to another layer");
  if (B->epoch != L->epoch)
    return fail(SCUTE_E_STATE, "scute_layer_forward: plan is stale (adapters changed since planning)");
  if (L->device < 0)
    return fail(SCUTE_E_UNSUPPORTED, "scute_layer_forward: host-only layer has no forward");
  if (B->n == 0) return SCUTE_OK;
  if (!x || !W || !y) return fail(SCUTE_E_INVALID, "scute_layer_forward: null x, W or y");
  if (((uintptr_t)x | (uintptr_t)W | (uintptr_t)y) & 15)
    return fail(SCUTE_E_INVALID, "scute_layer_forward: x, W and y must be 16-byte aligned");
  if (B->n_vera > 0 && (!L->A_sh || !L->B_sh))
    return fail(SCUTE_E_STATE, "scute_layer_forward: shared VeRA pair not set");
  int prev = -1;
  (void)hipGetDevice(&prev);
  if (prev != L->device) (void)hipSetDevice(L->device);
  scute_status st = launch_forward(L, B, x, W, y, (hipStream_t)stream, nullptr);
  if (prev != L->device && prev >= 0) (void)hipSetDevice(prev);
  return st;
}

namespace scute {
__global__ void k_empty() {}

// h = silu(g) (.) u, four elements per thread and grid-stride rounds
__global__ void __launch_bounds__(256) k_silu_gate(const float* __restrict__ g, const float* __restrict__ u,
                                                   float* h, int64_t count) {
  const int64_t n4 = count / 4;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const float4 gv = reinterpret_cast<const float4*>(g)[i];
    const float4 uv = reinterpret_cast<const float4*>(u)[i];
    float4 o;
    o.x = gv.x / (1.f + expf(-gv.x)) * uv.x;
    o.y = gv.y / (1.f + expf(-gv.y)) * uv.y;
    o.z = gv.z / (1.f + expf(-gv.z)) * uv.z;
    o.w = gv.w / (1.f + expf(-gv.w)) * uv.w;
    reinterpret_cast<float4*>(h)[i] = o;
  }
  if (blockIdx.x == 0 && threadIdx.x < count - 4 * n4) {
    const int64_t i = 4 * n4 + threadIdx.x;
    h[i] = g[i] / (1.f + expf(-g[i])) * u[i];
  }
}
}  // namespace scute

extern "C" scute_status scute_silu_gate(const float* g, const float* u, float* h, int64_t count, void* stream) {
  using namespace scute;
  if (count < 0) return fail(SCUTE_E_INVALID, "scute_silu_gate: count must be >= 0");
  if (count == 0) return SCUTE_OK;
  if (!g || !u || !h) return fail(SCUTE_E_INVALID, "scute_silu_gate: null pointer");
  if (((uintptr_t)g | (uintptr_t)u | (uintptr_t)h) & 15)
    return fail(SCUTE_E_INVALID, "scute_silu_gate: g, u and h must be 16-byte aligned");
  const int64_t blocks = std::min<int64_t>(std::max<int64_t>(1, (count / 4 + 255) / 256), 8192);
  hipLaunchKernelGGL(k_silu_gate, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, g, u, h, count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "scute_silu_gate");
  return SCUTE_OK;
}

extern "C" scute_status scute_launch_empty(int32_t count, void* stream) {
  using namespace scute;
  if (count < 0) return fail(SCUTE_E_INVALID, "scute_launch_empty: count must be >= 0");
  for (int32_t i = 0; i < count; ++i) hipLaunchKernelGGL(k_empty, dim3(1), dim3(64), 0, (hipStream_t)stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "scute_launch_empty");
  return SCUTE_OK;
}

extern "C" scute_status scute_profile_enable(scute_layer* L, int32_t enable) {
  if (!L) return fail(SCUTE_E_INVALID, "scute_profile_enable: layer is null");
  if (L->device < 0 && enable)
    return fail(SCUTE_E_UNSUPPORTED, "scute_profile_enable: host-only layer");
  L->profiling = enable != 0;
  return SCUTE_OK;
}

extern "C" scute_status scute_profile_read(scute_layer* L, scute_kernel_time* out,
                                           int32_t capacity, int32_t* count) {
  if (!L || !count) return fail(SCUTE_E_INVALID, "scute_profile_read: null argument");
  if (capacity > 0 && !out) return fail(SCUTE_E_INVALID, "scute_profile_read: out is null");
  for (const ProfEvent& ev : L->prof_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(ev.stop) == hipSuccess &&
        hipEventElapsedTime(&ms, ev.start, ev.stop) == hipSuccess) {
      L->prof_ms[ev.kind] += ms;
      L->prof_count[ev.kind] += 1;
    }
    L->prof_pool.push_back(ev.start);
    L->prof_pool.push_back(ev.stop);
  }
  L->prof_pending.clear();
  *count = (int32_t)L->prof_names.size();
  for (int32_t i = 0; i < *count && i < capacity; ++i) {
    memset(out[i].name, 0, sizeof(out[i].name));
    strncpy(out[i].name, L->prof_names[i].c_str(), sizeof(out[i].name) - 1);
    out[i].launches = L->prof_count[i];
    out[i].total_ms = L->prof_ms[i];
  }
  for (size_t i = 0; i < L->prof_ms.size(); ++i) {
    L->prof_ms[i] = 0.0;
    L->prof_count[i] = 0;
  }
  return SCUTE_OK;
}

// ---------------------------------------------------------------------------
// forward without allocation: the generic kernels on the batch in token
// order, their rotation output and shrink sums in a static device array
// ---------------------------------------------------------------------------
namespace scute {
namespace {

// Each device that loads this library holds its own copy until the process
// ends. Host code reaches it only through the address hipGetSymbolAddress
// returns on that device (the name is a host-side stand-in there).
static __device__ __align__(256) uint8_t scratch[SCUTE_NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[NOALLOC_MAX_DEVICES] = {};

// the layer-wide facts the token-order forward needs (recomputed after
// every load / unload)
void layer_facts(scute_layer* L) {
  if (L->na_epoch == L->epoch) return;
  int32_t rk = 0;
  bool rot = false, rproj = false;
  for (const SlotEntry& E : L->table) {
    if (!(E.flags & F_LOADED)) continue;
    if ((E.flags & F_TERM) && E.rank > rk) rk = E.rank;
    if (E.flags & F_R) rot = true;
    if (E.flags & F_RPROJ) rproj = true;
  }
  L->na_max_rank = rk;
  L->na_rot = rot;
  L->na_rproj = rproj;
  L->na_epoch = L->epoch;
}

template <typename T>
void launch_noalloc(scute_layer* L, const int32_t* ta, int32_t n, const T* x, const T* W, float* y,
                    uint8_t* ws, size_t o_t, size_t o_u, hipStream_t st) {
  const int64_t d_in = L->d_in, d_out = L->d_out;
  const int32_t na = L->max_adapters, rk = L->na_max_rank;
  const bool vera = L->n_vera_loaded > 0;
  T* delta = (T*)ws;  // one block of n rows per projection when an adapter rotates per projection
  float* t = (float*)(ws + o_t);
  float* u = (float*)(ws + o_u);
  const unsigned npz = L->na_rproj ? (unsigned)L->n_proj : 1u;
  if (L->na_rot)
    hipLaunchKernelGGL(k_rotate_ref<T>, dim3(cdiv(d_in, 256), n, npz), dim3(256), 0, st, x, nullptr, ta,
                       L->table_dev, na, d_in, n, delta);
  if (rk > 0)
    hipLaunchKernelGGL(k_shrink_ref<T>, dim3(rk, n), dim3(256), 0, st, x, nullptr, ta, L->table_dev, na,
                       d_in, rk, t);
  if (vera)
    hipLaunchKernelGGL(k_vera_shrink_ref<T>, dim3(L->r_v, n), dim3(256), 0, st, x, nullptr, ta, nullptr,
                       L->table_dev, na, (const T*)L->A_sh, d_in, L->r_v, u);
  hipLaunchKernelGGL(k_gemm_ref<T>, dim3(cdiv(d_out, 32), cdiv(n, 32)), dim3(256), 0, st, x, W,
                     (const T*)delta, nullptr, ta, L->table_dev, na, n, L->na_rot ? n : 0, d_in, d_out,
                     proj_starts(L, L->na_rproj), y);
  if (rk > 0 || vera)
    hipLaunchKernelGGL(k_expand_ref<T>, dim3(cdiv(d_out, 256), n), dim3(256), 0, st, t, u,
                       (const T*)L->B_sh, nullptr, ta, L->table_dev, na, rk, L->r_v, d_out, y);
}

}  // namespace

// Takes the device address of `scratch` on `device` (which must be
// current), once per device.
scute_status noalloc_setup(int32_t device) {
  if (device < 0 || device >= NOALLOC_MAX_DEVICES) return SCUTE_OK;  // the forward reports it
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch[device]) return SCUTE_OK;
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
  g_scratch[device] = p;
  return SCUTE_OK;
}

}  // namespace scute

extern "C" scute_status scute_layer_forward_noalloc(scute_layer* L, const int32_t* token_adapter, int32_t n,
                                                    const void* x, const void* W, float* y, void* stream) {
  using namespace scute;
  try {
    if (!L) return fail(SCUTE_E_INVALID, "scute_layer_forward_noalloc: layer is null");
    if (L->device < 0)
      return fail(SCUTE_E_UNSUPPORTED, "scute_layer_forward_noalloc: host-only layer has no forward");
    if (n < 0 || n > 65535) return fail(SCUTE_E_SHAPE, "scute_layer_forward_noalloc: n must be in [0, 65535]");
    if (n == 0) return SCUTE_OK;
    if (!token_adapter || !x || !W || !y)
      return fail(SCUTE_E_INVALID, "scute_layer_forward_noalloc: null token_adapter, x, W or y");
    if ((((uintptr_t)x | (uintptr_t)W | (uintptr_t)y) & 15) || ((uintptr_t)token_adapter & 3))
      return fail(SCUTE_E_INVALID,
                  "scute_layer_forward_noalloc: x, W, y must be 16-byte and token_adapter 4-byte aligned");
    const bool vera = L->n_vera_loaded > 0;
    if (vera && (!L->A_sh || !L->B_sh))
      return fail(SCUTE_E_STATE, "scute_layer_forward_noalloc: shared VeRA pair not set");
    layer_facts(L);
    auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
    const size_t es = dtype_size(L->act);
    const size_t npz = L->na_rproj ? (size_t)L->n_proj : 1;  // delta blocks
    const size_t o_t = L->na_rot ? al(npz * n * L->d_in * es) : 0;
    const size_t o_u = o_t + al((size_t)n * L->na_max_rank * 4);
    const size_t need = o_u + (vera ? (size_t)n * L->r_v * 4 : 0);
    if (need > (size_t)SCUTE_NOALLOC_SCRATCH_BYTES)
      return fail(SCUTE_E_SHAPE, "scute_layer_forward_noalloc: the batch needs " + std::to_string(need) +
                                     " bytes of scratch, more than the " +
                                     std::to_string((size_t)SCUTE_NOALLOC_SCRATCH_BYTES) + " it has");
    if (L->device >= NOALLOC_MAX_DEVICES)
      return fail(SCUTE_E_UNSUPPORTED, "scute_layer_forward_noalloc: device index past 63");
    int prev = -1;
    (void)hipGetDevice(&prev);
    if (prev != L->device) (void)hipSetDevice(L->device);
    scute_status stt = noalloc_setup(L->device);
    void* ws = nullptr;
    {
      std::lock_guard<std::mutex> g(g_scratch_mu);
      ws = g_scratch[L->device];
    }
    if (stt == SCUTE_OK) {
      hipStream_t st = (hipStream_t)stream;
      if (L->act == SCUTE_BF16)
        launch_noalloc<uint16_t>(L, token_adapter, n, (const uint16_t*)x, (const uint16_t*)W, y,
                                 (uint8_t*)ws, o_t, o_u, st);
      else
        launch_noalloc<float>(L, token_adapter, n, (const float*)x, (const float*)W, y, (uint8_t*)ws, o_t,
                              o_u, st);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) stt = hip_fail(e, "scute_layer_forward_noalloc: launch");
    }
    if (prev != L->device && prev >= 0) (void)hipSetDevice(prev);
    return stt;
  } catch (...) {
    return fail(SCUTE_E_INVALID, "scute_layer_forward_noalloc: unexpected error");
  }
}
