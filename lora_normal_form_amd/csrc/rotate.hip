// OFT rotation as a pass of its own: delta = x (R - I) for the rotated rows,
// fp32 accumulate, rounded once to bf16. The rotation has to come before the
// shared GEMM (R acts on the input, the expand comes after the GEMM), and
// the rotated rows then go through the same GEMM as every other row
// ("Where is the cheapest place to compute the remaining slots?",
// paper-daily.com explainer of "Scute: Exact Batched Serving for PEFT
// Adapters Beyond LoRA"). Used by the fused decode path and by the decode
// path's rotate-pass route.

#include "internal.h"
#include "kernels.h"

namespace scute {

namespace {

struct RotArgs {
  const uint16_t* x;
  const FdRotItem* items;
  uint16_t* dx;
  int32_t d_in;
};

// One item: up to 4 rows of one adapter segment over NC columns (512, or 256
// for blocks of 64). Column j of the block-diagonal (R - I) is stored as its
// BLK values in a row, so the item's columns are one contiguous run of NC
// BLK bf16: the work-group loads it with coalesced 16-byte loads into LDS
// (column j at j CS bytes; the 16-byte pad puts the columns 16 neighbouring
// lanes read in distinct banks), and the rows' x over the same columns too.
// Thread t then computes columns t and t + 256 for every row of the item,
// one fp32 dot product per column in k order, and the bf16 results leave as
// 16-byte row stores through LDS. Other block sizes (BLK = 0) take a scalar
// loop per column.
template <int BLK>
__global__ void __launch_bounds__(256) k_fd_rotate(RotArgs a) {
  constexpr int NC = BLK == 64 ? 256 : 512;
  constexpr int PPC = BLK > 0 ? BLK / 8 : 1;
  constexpr int NR = NC * PPC / 256;
  constexpr int CS = BLK * 2 + (BLK >= 16 ? 16 : 0);
  __shared__ __attribute__((aligned(16))) uint8_t sp[BLK > 0 ? NC * CS : 16];
  __shared__ __attribute__((aligned(16))) uint16_t sx[4][NC];
  __shared__ __attribute__((aligned(16))) uint16_t so[4][NC];
  const FdRotItem it = a.items[blockIdx.x];
  const int t = threadIdx.x;
  const int ncols = min(NC, a.d_in - it.c0);  // a multiple of 64
  const int nr = it.n;
  if constexpr (BLK > 0) {
    const uint16_t* pg = it.P + (size_t)it.c0 * BLK;
    uint4 pv[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int q = 256 * i + t;
      pv[i] = q < ncols * PPC ? ldg16(pg + 8 * q) : make_uint4(0, 0, 0, 0);
    }
    {
      const int r = t >> 6, pc = t & 63;
      if (r < nr && 8 * pc < ncols)
        *reinterpret_cast<uint4*>(&sx[r][8 * pc]) = ldg16(a.x + (size_t)it.tok[r] * a.d_in + it.c0 + 8 * pc);
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int q = 256 * i + t;
      *reinterpret_cast<uint4*>(sp + (q / PPC) * CS + 16 * (q % PPC)) = pv[i];
    }
    lds_barrier();
#pragma unroll
    for (int cc = 0; cc < NC / 256; ++cc) {
      const int col = t + 256 * cc;
      if (col < ncols) {
        const int kb0 = col / BLK * BLK;
        uint4 pc[PPC];
#pragma unroll
        for (int p = 0; p < PPC; ++p) pc[p] = *reinterpret_cast<const uint4*>(sp + col * CS + 16 * p);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (r < nr) {
            float v = 0.f;
#pragma unroll
            for (int p = 0; p < PPC; ++p) v = dot8(*reinterpret_cast<const uint4*>(&sx[r][kb0 + 8 * p]), pc[p], v);
            so[r][col] = f2bf(v);
          }
      }
    }
  } else {
    for (int col = t; col < ncols; col += 256) {
      const int64_t cl = it.c0 + col;
      const int64_t kb = cl / it.blk, jj = cl - kb * it.blk;
      const uint16_t* pb = it.P + ((size_t)kb * it.blk + jj) * it.blk;
      for (int r = 0; r < nr; ++r) {
        const uint16_t* xr = a.x + (size_t)it.tok[r] * a.d_in + kb * it.blk;
        float v = 0.f;
        for (int i = 0; i < it.blk; ++i) v += bf2f(ldg(xr + i)) * bf2f(ldg(pb + i));
        so[r][col] = f2bf(v);
      }
    }
  }
  lds_barrier();
  for (int o = t; o < 4 * NC / 8; o += 256) {
    const int r = o / (NC / 8), pc = o % (NC / 8);
    if (r < nr && 8 * pc < ncols)
      *(GLOBAL u32x4*)(a.dx + (size_t)(it.p0 + r) * a.d_in + it.c0 + 8 * pc) =
          *reinterpret_cast<const u32x4*>(&so[r][8 * pc]);
  }
}

}  // namespace

scute_status launch_rotate_items(const FdRotItem* items, int32_t n_items, int32_t blk, const uint16_t* x,
                                 uint16_t* dx, int32_t d_in, hipStream_t st) {
  if (n_items <= 0) return SCUTE_OK;
  if (!items || !x || !dx) return fail(SCUTE_E_STATE, "rotation pass: tables or buffers missing");
  RotArgs ra{x, items, dx, d_in};
  const dim3 g(n_items), b(256);
  switch (blk) {  // one block size for every item (else the scalar form)
    case 8: hipLaunchKernelGGL(k_fd_rotate<8>, g, b, 0, st, ra); break;
    case 16: hipLaunchKernelGGL(k_fd_rotate<16>, g, b, 0, st, ra); break;
    case 32: hipLaunchKernelGGL(k_fd_rotate<32>, g, b, 0, st, ra); break;
    case 64: hipLaunchKernelGGL(k_fd_rotate<64>, g, b, 0, st, ra); break;
    default: hipLaunchKernelGGL(k_fd_rotate<0>, g, b, 0, st, ra); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch k_fd_rotate");
  return SCUTE_OK;
}

}  // namespace scute
