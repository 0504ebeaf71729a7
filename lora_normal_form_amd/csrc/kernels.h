// Device helpers shared by the HIP kernels of the decode and prefill paths
// (bf16 <-> fp32, 32x32x16 bf16 MFMA, global / buffer loads, system-coherent
// exchange, explicit vector-memory waits and work-group barriers).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace scute {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f2bf(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
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
__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  const u32x4 v = *(const GLOBAL u32x4*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ f32x4 ldg4(const float* p) { return *(const GLOBAL f32x4*)p; }
__device__ __forceinline__ void stg4(float* p, f32x4 v) { *(GLOBAL f32x4*)p = v; }
// c + the dot product of 8 bf16 pairs, on four bf16 dot2 instructions
// (fp32 accumulate)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot8(uint4 a, uint4 b, float c) {
  const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, av[i]),
                                        __builtin_bit_cast(bf16x2_t, bv[i]), c, false);
  return c;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Raw buffer resources over a byte range: loads past the range return zero,
// stores past it are dropped. (The third word's data-format field must be
// non-zero on gfx9 for raw dword accesses.)
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 ldb16(rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Exchange of partial results between work-groups on any XCD without
// whole-cache maintenance: the exchanged values are written and read with
// system-coherent buffer accesses (cache policy sc0 sc1: written through to
// memory, read from memory, past the per-XCD L2). They are ordinary
// compiler-visible memory operations, so the compiler waits for their
// results. A writer waits for its stores to complete before announcing them
// with an atomic on a counter; a reader issues its loads only after the
// atomic that saw every announcement has returned.
constexpr int CPOL_SYS = 17;  // sc0 | sc1
__device__ __forceinline__ void st_sys4(rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, CPOL_SYS);
}
__device__ __forceinline__ f32x4 ld_sys4(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL_SYS));
}
__device__ __forceinline__ void st_sys1(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, CPOL_SYS);
}
__device__ __forceinline__ void st_sys2(rsrc_t r, uint32_t off, uint32_t lo, uint32_t hi) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, r, off, 0, CPOL_SYS);
}
__device__ __forceinline__ uint4 ld_sys16(rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL_SYS));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float ld_sys1(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, CPOL_SYS));
}
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ int arrive(int32_t* cnt) {
  return __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void reset_counter(int32_t* cnt) {
  __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// s_waitcnt immediate (gfx9 encoding) waiting until at most `n` vector
// memory operations are outstanding; export and LDS counters unconstrained
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Work-group barrier that orders LDS traffic without waiting for outstanding
// global loads (the LDS-filling loads are awaited explicitly with s_waitcnt
// before it; LDS reads are consumed before it in program order).
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }
// Work-group barrier after LDS writes that other waves read next: waits for
// this wave's LDS operations first.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Keeps the compiler from moving memory operations across this point (the
// explicit vector-memory waits count loads in program order).
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const uint16_t* uni_ptr(const uint16_t* p) {
  const uint64_t v = (uint64_t)p;
  return (const uint16_t*)(((uint64_t)(uint32_t)uni((int)(v >> 32)) << 32) |
                           (uint32_t)uni((int)(uint32_t)v));
}
// two fp32 values (bit patterns) -> packed bf16, round to nearest even (one
// v_cvt_pk_bf16_f32 on gfx950)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(uint32_t lo, uint32_t hi) {
  const f32x2 v = {__uint_as_float(lo), __uint_as_float(hi)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// One 32x32 shrink tile over a K slice of 256 on 32x32x16 MFMA: lane (m, h)
// holds row m of both operands (xr: its x row, ar: its A row, each already
// offset to the slice and to the lane's 32-element half of every 64-element
// block; the k order inside a block is permuted identically on both).
// Element i of the result: operand-a row 8 (i / 4) + 4 h + i % 4, A row m.
__device__ __forceinline__ f32x16 shrink_tile(const uint16_t* xr, const uint16_t* ar,
                                               f32x16 acc = f32x16{}) {
  uint4 xa[16], wa[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    xa[q] = ldg16(xr + 64 * (q >> 2) + 8 * (q & 3));
    wa[q] = ldg16(ar + 64 * (q >> 2) + 8 * (q & 3));
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) acc = mfma32(xa[q], wa[q], acc);
  return acc;
}

}  // namespace scute
