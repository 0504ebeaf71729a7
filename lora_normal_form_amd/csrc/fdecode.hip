// Fused MFMA decode path (bf16 activations, fp32 accumulate, up to 256 rows).
//
// The layer ((x R) W) (.) s + b + sum_k c_k (((x A_k) (.) d_k) B_k (.) e_k)
// ("The big picture: six extra slots in the LoRA computation", paper-daily.com
// explainer of "Scute: Exact Batched Serving for PEFT Adapters Beyond LoRA")
// runs in at most two launches per forward:
//
// k_fd_rotate (rotate.hip; only when some row rotates): delta = x (R - I)
//   for the rotated rows, fp32 accumulate, rounded once to bf16. The
//   rotation comes before the shared GEMM, which then multiplies x and delta
//   by the same W fragments ("Where is the cheapest place to compute the
//   remaining slots?": rows are rotated by a kernel ahead of the GEMM and
//   then share it).
//
// k_fd_main, one work-group of 4 waves per (128-column tile, K slice):
//   K loop   the base GEMM of the tile's 128 outputs over the slice for every
//            row of the batch (wave w owns 32 outputs) on 32x32x16 bf16 MFMA
//            with W as the A operand, so a lane's accumulator holds one row
//            and 16 outputs. x and delta rows stream into an LDS ring by
//            direct loads shared by the four waves; W streams into registers
//            and through a per-wave LDS block into the MFMA layout.
//            The shrinks ride on the same loop: shrink block j (32 rank rows
//            of adapters' A', or of the shared A_sh, with one row group's x
//            rows) belongs to wave j / CG of column tile j % CG (all its K
//            slices); its A rows load straight into the MFMA layout beside W
//            and multiply the staged x rows already in LDS, so t = x A' and
//            the VeRA u = x A_sh cost no pass of their own (A_sh is read once
//            per K slice for the whole batch).
//   shrink   each slice stores its partial sums of the block (its K range),
//            and the last slice to arrive at the block adds the slices'
//            partials in slice order, stores the finished t (the rows of the
//            rank's adapter segment) or u (every VeRA row) and publishes the
//            block as done for this forward. No float atomics: every forward
//            gives the same bits.
//   meet     every slice stores its raw partial piece (row group g, wave w:
//            32 rows x 32 outputs) and counts its arrival; one slice per
//            piece (slice g % S: the pieces dealt round the slices) waits
//            for all of them, adds the slices' pieces in slice order and
//            finishes it: (.) s, the own low-rank expand t B' (not scaled by
//            s: s multiplies the base output only), the shared VeRA product
//            ((u (.) d) B_sh) (.) e, b, then stores y. Before it reads t and u
//            it also waits until the blocks of its row group are published.
//            Both are bounded waits that record a failure instead of
//            hanging; no slice waits on anything before it has stored its
//            pieces and arrived at its block, so the waits end whenever the
//            grid (at most one work-group per compute unit) is resident.

#include <algorithm>

#include "internal.h"
#include "kernels.h"

namespace scute {

namespace {

constexpr int FSK = 64;          // k per stage
constexpr int FROW = 2 * FSK;    // bytes per staged row and stage
constexpr int FWAVES = 4;        // waves (32 outputs each)
constexpr int XL = 4;            // shrink-block loads per wave and stage
constexpr int WL = 4 + XL;       // W + shrink-block loads per wave and stage

// ring depth by staged row groups (LDS: R stages of 32 MGT rows + 16 KB of
// W blocks + row records)
template <int MGT>
struct FdCfg {
  static constexpr int STAGE = 32 * MGT * FROW;
  static constexpr int R = MGT <= 4 ? 5 : (MGT <= 6 ? 4 : 3);
};

// number of loads a wave has issued after stage T's last load when it waits
// for stage T (issue order: W(0..R-2), X(0..R-2) before the loop; step t
// issues W(t+R-1), waits for stage t, passes the barrier, issues X(t+R-1);
// W(t) stands for the stage's W and shrink-block loads); stages past the
// last are not issued. The compiler may move loads later, which only makes
// the wait stricter.
__host__ __device__ constexpr int fd_after(int T, int NST, int R, int MGT) {
  int n = 0;
  for (int u = T + 1; u <= R - 2; ++u)
    if (u < NST) n += MGT;
  const int first = T <= R - 2 ? 0 : T - R + 2;
  for (int tau = first; tau < T; ++tau)
    if (tau + R - 1 < NST) n += WL + MGT;
  if (T + R - 1 < NST) n += WL;
  return n;
}

struct FdArgs {
  const uint16_t* x;
  const uint16_t* dx;
  const uint16_t* W;
  uint32_t x_bytes, dx_bytes, w_bytes, acc_bytes;
  const FdRow* rows;
  const FdStep* steps;
  const int32_t* goff;
  const int32_t* xoff;
  const FdXBlock* xb;
  int32_t n_xb;
  uint16_t* acc;      // [M_pad][AW] finished shrink sums (bf16)
  float* xpart;       // [n_xb][S][4 KB] partial shrink tiles
  int32_t* xcnt;      // [n_xb] block arrival counters
  uint32_t* xdone;    // [n_xb] forward number each block was finished for
  uint32_t xpart_bytes;
  uint32_t epoch;     // this forward's number (1, 2, ..)
  const uint16_t* B_sh;
  int32_t r_v;
  float* part;
  int32_t* cnt;
  uint32_t part_bytes;
  float* y;
  int32_t* err;
  int32_t d_in, d_out, MG, g_rot, S, C, RT, AW, k_chunk, gv0, gv1;
  int32_t CG;  // column tiles of the grid (tiles past d_out carry shrink blocks only)
  int32_t spin_limit;  // polls before a wait gives up
  uint32_t wait_bias;  // added to the forward number the waits look for (0; 1 makes them fail)
};

// W and the wave's shrink-block rows of one stage. W: the wave's 32 W rows
// x 128 bytes, 8 whole rows per instruction (lane l: row 8 s + l / 8, piece
// (l % 8) ^ (l / 8)) through a buffer resource. Shrink block: lane (m, h)
// loads the 64 bytes of rank row m it multiplies (pieces 4 h .. 4 h + 3),
// already in the A-operand layout (a wave without a block loads a dummy).
struct FdWSrc {
  rsrc_t r;
  uint32_t voff, rstep;
  const uint16_t* arow;  // this lane's shrink-block row at the slice's first k
};
__device__ __forceinline__ void fd_load_w(uint4 (&wr)[WL], const FdWSrc& ws, int stage) {
  const int soff = stage * FROW;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    wr[s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ws.r, ws.voff + s * ws.rstep, soff, 0));
#pragma unroll
  for (int s = 0; s < XL; ++s) wr[4 + s] = ldg16(ws.arow + stage * FSK + 8 * s);
}

// X of one stage, this wave's share: instructions w + 4 j (j < MGT) of the
// stage's 4 MGT, each filling 8 staged rows (lane l: row 8 q + l / 8; its
// 16-byte piece (l % 8) ^ ((row >> 1) % 8)); x rows through the x resource,
// delta rows through the delta resource (rows past the rotated ones read 0)
template <int MGT>
__device__ __forceinline__ void fd_stage_x(uint8_t* slot, rsrc_t rx, rsrc_t rd, const uint32_t* voff,
                                           int w, int mx_instr, int stage) {
  const int soff = stage * FROW;
#pragma unroll
  for (int j = 0; j < MGT; ++j) {
    const int q = w + 4 * j;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(q < mx_instr ? rx : rd, (lds_void*)(slot + q * 1024), 16,
                                             voff[j], soff, 0, 0);
  }
}

__device__ __forceinline__ uint4 fd_xfrag(const uint8_t* slot, int r, int piece) {
  return *reinterpret_cast<const uint4*>(slot + r * FROW + 16 * (piece ^ ((r >> 1) & 7)));
}

// one stage: 4 MFMA k-steps of 16 over every staged row group; W passes
// through the wave's LDS block (row r's piece p at slot p ^ (r % 8)) into
// the A-operand layout (lane (m, h): output m, pieces 4 h + s). A wave with
// a shrink block multiplies it with its group's x rows too (the block's k
// order: step s takes pieces 4 h + s, as W does).
template <int MGT>
__device__ __forceinline__ void fd_mma(const uint8_t* slot, const uint4 (&wl)[WL], uint8_t* wsw,
                                       f32x16 (&acc)[MGT], f32x16& xacc, int xg, int m, int h) {
#pragma unroll
  for (int s = 0; s < 4; ++s) *reinterpret_cast<uint4*>(wsw + s * 1024 + (32 * h + m) * 16) = wl[s];
  uint4 wr[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    wr[s] = *reinterpret_cast<const uint4*>(wsw + m * 128 + 16 * ((4 * h + s) ^ (m & 7)));
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 xv[MGT];
#pragma unroll
    for (int g = 0; g < MGT; ++g) xv[g] = fd_xfrag(slot, 32 * g + m, 4 * h + s);
#pragma unroll
    for (int g = 0; g < MGT; ++g) acc[g] = mfma32(wr[s], xv[g], acc[g]);
    if (xg >= 0) xacc = mfma32(wl[4 + s], fd_xfrag(slot, 32 * xg + m, 4 * h + s), xacc);
  }
}

template <int R>
struct FdRing {
  uint8_t* s[5];
  __device__ __forceinline__ uint8_t* at(int t) const { return s[t % R]; }
};

// K loop step T (compile time): prefetch W(T+R-1), wait for stage T, barrier,
// prefetch X(T+R-1) into the slot stage T-1 used, multiply stage T
template <int MGT, int NST, int R, int T>
__device__ __forceinline__ void fd_ksteps(const FdRing<R>& ring, uint4 (&wb)[R][WL], uint8_t* wsw,
                                          const FdWSrc& ws, rsrc_t rx, rsrc_t rd, const uint32_t* xvoff,
                                          int w, int mxi, f32x16 (&acc)[MGT], f32x16& xacc, int xg,
                                          int m, int h) {
  if constexpr (T < NST) {
    constexpr int TN = T + R - 1;
    if constexpr (TN < NST) fd_load_w(wb[TN % R], ws, TN);
    issue_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(fd_after(T, NST, R, MGT)));
    wg_barrier();
    if constexpr (TN < NST) fd_stage_x<MGT>(ring.at(TN), rx, rd, xvoff, w, mxi, TN);
    fd_mma<MGT>(ring.at(T), wb[T % R], wsw, acc, xacc, xg, m, h);
    fd_ksteps<MGT, NST, R, T + 1>(ring, wb, wsw, ws, rx, rd, xvoff, w, mxi, acc, xacc, xg, m, h);
  }
}

// s_waitcnt vmcnt(n) for a wave-uniform n known only at run time (the
// instruction takes an immediate): one branch per count; counts past 63 wait
// for less
template <int N>
__device__ __forceinline__ void wait_vm_rt(int n) {
  if constexpr (N < 63) {
    if (n == N)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
    else
      wait_vm_rt<N + 1>(n);
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(63));
  }
}

// runtime-length K loop (stage counts without a compiled unrolled loop): the
// same steps and the same exact waits
template <int MGT, int R>
__device__ __forceinline__ void fd_kloop_rt(int nst, const FdRing<R>& ring, uint4 (&wb)[R][WL],
                                            uint8_t* wsw, const FdWSrc& ws, rsrc_t rx, rsrc_t rd,
                                            const uint32_t* xvoff, int w, int mxi, f32x16 (&acc)[MGT],
                                            f32x16& xacc, int xg, int m, int h) {
#pragma unroll 1
  for (int t = 0; t < nst; t += R) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int T = t + i;
      if (T < nst) {
        const int TN = T + R - 1;
        if (TN < nst) fd_load_w(wb[(i + R - 1) % R], ws, TN);
        issue_fence();
        wait_vm_rt<0>(min(fd_after(T, nst, R, MGT), 63));
        wg_barrier();
        if (TN < nst) fd_stage_x<MGT>(ring.s[(i + R - 1) % R], rx, rd, xvoff, w, mxi, TN);
        fd_mma<MGT>(ring.s[i], wb[i], wsw, acc, xacc, xg, m, h);
      }
    }
  }
}

__device__ __forceinline__ int ld_sys_i32(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// 16 fp32 values of a piece: lane-contiguous 16-byte parts, part q of every
// lane in one 1 KB run (so each store instruction writes whole lines)
__device__ __forceinline__ uint32_t piece_part(uint32_t base, int q, int lane) {
  return base + (uint32_t)q * 1024u + (uint32_t)lane * 16u;
}

constexpr int FD_LDS_STEPS = 256;  // expand-step descriptors kept in LDS

// Slice finishing piece (g, w) of a tile: the groups are dealt round the
// slices (group g to slice g % S), so with MG <= S each wave finishes at most
// one piece and with MG > S neighbouring groups (VeRA rows and the rest come
// in runs of groups) land on different slices. Accumulator element i: row
// 32 g + m, output f0 + 8 (i / 4) + 4 h + i % 4.
__device__ __forceinline__ int fd_reducer(int g, int S) { return g % S; }

constexpr int FD_TJ = 4;  // own shrink sums a lane holds (ranks up to 64 in 16-rank steps)

// B' fragments of own expand steps s0 .. s0 + NB - 1 (A operand: B' row f of
// output fm, ranks kk + 8 h .. + 7)
template <int NB>
__device__ __forceinline__ void fd_load_bq(const FdArgs& a, const FdStep* sst, int s0, int e1, int64_t fm,
                                           int h, uint4 (&bq)[NB]) {
#pragma unroll
  for (int j = 0; j < NB; ++j)
    if (s0 + j < e1) {
      const FdStep st = s0 + j < FD_LDS_STEPS ? sst[s0 + j] : a.steps[s0 + j];
      const rsrc_t br = make_rsrc(uni_ptr(st.bp), (uint32_t)((int64_t)a.d_out * uni(st.rank) * 2));
      bq[j] = ldb16(br, (uint32_t)((fm * st.rank + st.kk + 8 * h) * 2));
    }
}
// B_sh fragments of VeRA steps s0 .. s0 + NB - 1 (ranks 16 s + 8 h .. + 7)
template <int NB>
__device__ __forceinline__ void fd_load_bv(const FdArgs& a, int s0, int nks, int64_t fm, int h,
                                           uint4 (&bv)[NB]) {
  const rsrc_t bsr = make_rsrc(a.B_sh, (uint32_t)((int64_t)a.d_out * a.r_v * 2));
#pragma unroll
  for (int j = 0; j < NB; ++j)
    if (s0 + j < nks) bv[j] = ldb16(bsr, (uint32_t)((fm * a.r_v + 16 * (s0 + j) + 8 * h) * 2));
}

// Bounded wait (spin_limit polls, ~2^20) until `ready` holds in every lane;
// a wait that gives up records the failure in the error flag and goes on.
template <typename F>
__device__ __forceinline__ void fd_wait(const FdArgs& a, int lane, F ready) {
  int spins = 0;
  for (;;) {
    if (__ballot(!ready()) == 0) return;
    __builtin_amdgcn_s_sleep(2);
    if (++spins > a.spin_limit) {
      if (lane == 0) __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      return;
    }
  }
}

// The slice's share of the finishing: it waits until every slice has stored
// the piece, adds the slices' raw sums in slice order and applies (.) s; then
// it waits until the group's shrink blocks are finished for this forward and
// adds the own expand (t B': t is not scaled by s, which multiplies the base
// output only), the VeRA product ((u (.) d) B_sh) (.) e and b, and stores y.
// The B' and B_sh fragments of the first steps load before the waits.
template <int NB>
__device__ void fd_finish_piece(const FdArgs& a, const FdRow& rr, const f32x16& mine, int g, int k,
                                int f0, int lane, int m, int h, rsrc_t pr, uint32_t piece_base0,
                                uint32_t piece_stride, const int32_t* pcnt, const FdStep* sst) {
  const int row = 32 * g + m;
  const int f4 = f0 + 4 * h;
  const int64_t fm = (int64_t)f0 + m;  // A-operand row (output) in expand steps
  const int fl = rr.flags;
  // (a) what depends on nothing written in this forward: the row's factor
  //     vectors and the first expand steps' B' and B_sh fragments
  f32x4 s4[4], e4[4], b4[4];
  if (fl & FR_S)
#pragma unroll
    for (int q = 0; q < 4; ++q) s4[q] = ldg4(rr.s + f4 + 8 * q);
  if (fl & FR_E)
#pragma unroll
    for (int q = 0; q < 4; ++q) e4[q] = ldg4(rr.e + f4 + 8 * q);
  if (fl & FR_B)
#pragma unroll
    for (int q = 0; q < 4; ++q) b4[q] = ldg4(rr.b + f4 + 8 * q);
  const int e0 = uni(a.goff[g]), e1 = uni(a.goff[g + 1]);
  const int nks = g >= a.gv0 && g < a.gv1 ? a.r_v / 16 : 0;
  uint4 bq[NB], bv[NB];
  fd_load_bq<NB>(a, sst, e0, e1, fm, h, bq);
  fd_load_bv<NB>(a, 0, nks, fm, h, bv);
  issue_fence();
  // (b) every slice's piece stored: its arrival count grows by S per forward
  if (a.S > 1) {
    const uint32_t need = (uint32_t)a.S * (a.epoch + a.wait_bias);
    fd_wait(a, lane, [&] {
      return lane != 0 ||
             (int)((uint32_t)__hip_atomic_load(pcnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) - need) >= 0;
    });
  }
  // (c) the slices' sums, in slice order, NB slices' loads at a time; (.) s
  f32x16 tot = {};
  for (int s0 = 0; s0 < a.S; s0 += NB) {
    f32x4 v[NB][4];
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (s0 + j < a.S && s0 + j != k)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[j][q] = ld_sys4(pr, piece_part(piece_base0 + (uint32_t)(s0 + j) * piece_stride, q, lane));
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (s0 + j < a.S) {
        if (s0 + j == k) {
          tot += mine;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) tot[4 * q + i] += v[j][q][i];
        }
      }
  }
  if (fl & FR_S)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[4 * q + i] *= s4[q][i];
  // (d) the group's shrink blocks finished for this forward (lane j: block
  //     xoff[g] + j, 64 at a time)
  {
    const int b0 = uni(a.xoff[g]), nb = uni(a.xoff[g + 1]) - b0;
    for (int j0 = 0; j0 < nb; j0 += 64)
      fd_wait(a, lane, [&] {
        return j0 + lane >= nb ||
               __hip_atomic_load(a.xdone + b0 + j0 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) ==
                   a.epoch + a.wait_bias;
      });
  }
  const rsrc_t racc = make_rsrc(a.acc, a.acc_bytes);
  // (e) this lane's own shrink sums (row `row`, ranks 16 j + 8 h .. + 7) for
  //     ranks up to 16 FD_TJ, all in one round
  const int rk = rr.rank;
  uint4 tr[FD_TJ];
#pragma unroll
  for (int j = 0; j < FD_TJ; ++j) {
    tr[j] = make_uint4(0, 0, 0, 0);
    if (16 * j < rk && rk <= 16 * FD_TJ)
      tr[j] = ld_sys16(racc, (uint32_t)(((int64_t)row * a.AW + 16 * j + 8 * h) * 2));
  }
  // (f) own expand: the group's steps, NB at a time (B = this lane's row's 8
  //     shrink sums of the step's ranks, zero outside the step's rows and
  //     the term's rank)
  for (int s0 = e0; s0 < e1; s0 += NB) {
    if (s0 != e0) fd_load_bq<NB>(a, sst, s0, e1, fm, h, bq);
    uint4 tq[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (s0 + j < e1) {
        const FdStep st = s0 + j < FD_LDS_STEPS ? sst[s0 + j] : a.steps[s0 + j];
        const int kk = st.kk + 8 * h;
        const bool in = kk < st.rank && row >= st.lo && row < st.hi;
        tq[j] = make_uint4(0, 0, 0, 0);
        if (uni(st.rank) <= 16 * FD_TJ) {
          const int jj = uni(st.kk) >> 4;
          const uint4 tv = jj == 0 ? tr[0] : jj == 1 ? tr[1] : jj == 2 ? tr[2] : tr[3];
          if (in) tq[j] = tv;
        } else if (in) {
          tq[j] = ld_sys16(racc, (uint32_t)(((int64_t)row * a.AW + kk) * 2));
        }
      }
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (s0 + j < e1) tot = mfma32(bq[j], tq[j], tot);
  }
  // (g) the shared VeRA term for a group holding VeRA rows (the stored u is
  //     already scaled by d; only VeRA rows load theirs), then (.) e
  if (nks > 0) {
    f32x16 v = {};
    const bool vrow = (fl & FR_VERA) != 0;
    for (int s0 = 0; s0 < nks; s0 += NB) {
      if (s0 != 0) fd_load_bv<NB>(a, s0, nks, fm, h, bv);
      uint4 uq[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j)
        if (s0 + j < nks) {
          uq[j] = make_uint4(0, 0, 0, 0);
          if (vrow) uq[j] = ld_sys16(racc, (uint32_t)(((int64_t)row * a.AW + a.RT + 16 * (s0 + j) + 8 * h) * 2));
        }
#pragma unroll
      for (int j = 0; j < NB; ++j)
        if (s0 + j < nks) v = mfma32(bv[j], uq[j], v);
    }
    if (fl & FR_E)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[4 * q + i] += v[4 * q + i] * e4[q][i];
  }
  // (h) b, then y
  if (fl & FR_B)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[4 * q + i] += b4[q][i];
  if (rr.tok >= 0) {
    float* yr = a.y + (size_t)rr.tok * a.d_out + f4;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      stg4(yr + 8 * q, f32x4{tot[4 * q], tot[4 * q + 1], tot[4 * q + 2], tot[4 * q + 3]});
  }
}

// The last slice to arrive at shrink block j finishes it: the slices'
// partial tiles added in slice order, rounded once to bf16 (the expand's
// operand type) and stored as t (own ranks: the rows of the rank's adapter)
// or u (VeRA ranks: every VeRA row of the group) in the shrink buffer, then
// the block is published as done for this forward.
// Lane (m, h) holds row 32 g + m and rank rows 8 q + 4 h .. + 3 (q < 4);
// each run of 4 rank rows belongs to one adapter (adapters start at rank
// rows that are multiples of 8 within a block), so it stores as one float4.
__device__ void fd_finish_block(const FdArgs& a, int j, int g, int k, const f32x16& mine, int lane,
                                int m, int h, rsrc_t xr, uint32_t xbase) {
  f32x16 tot = {};
  for (int s0 = 0; s0 < a.S; s0 += 8) {
    f32x4 v[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (s0 + i < a.S && s0 + i != k)
#pragma unroll
        for (int q = 0; q < 4; ++q) v[i][q] = ld_sys4(xr, piece_part(xbase + (uint32_t)(s0 + i) * 4096u, q, lane));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (s0 + i < a.S) {
        if (s0 + i == k) {
          tot += mine;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) tot[4 * q + e] += v[i][q][e];
        }
      }
  }
  const FdXBlock* B = a.xb + j;
  const int row = 32 * g + m;
  const int vera = uni(B->vera);
  const FdRow& rr = a.rows[row];
  const bool vrow = (rr.flags & FR_VERA) != 0;
  const rsrc_t racc = make_rsrc(a.acc, a.acc_bytes);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rk = 8 * q + 4 * h;
    const int col = B->col[rk];
    const int lh = B->lohi[rk];
    const bool ok = col >= 0 && (vera ? vrow : (row >= (lh & 0xFFFF) && row < (lh >> 16)));
    if (ok) {
      f32x4 v = f32x4{tot[4 * q], tot[4 * q + 1], tot[4 * q + 2], tot[4 * q + 3]};
      if (vera) v *= ldg4(rr.d + (col - a.RT));  // u = (x A_sh) (.) d of the row's adapter
      const u32x4 vb = __builtin_bit_cast(u32x4, v);
      st_sys2(racc, (uint32_t)(((int64_t)row * a.AW + col) * 2), pack_bf2(vb.x, vb.y), pack_bf2(vb.z, vb.w));
    }
  }
  wait_vm_all();
  if (lane == 0) __hip_atomic_store(a.xdone + j, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

template <int MGT, int NST>
__global__ void __launch_bounds__(256, 1) k_fd_main(FdArgs a) {
  using Cfg = FdCfg<MGT>;
  constexpr int R = Cfg::R;
  constexpr int ST = Cfg::STAGE;
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[ST];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[ST];
  __shared__ __attribute__((aligned(1024))) uint8_t slot2[ST];
  __shared__ __attribute__((aligned(1024))) uint8_t slot3[R > 3 ? ST : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t slot4[R > 4 ? ST : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t wst[FWAVES * 4096];
  __shared__ FdRow rec[32 * MGT];
  __shared__ FdStep sst[FD_LDS_STEPS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31, h = lane >> 5;
  const int MG = a.MG;
  const int Mx = 32 * MG;
  // tile (column tile c, K slice k): work-groups go round-robin to the XCDs,
  // so k = id % S keeps each slice's x rows in one XCD's L2
  const int k = (int)blockIdx.x % a.S, c = (int)blockIdx.x / a.S;
  const int f0 = 128 * c + 32 * w;  // this wave's first output
  const int64_t kbase = (int64_t)k * a.k_chunk;
  const int nst = NST > 0 ? NST : a.k_chunk / FSK;

  // (0) the rows' records (LDS, read after the loop), this lane's staged
  //     rows' sources and the wave's shrink block (block w CG + c: at most
  //     one per wave, spread over the tiles first)
  if (tid < Mx) rec[tid] = a.rows[tid];
  {
    const int ns = min(uni(a.goff[MG]), FD_LDS_STEPS);
    if (tid < ns) sst[tid] = a.steps[tid];
  }
  const int mxi = Mx / 8;  // x instructions of a stage (then delta)
  uint32_t xvoff[MGT];
#pragma unroll
  for (int j = 0; j < MGT; ++j) {
    const int q = w + 4 * j;
    const int r = 8 * q + (lane >> 3);
    const int piece = (lane & 7) ^ ((r >> 1) & 7);
    if (q < mxi) {
      const int src = a.rows[min(r, Mx - 1)].src;
      xvoff[j] = (uint32_t)(((int64_t)src * a.d_in + kbase + 8 * piece) * 2);
    } else {
      xvoff[j] = (uint32_t)(((int64_t)(r - Mx) * a.d_in + kbase + 8 * piece) * 2);
    }
  }
  const int xbi = w * a.CG + c;  // this wave's shrink block, if any
  int xg = -1;
  const uint16_t* arow = a.x;  // dummy source without a block
  if (xbi < a.n_xb) {
    xg = uni(a.xb[xbi].g);
    const uint16_t* ar = a.xb[xbi].arow[m];
    if (ar) arow = ar + kbase + 32 * h;
  }
  const rsrc_t rx = make_rsrc(a.x, a.x_bytes);
  const rsrc_t rd = make_rsrc(a.dx, a.dx_bytes);
  const FdWSrc ws{make_rsrc(a.W, a.w_bytes),
                  (uint32_t)((((int64_t)f0 + (lane >> 3)) * a.d_in + kbase) * 2 + 16 * ((lane & 7) ^ (lane >> 3))),
                  (uint32_t)(8 * a.d_in * 2), arow};
  uint8_t* wsw = wst + w * 4096;
  const FdRing<R> ring{{slot0, slot1, slot2, slot3, slot4}};

  // (1) prefetch: W(0..R-2), then X(0..R-2)
  uint4 wb[R][WL];
#pragma unroll
  for (int t = 0; t < R - 1; ++t)
    if (NST == 0 ? t < nst : t < NST) fd_load_w(wb[t], ws, t);
#pragma unroll
  for (int t = 0; t < R - 1; ++t)
    if (NST == 0 ? t < nst : t < NST) fd_stage_x<MGT>(ring.s[t], rx, rd, xvoff, w, mxi, t);

  f32x16 acc[MGT];
#pragma unroll
  for (int g = 0; g < MGT; ++g) acc[g] = f32x16{};
  f32x16 xacc = {};

  // (2) K loop
  if constexpr (NST > 0)
    fd_ksteps<MGT, NST, R, 0>(ring, wb, wsw, ws, rx, rd, xvoff, w, mxi, acc, xacc, xg, m, h);
  else
    fd_kloop_rt<MGT, R>(nst, ring, wb, wsw, ws, rx, rd, xvoff, w, mxi, acc, xacc, xg, m, h);
  wait_vm_all();

  // waves of the last tile whose 32 outputs lie past d_out stop after the
  // shrink publication below
  const bool live = f0 < a.d_out;

  // (4) delta rows: group MG + j folds onto x group j (rotated rows come
  //     first in the sorted order)
  const int g_rot = a.g_rot;
#pragma unroll
  for (int gp = 1; gp < MGT; ++gp)
#pragma unroll
    for (int g = 0; g < gp; ++g)
      if (gp - g == MG && g < g_rot) acc[g] += acc[gp];

  // (5) pieces: store this slice's raw sums, count the arrival (after the
  //     shrink block's publication), and finish the pieces this slice
  //     arrived at last
  const rsrc_t pr = make_rsrc(a.part, a.part_bytes);
  const uint32_t piece_stride = (uint32_t)MG * FWAVES * 4096u;  // between slices
  const uint32_t tile_base = (uint32_t)c * (uint32_t)a.S * piece_stride;
  if (live && a.S > 1) {
#pragma unroll
    for (int g = 0; g < MGT; ++g)
      if (g < MG) {
        const uint32_t o = tile_base + (uint32_t)k * piece_stride + (uint32_t)(g * FWAVES + w) * 4096u;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          st_sys4(pr, piece_part(o, q, lane),
                  f32x4{acc[g][4 * q], acc[g][4 * q + 1], acc[g][4 * q + 2], acc[g][4 * q + 3]});
      }
  }
  // (6) the shrink block's partial sums of this slice (element i: rank row
  //     8 (i / 4) + 4 h + i % 4 of the block, sorted row 32 xg + m)
  const rsrc_t xr = make_rsrc(a.xpart, a.xpart_bytes);
  const uint32_t xbase = (uint32_t)xbi * (uint32_t)a.S * 4096u;
  if (xg >= 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      st_sys4(xr, piece_part(xbase + (uint32_t)k * 4096u, q, lane),
              f32x4{xacc[4 * q], xacc[4 * q + 1], xacc[4 * q + 2], xacc[4 * q + 3]});
  }
  wait_vm_all();  // the pieces and the block's partial have landed
  // arrivals: the pieces first (their finishing waits on them), then the
  // shrink block, which the last slice to arrive finishes
  if (live && a.S > 1 && lane < MG)
    __hip_atomic_fetch_add(a.cnt + (c * MG + lane) * FWAVES + w, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  if (xg >= 0) {
    int old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(a.xcnt + xbi, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    old = __shfl(old, 0, 64);
    if ((old + 1) % a.S == 0) fd_finish_block(a, xbi, xg, k, xacc, lane, m, h, xr, xbase);
  }
  if (!live) return;
#pragma unroll
  for (int g = 0; g < MGT; ++g)
    if (g < MG && fd_reducer(g, a.S) == k)
      fd_finish_piece<MGT <= 5 ? 8 : 4>(a, rec[32 * g + m], acc[g], g, k, f0, lane, m, h, pr,
                      tile_base + (uint32_t)(g * FWAVES + w) * 4096u, piece_stride,
                      a.cnt + (c * MG + g) * FWAVES + w, sst);
}

template <int MGT>
void launch_fd_main(const FdArgs& a, int grid, int nst, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  switch (nst) {
    case 8: hipExtLaunchKernelGGL((k_fd_main<MGT, 8>), dim3(grid), dim3(256), 0, st, e0, e1, 0, a); break;
    case 16: hipExtLaunchKernelGGL((k_fd_main<MGT, 16>), dim3(grid), dim3(256), 0, st, e0, e1, 0, a); break;
    case 32: hipExtLaunchKernelGGL((k_fd_main<MGT, 32>), dim3(grid), dim3(256), 0, st, e0, e1, 0, a); break;
    default: hipExtLaunchKernelGGL((k_fd_main<MGT, 0>), dim3(grid), dim3(256), 0, st, e0, e1, 0, a); break;
  }
}

}  // namespace

scute_status launch_fdecode(scute_layer* L, const scute_batch* B, const void* x, const void* W,
                            float* y, hipStream_t st, int32_t* launches) {
  const FdPlan& P = B->fp;
  int nl = 0;
  if (P.n_rot_items > 0) {
    if (!B->delta || !P.rot) return fail(SCUTE_E_STATE, "fused decode: rotation tables missing");
    ProfScope ps(L, st, "fd_rotate");
    scute_status rs = launch_rotate_items(P.rot, P.n_rot_items, P.rot_blk, (const uint16_t*)x,
                                          (uint16_t*)B->delta, (int32_t)L->d_in, st);
    if (rs != SCUTE_OK) return rs;
    ++nl;
  }
  FdArgs a{};
  a.x = (const uint16_t*)x;
  a.dx = (const uint16_t*)B->delta;
  a.W = (const uint16_t*)W;
  a.x_bytes = (uint32_t)((size_t)B->n * L->d_in * 2);
  a.dx_bytes = (uint32_t)((size_t)B->n_rot * L->d_in * 2);
  a.w_bytes = (uint32_t)((size_t)L->d_out * L->d_in * 2);
  a.acc_bytes = P.acc_bytes;
  a.rows = P.rows;
  a.steps = P.steps;
  a.goff = P.goff;
  a.xb = P.xb;
  a.n_xb = P.n_xb;
  a.acc = P.acc;
  a.xpart = P.xpart;
  a.xcnt = P.xcnt;
  a.xdone = P.xdone;
  a.xpart_bytes = P.xpart_bytes;
  a.epoch = P.fwd + 1;
  a.xoff = P.xoff;
  a.B_sh = (const uint16_t*)L->B_sh;
  a.r_v = L->r_v;
  a.part = P.part;
  a.cnt = P.cnt;
  a.part_bytes = P.part_bytes;
  a.y = y;
  a.err = P.err;
  a.d_in = (int32_t)L->d_in;
  a.d_out = (int32_t)L->d_out;
  a.MG = P.MG;
  a.g_rot = P.g_rot;
  a.S = P.S;
  a.C = P.C;
  a.RT = P.RT;
  a.AW = P.AW;
  a.k_chunk = (int32_t)(L->d_in / P.S);
  a.gv0 = P.gv0;
  a.gv1 = P.gv1;
  a.CG = P.CG;
  a.spin_limit = P.spin_limit;
  a.wait_bias = P.wait_bias;
  if (!a.rows || !a.goff || !a.xoff || !a.acc || !a.cnt || !a.err ||
      (P.n_xb > 0 && (!a.xb || !a.xpart || !a.xcnt || !a.xdone)) ||
      (P.S > 1 && !a.part) || (B->n_rot > 0 && !a.dx) || (P.gv1 > P.gv0 && !a.B_sh))
    return fail(SCUTE_E_STATE, "fused decode: plan tables missing");
  const int grid = P.CG * P.S;
  {
    ProfScope ps(L, st, "fd_main", true);
    switch (P.MGT) {
      case 1: launch_fd_main<1>(a, grid, P.NST, st, ps.ev_start(), ps.ev_stop()); break;
      case 2: launch_fd_main<2>(a, grid, P.NST, st, ps.ev_start(), ps.ev_stop()); break;
      case 3: launch_fd_main<3>(a, grid, P.NST, st, ps.ev_start(), ps.ev_stop()); break;
      case 4: launch_fd_main<4>(a, grid, P.NST, st, ps.ev_start(), ps.ev_stop()); break;
      case 5: launch_fd_main<5>(a, grid, P.NST, st, ps.ev_start(), ps.ev_stop()); break;
      case 6: launch_fd_main<6>(a, grid, P.NST, st, ps.ev_start(), ps.ev_stop()); break;
      case 7: launch_fd_main<7>(a, grid, P.NST, st, ps.ev_start(), ps.ev_stop()); break;
      case 8: launch_fd_main<8>(a, grid, P.NST, st, ps.ev_start(), ps.ev_stop()); break;
      default: return fail(SCUTE_E_UNSUPPORTED, "fused decode: unsupported staged row groups");
    }
    ++nl;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch k_fd_main");
  // the blocks of the next forward are published under the next number
  ++P.fwd;
  if (launches) *launches = nl;
  return SCUTE_OK;
}

}  // namespace scute
