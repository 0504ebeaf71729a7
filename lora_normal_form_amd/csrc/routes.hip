// Route variants of the decode path: the steps the default route fuses into
// the GEMM's epilogue (or its prologue), each run as a pass of its own, for
// the route comparison and the time model of "Where is the cheapest place
// to compute the remaining slots?" (paper-daily.com explainer of "Scute:
// Exact Batched Serving for PEFT Adapters Beyond LoRA"). That section
// compares applying DoRA's / (IA)^3's s inside the expand (which reads and
// writes the output tile by tile anyway, so s costs one more read) with a
// separate pass that first copies s to every row and then multiplies the
// output; it multiplies VeRA's shared pair for the whole batch; and it
// rotates OFT rows in a pass before the GEMM. Its time model prices a route
// by the bytes it moves over the memory bandwidth plus its launches times a
// fixed launch cost.
//
// Passes (each one launch, all on the batch's sorted rows; y is indexed by
// token through perm):
//   k_route_expand<SCALE>  per chunk of one adapter's rows: y = y (.) s
//                          (SCALE only) + b + t B' (t: the prologue's fp32
//                          shrink sums)
//   k_route_vera           every VeRA row of the batch: y += e (.) (u B_sh)
//                          on MFMA, B_sh read once per 32 VeRA rows (u: the
//                          prologue's shrink sums, already scaled by d)
//   k_route_s_copy         S[p] = s of row p's adapter (ones without s)
//   k_route_s_mul          y (.)= S
// The rotation pass is k_fd_rotate (rotate.hip).

#include "internal.h"
#include "kernels.h"

namespace scute {

namespace {

struct RtArgs {
  const SlotEntry* table;
  const int32_t* perm;         // sorted row -> token
  const int32_t* row_adapter;  // sorted row -> adapter
  const int32_t* vera_pos;     // sorted positions of the VeRA rows
  const RtChunk* chunks;
  const float* acc;            // [M_pad][AW] this forward's shrink sums
  const uint16_t* B_sh;        // [d_out][r_v]
  float* y;                    // [n][d_out] by token
  float* S;                    // [n][d_out] by sorted row (separate s pass)
  int32_t n, n_vera, AW, RT, r_v;
  int64_t d_out;
};

// thread t of the block: column blockIdx.x 256 + t over the chunk's rows;
// the rows' y values and shrink sums load before any is used
template <bool SCALE>
__global__ void __launch_bounds__(256) k_route_expand(RtArgs a) {
  constexpr int CH = 16;  // rows per chunk (at most)
  const RtChunk ch = a.chunks[blockIdx.y];
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (col >= a.d_out) return;
  const SlotEntry E = a.table[ch.a];
  const float sv = (SCALE && (E.flags & F_S)) ? E.s[col] : 1.f;
  const float bv = (E.flags & F_B) ? E.b[col] : 0.f;
  const int r = (E.flags & F_TERM) ? E.rank : 0;
  const uint16_t* Bc = (const uint16_t*)E.B + (size_t)col * r;  // B' row of this output
  // every load of the first 64 ranks goes out before the first is used: the
  // B' row, the rows' y values, then their shrink sums
  uint4 bq[8];
#pragma unroll
  for (int q = 0; q < 8; ++q)
    if (8 * q < r) bq[q] = ldg16(Bc + 8 * q);
  float yv[CH];
  size_t yo[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i)
    if (i < ch.n) {
      yo[i] = (size_t)a.perm[ch.p0 + i] * a.d_out + col;
      yv[i] = a.y[yo[i]];
    }
#pragma unroll
  for (int i = 0; i < CH; ++i)
    if (i < ch.n) yv[i] = (SCALE ? yv[i] * sv : yv[i]) + bv;
  for (int k0 = 0; k0 < r; k0 += 64) {
    if (k0 > 0)
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (k0 + 8 * q < r) bq[q] = ldg16(Bc + k0 + 8 * q);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (k0 + 8 * q < r) {
        const uint32_t w[4] = {bq[q].x, bq[q].y, bq[q].z, bq[q].w};
        float bf[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf[2 * j] = __uint_as_float(w[j] << 16);
          bf[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
#pragma unroll
        for (int i = 0; i < CH; ++i)
          if (i < ch.n) {
            const f32x4* tp = reinterpret_cast<const f32x4*>(a.acc + (size_t)(ch.p0 + i) * a.AW + k0 + 8 * q);
            const f32x4 t0 = tp[0], t1 = tp[1];
            yv[i] += t0[0] * bf[0] + t0[1] * bf[1] + t0[2] * bf[2] + t0[3] * bf[3] +
                     t1[0] * bf[4] + t1[1] * bf[5] + t1[2] * bf[6] + t1[3] * bf[7];
          }
      }
  }
#pragma unroll
  for (int i = 0; i < CH; ++i)
    if (i < ch.n) a.y[yo[i]] = yv[i];
}

// One work-group of 4 waves per 32 output columns and 32 VeRA rows (grid:
// d_out / 32 column tiles x VeRA row blocks) on 32x32x16 bf16 MFMA with B_sh
// as the A operand (lane (m, h): B_sh row c0 + m, ranks k + 8 h .. + 7, one
// 16-byte load) and the rows' u (already scaled by d, rounded to bf16) as
// the B operand. Wave w takes the 16-rank steps w, w + 4, .. (all its loads
// issued together), and the four partial tiles are added in wave order
// through LDS. Accumulator element i of lane (m, h): VeRA row v0 + m, output
// c0 + 8 (i / 4) + 4 h + i % 4; y += e (.) that, for the row's adapter's e.
__global__ void __launch_bounds__(256) k_route_vera(RtArgs a) {
  __shared__ float red[3][16][64];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, m = lane & 31, h = lane >> 5;
  const int64_t c0 = (int64_t)blockIdx.x * 32;
  const int v0 = blockIdx.y * 32;
  const bool vrow = v0 + m < a.n_vera;
  const int p = vrow ? a.vera_pos[v0 + m] : 0;
  const rsrc_t bs = make_rsrc(a.B_sh, (uint32_t)((int64_t)a.d_out * a.r_v * 2));
  const float* up = a.acc + (size_t)p * a.AW + a.RT;
  const int nks = a.r_v / 16;
  f32x16 acc = {};
  for (int j0 = w; j0 < nks; j0 += 16) {
    uint4 bq[4];
    f32x4 u0[4], u1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j0 + 4 * j < nks) {
        const int k = 16 * (j0 + 4 * j) + 8 * h;
        bq[j] = ldb16(bs, (uint32_t)(((c0 + m) * a.r_v + k) * 2));
        if (vrow) {
          u0[j] = ldg4(up + k);
          u1[j] = ldg4(up + k + 4);
        }
      }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j0 + 4 * j < nks) {
        uint4 uq = make_uint4(0, 0, 0, 0);
        if (vrow)
          uq = make_uint4(pack_bf2(__float_as_uint(u0[j][0]), __float_as_uint(u0[j][1])),
                          pack_bf2(__float_as_uint(u0[j][2]), __float_as_uint(u0[j][3])),
                          pack_bf2(__float_as_uint(u1[j][0]), __float_as_uint(u1[j][1])),
                          pack_bf2(__float_as_uint(u1[j][2]), __float_as_uint(u1[j][3])));
        acc = mfma32(bq[j], uq, acc);
      }
  }
  if (w > 0)
#pragma unroll
    for (int i = 0; i < 16; ++i) red[w - 1][i][lane] = acc[i];
  lds_barrier();
  if (w > 0 || !vrow) return;
#pragma unroll
  for (int q = 1; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] += red[q - 1][i][lane];
  const SlotEntry E = a.table[a.row_adapter[p]];
  float* yr = a.y + (size_t)a.perm[p] * a.d_out;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t f = c0 + 8 * q + 4 * h;
    if (f < a.d_out) {
      const f32x4 e = ldg4(E.ve + f);
      const f32x4 v = {acc[4 * q] * e[0], acc[4 * q + 1] * e[1], acc[4 * q + 2] * e[2], acc[4 * q + 3] * e[3]};
      stg4(yr + f, ldg4(yr + f) + v);
    }
  }
}

// 4 columns per thread
__global__ void __launch_bounds__(256) k_route_s_copy(RtArgs a) {
  const int p = blockIdx.y;
  const int64_t c4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (c4 >= a.d_out) return;
  const int32_t ad = a.row_adapter[p];
  f32x4 v = {1.f, 1.f, 1.f, 1.f};
  if (ad >= 0) {
    const SlotEntry E = a.table[ad];
    if (E.flags & F_S) v = ldg4(E.s + c4);
  }
  stg4(a.S + (size_t)p * a.d_out + c4, v);
}

__global__ void __launch_bounds__(256) k_route_s_mul(RtArgs a) {
  const int p = blockIdx.y;
  const int64_t c4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (c4 >= a.d_out) return;
  float* yp = a.y + (size_t)a.perm[p] * a.d_out + c4;
  stg4(yp, ldg4(yp) * ldg4(a.S + (size_t)p * a.d_out + c4));
}

}  // namespace

int32_t decode_route_launches(const scute_batch* B) {
  const DecodePlan& D = B->dp;
  int32_t nl = 0;
  if ((D.route & SCUTE_PLAN_ROUTE_ROTATE_PASS) && D.n_rot_items > 0) ++nl;
  if (D.route & SCUTE_PLAN_ROUTE_SEPARATE_S) nl += 2;
  if ((D.route & SCUTE_PLAN_ROUTE_EXPAND_PASS) && D.n_chunks > 0) ++nl;
  if ((D.route & (SCUTE_PLAN_ROUTE_EXPAND_PASS | SCUTE_PLAN_ROUTE_VERA_PASS)) && B->n_vera > 0) ++nl;
  return nl;
}

scute_status launch_route_rotate(scute_layer* L, const scute_batch* B, const void* x, hipStream_t st,
                                 int32_t* nl) {
  const DecodePlan& D = B->dp;
  if (!(D.route & SCUTE_PLAN_ROUTE_ROTATE_PASS) || D.n_rot_items == 0) return SCUTE_OK;
  ProfScope ps(L, st, "route_rotate");
  scute_status s = launch_rotate_items(D.rot, D.n_rot_items, D.rot_blk, (const uint16_t*)x,
                                       D.xs + (size_t)D.M_pad * L->d_in, (int32_t)L->d_in, st);
  if (s == SCUTE_OK) ++*nl;
  return s;
}

scute_status launch_route_passes(scute_layer* L, const scute_batch* B, float* y, const float* acc,
                                 hipStream_t st, int32_t* nl) {
  const DecodePlan& D = B->dp;
  const uint32_t R = D.route;
  if (!(R & (SCUTE_PLAN_ROUTE_EXPAND_PASS | SCUTE_PLAN_ROUTE_VERA_PASS))) return SCUTE_OK;
  RtArgs a{};
  a.table = L->table_dev;
  a.perm = B->d_perm;
  a.row_adapter = B->d_row_adapter;
  a.vera_pos = B->d_vera_pos;
  a.chunks = D.chunks;
  a.acc = acc;
  a.B_sh = (const uint16_t*)L->B_sh;
  a.y = y;
  a.S = D.S_rows;
  a.n = B->n;
  a.n_vera = B->n_vera;
  a.AW = D.AW;
  a.RT = D.RT;
  a.r_v = L->r_v;
  a.d_out = L->d_out;
  const unsigned cols4 = (unsigned)((L->d_out / 4 + 255) / 256);
  if (R & SCUTE_PLAN_ROUTE_SEPARATE_S) {
    if (!a.S) return fail(SCUTE_E_STATE, "route: separate-s buffer missing");
    {
      ProfScope ps(L, st, "route_s_copy");
      hipLaunchKernelGGL(k_route_s_copy, dim3(cols4, B->n), dim3(256), 0, st, a);
    }
    {
      ProfScope ps(L, st, "route_s_mul");
      hipLaunchKernelGGL(k_route_s_mul, dim3(cols4, B->n), dim3(256), 0, st, a);
    }
    *nl += 2;
  }
  if ((R & SCUTE_PLAN_ROUTE_EXPAND_PASS) && D.n_chunks > 0) {
    ProfScope ps(L, st, "route_expand");
    const dim3 g((unsigned)((L->d_out + 255) / 256), D.n_chunks);
    if (R & SCUTE_PLAN_ROUTE_SEPARATE_S)
      hipLaunchKernelGGL(k_route_expand<false>, g, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(k_route_expand<true>, g, dim3(256), 0, st, a);
    ++*nl;
  }
  if (B->n_vera > 0) {
    if (!a.B_sh || !a.vera_pos) return fail(SCUTE_E_STATE, "route: VeRA tables missing");
    ProfScope ps(L, st, "route_vera");
    hipLaunchKernelGGL(k_route_vera, dim3((unsigned)((L->d_out + 31) / 32), (B->n_vera + 31) / 32), dim3(256), 0,
                       st, a);
    ++*nl;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch route passes");
  return SCUTE_OK;
}

}  // namespace scute
