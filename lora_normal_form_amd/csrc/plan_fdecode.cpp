// Tables of the fused MFMA decode path (bf16, up to 256 rows per batch).
//
// The base GEMM y = (x W + delta W) (.) s + b is cut into 128-output column
// tiles and S slices of the K dimension, one work-group each; the slices of
// a tile meet per 32x32 piece in a workspace (the last slice to arrive at a
// piece adds all of them in slice order). The low-rank terms: the expand
// works on tiles that each belong to one adapter and VeRA's shared B is
// applied to every VeRA row of the batch at once ("Where is the cheapest
// place to compute the remaining slots?", paper-daily.com explainer of
// "Scute: Exact Batched Serving for PEFT Adapters Beyond LoRA"). Own-term
// expand steps of 16 ranks (one adapter segment's rows within one row group)
// are listed per row group for the wave that finishes the group's piece; the
// VeRA term's r_v / 16 rank steps apply to every row group holding VeRA rows.
// The shrinks are cut into blocks of 32 rank rows (A' rows of the adapters
// with rows in one row group, or A_sh rows for one group holding VeRA rows)
// that ride on the GEMM's K loop, one per wave; the rotation items (4 rows x
// 512 or 256 columns) are listed with every pointer and token resolved.

#include <string.h>

#include <algorithm>

#include "internal.h"

namespace scute {

namespace {

size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

}  // namespace

scute_status build_fdecode_plan(const scute_layer* L, scute_batch* B, hipStream_t st) {
  FdPlan& F = B->fp;
  F = FdPlan{};
  const int32_t n = B->n;
  const int64_t d_in = L->d_in, d_out = L->d_out;
  // the fused path: SCUTE_DECODE=1, or any decode path mode (not 0) when the
  // plan asks for bit-repeatable forwards
  // (SCUTE_DECODE unset: -1, the choice below)
  const int mode = env_int("SCUTE_DECODE", -1);
  const bool det = (B->flags & SCUTE_PLAN_DETERMINISTIC) != 0;
  if (mode == 0 || (mode != 1 && mode != -1 && !det)) return SCUTE_OK;
  if (L->act != SCUTE_BF16 || n <= 0 || n > 256) return SCUTE_OK;
  // rows that rotate per projection take the two-launch decode path or the
  // generic kernels
  if (B->rproj) return SCUTE_OK;
  if (d_in % 64 != 0 || d_out % 32 != 0) return SCUTE_OK;
  // W, x and every workspace are addressed through buffer ranges with
  // 32-bit offsets
  if (d_in * d_out * 2 >= ((int64_t)1 << 32) || (int64_t)n * d_in * 2 >= ((int64_t)1 << 31)) return SCUTE_OK;
  if (B->n_vera > 0 && (L->r_v % 32 != 0 || d_in % 256 != 0)) return SCUTE_OK;
  for (int32_t i = 0; i < B->nseg(); ++i) {
    const SlotEntry& E = L->table[B->seg[3 * i]];
    if ((E.flags & F_TERM) && (E.rank % 8 != 0)) return SCUTE_OK;
  }
  F.MG = (n + 31) / 32;
  F.g_rot = (B->n_rot + 31) / 32;
  F.MGT = F.MG + F.g_rot;
  if (F.MGT > 8) return SCUTE_OK;
  if (mode == -1 && !det) {
    // path unset: the fused path only for many staged row groups and no own
    // low-rank term (see FUSED_MIN_GROUPS)
    bool own = false;
    for (int32_t i = 0; i < B->nseg(); ++i) own |= (L->table[B->seg[3 * i]].flags & F_TERM) != 0;
    if (own || F.MGT < FUSED_MIN_GROUPS) {
      F = FdPlan{};
      return SCUTE_OK;
    }
  }
  F.M_pad = 32 * F.MG;
  F.RT = (B->max_rank + 15) / 16 * 16;
  F.AW = F.RT + (B->n_vera > 0 ? L->r_v : 0);
  F.C = (int32_t)((d_out + 127) / 128);
  // K slices: the most (up to 16) that keep one work-group per compute
  // unit and at least 4 stages of 64 k per slice
  const int32_t cu = L->num_cu > 0 ? L->num_cu : 256;
  int32_t S = 1;
  while (S < 16 && (int64_t)F.C * S * 2 <= cu && d_in % (64 * (int64_t)S * 2) == 0 &&
         d_in / (64 * (int64_t)S * 2) >= 4)
    S *= 2;
  S = env_int("SCUTE_FD_SPLITK", S);
  if (S < 1 || S > 64 || (S & (S - 1)) != 0 || d_in % (64 * (int64_t)S) != 0)
    return fail(SCUTE_E_INVALID, "bad SCUTE_FD_SPLITK (a power of two dividing d_in / 64)");
  F.S = S;
  F.NST = (int32_t)(d_in / 64 / S);

  // ---- rows ------------------------------------------------------------------
  struct RowRec {
    int32_t tok, src, flags;
    const float *s, *e, *b, *d;
    int32_t rank;
  };
  std::vector<RowRec> rr(F.M_pad);
  int32_t pmin = n, pmax = -1;
  for (int32_t p = 0; p < F.M_pad; ++p) {
    rr[p] = RowRec{p < n ? B->perm[p] : -1, B->perm[std::min(p, n - 1)], 0,
                   nullptr, nullptr, nullptr, nullptr, 0};
    if (p >= n) continue;
    const int32_t a = B->row_adapter[p];
    if (a < 0) continue;
    const SlotEntry& E = L->table[a];
    if (E.flags & F_TERM) rr[p].rank = E.rank;
    if (E.flags & F_S) {
      rr[p].s = E.s;
      rr[p].flags |= FR_S;
    }
    if (E.flags & F_B) {
      rr[p].b = E.b;
      rr[p].flags |= FR_B;
    }
    if (E.flags & F_VERA) {
      rr[p].e = E.ve;
      rr[p].d = E.vd;
      rr[p].flags |= FR_E | FR_VERA;
      pmin = std::min(pmin, p);
      pmax = std::max(pmax, p);
    }
  }
  if (pmax >= 0) {
    F.gv0 = pmin / 32;
    F.gv1 = pmax / 32 + 1;
  }

  // ---- own-term expand steps by row group; shrink blocks -------------------------
  // An adapter's rows are one segment of the sorted order; the part of it in
  // row group g needs the adapter's ranks in g: one expand step per 16
  // ranks, and its rank rows in a shrink block of group g.
  std::vector<std::vector<FdStep>> per(F.MG);
  std::vector<FdXBlock> xbs;
  std::vector<int32_t> xoff;
  for (int32_t g = 0; g < F.MG; ++g) {
    xoff.push_back((int32_t)xbs.size());
    FdXBlock cur{};
    int32_t fill = 0;
    auto flush = [&]() {
      if (fill == 0) return;
      for (int32_t mm = fill; mm < 32; ++mm) {
        cur.arow[mm] = nullptr;
        cur.col[mm] = -1;
        cur.lohi[mm] = 0;
      }
      cur.g = g;
      cur.vera = 0;
      xbs.push_back(cur);
      cur = FdXBlock{};
      fill = 0;
    };
    for (int32_t i = 0; i < B->nseg(); ++i) {
      const int32_t a = B->seg[3 * i], start = B->seg[3 * i + 1], len = B->seg[3 * i + 2];
      const SlotEntry& E = L->table[a];
      if (!(E.flags & F_TERM)) continue;
      const int32_t lo = std::max(start, 32 * g), hi = std::min(start + len, 32 * g + 32);
      if (lo >= hi) continue;
      for (int32_t kk = 0; kk < E.rank; kk += 16) {
        FdStep st{};
        st.kk = kk;
        st.rank = E.rank;
        st.lo = lo;
        st.hi = hi;
        st.bp = (const uint16_t*)E.B;
        st.g = g;
        per[g].push_back(st);
      }
      // the adapter's rank rows (a multiple of 8) start at a multiple of 8
      // within the block, so every run of 4 belongs to one adapter
      for (int32_t r = 0; r < E.rank; ++r) {
        cur.arow[fill] = (const uint16_t*)E.A + (size_t)r * d_in;
        cur.col[fill] = r;
        cur.lohi[fill] = lo | (hi << 16);
        if (++fill == 32) flush();
      }
    }
    flush();
    if (B->n_vera > 0 && g >= F.gv0 && g < F.gv1)
      for (int32_t j0 = 0; j0 < L->r_v; j0 += 32) {
        FdXBlock xb{};
        for (int32_t mm = 0; mm < 32; ++mm) {
          xb.arow[mm] = (const uint16_t*)L->A_sh + (size_t)(j0 + mm) * d_in;
          xb.col[mm] = F.RT + j0 + mm;
          xb.lohi[mm] = 0;
        }
        xb.g = g;
        xb.vera = 1;
        xbs.push_back(xb);
      }
  }
  xoff.push_back((int32_t)xbs.size());
  // one block per wave, spread over the column tiles first; when the tiles
  // of d_out have too few waves, the grid gets extra tiles past d_out that
  // carry shrink blocks only (their W rows read as zero without a memory
  // access). The grid stays within one work-group per compute unit, so the
  // finishing waves' wait for the shrink blocks always ends.
  F.n_xb = (int32_t)xbs.size();
  F.CG = std::max<int32_t>(F.C, (F.n_xb + 3) / 4);
  if ((int64_t)F.CG * S > cu) {
    F = FdPlan{};
    return SCUTE_OK;
  }
  std::vector<FdStep> steps;
  std::vector<int32_t> goff;
  for (int32_t g = 0; g < F.MG; ++g) {
    goff.push_back((int32_t)steps.size());
    steps.insert(steps.end(), per[g].begin(), per[g].end());
  }
  goff.push_back((int32_t)steps.size());

  // ---- rotation items ------------------------------------------------------------
  std::vector<FdRotItem> rot;
  int32_t blk0 = -1;
  for (int32_t i = 0; i < B->nseg(); ++i) {
    const SlotEntry& E = L->table[B->seg[3 * i]];
    if (!(E.flags & F_R)) continue;
    blk0 = blk0 == -1 ? E.blk : (blk0 == E.blk ? blk0 : 0);
  }
  F.rot_blk = (blk0 == 8 || blk0 == 16 || blk0 == 32 || blk0 == 64) ? blk0 : 0;
  F.rot_cols = F.rot_blk == 64 ? 256 : 512;
  for (int32_t i = 0; i < B->nseg(); ++i) {
    const int32_t a = B->seg[3 * i], start = B->seg[3 * i + 1], len = B->seg[3 * i + 2];
    const SlotEntry& E = L->table[a];
    if (!(E.flags & F_R)) continue;
    for (int32_t r0 = 0; r0 < len; r0 += 4)
      for (int64_t c0 = 0; c0 < d_in; c0 += F.rot_cols) {
        FdRotItem it{};
        it.p0 = start + r0;
        it.n = std::min(4, len - r0);
        it.c0 = (int32_t)c0;
        it.blk = E.blk;
        for (int32_t r = 0; r < 4; ++r) it.tok[r] = B->perm[it.p0 + std::min(r, it.n - 1)];
        it.P = (const uint16_t*)E.P;
        rot.push_back(it);
      }
  }
  F.n_rot_items = (int32_t)rot.size();

  // ---- one device allocation: tables, then zeroed workspaces -------------------
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t r = o;
    o += al256(bytes);
    return r;
  };
  const size_t o_rows = take(sizeof(FdRow) * (size_t)F.M_pad);
  const size_t o_steps = take(sizeof(FdStep) * steps.size() + 16);
  const size_t o_goff = take(4 * goff.size());
  const size_t o_xoff = take(4 * xoff.size());
  const size_t o_xb = take(sizeof(FdXBlock) * xbs.size() + 16);
  const size_t o_rot = take(sizeof(FdRotItem) * rot.size() + 16);
  const size_t o_ones = take(4 * (size_t)d_out);
  const size_t tables = o;
  const size_t o_zeros = take(4 * (size_t)std::max<int64_t>(d_out, L->r_v));
  const size_t acc_bytes = 2 * (size_t)F.M_pad * std::max<int32_t>(F.AW, 8);
  const size_t part_bytes = S > 1 ? (size_t)F.C * S * F.MG * 4 * 4096 : 0;
  const size_t xpart_bytes = (size_t)F.n_xb * S * 4096;
  if (part_bytes >= ((size_t)1 << 31) || acc_bytes >= ((size_t)1 << 31) ||
      xpart_bytes >= ((size_t)1 << 31)) {
    F = FdPlan{};
    return SCUTE_OK;
  }
  const size_t o_acc = take(acc_bytes);
  const size_t o_xpart = take(xpart_bytes);
  const size_t o_xcnt = take(4 * (size_t)F.n_xb + 4);
  const size_t o_xdone = take(4 * (size_t)F.n_xb + 4);
  const size_t o_part = take(part_bytes);
  const size_t o_cnt = take(4 * (size_t)F.C * F.MG * 4);
  const size_t o_err = take(4);
  const size_t total = o;

  hipError_t e = hipMalloc(&B->fd_dev, total);
  if (e != hipSuccess) return hip_fail(e, "hipMalloc(fused decode plan)");
  uint8_t* d = (uint8_t*)B->fd_dev;
  const float* ones = (const float*)(d + o_ones);
  const float* zeros = (const float*)(d + o_zeros);
  std::vector<FdRow> rows(F.M_pad);
  for (int32_t p = 0; p < F.M_pad; ++p)
    rows[p] = FdRow{rr[p].s ? rr[p].s : ones, rr[p].e ? rr[p].e : ones, rr[p].b ? rr[p].b : zeros,
                    rr[p].d ? rr[p].d : zeros, rr[p].tok, rr[p].src, rr[p].flags, rr[p].rank};

  std::vector<uint8_t> h(tables, 0);
  memcpy(h.data() + o_rows, rows.data(), sizeof(FdRow) * rows.size());
  if (!steps.empty()) memcpy(h.data() + o_steps, steps.data(), sizeof(FdStep) * steps.size());
  memcpy(h.data() + o_goff, goff.data(), 4 * goff.size());
  memcpy(h.data() + o_xoff, xoff.data(), 4 * xoff.size());
  if (!xbs.empty()) memcpy(h.data() + o_xb, xbs.data(), sizeof(FdXBlock) * xbs.size());
  if (!rot.empty()) memcpy(h.data() + o_rot, rot.data(), sizeof(FdRotItem) * rot.size());
  for (int64_t j = 0; j < d_out; ++j) {
    const float one = 1.0f;
    memcpy(h.data() + o_ones + 4 * j, &one, 4);
  }
  // workspaces start at zero: the shrink sums, the arrival counters (which
  // then only grow: a slice is last at a piece or block when its arrival
  // makes the count a multiple of S), the blocks' forward numbers and the
  // error flag
  e = hipMemsetAsync(d + tables, 0, total - tables, st);
  if (e == hipSuccess) e = hipMemcpyAsync(d, h.data(), tables, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    (void)hipFree(B->fd_dev);
    B->fd_dev = nullptr;
    F = FdPlan{};
    return hip_fail(e, "upload fused decode plan");
  }
  F.rows = (const FdRow*)(d + o_rows);
  F.steps = (const FdStep*)(d + o_steps);
  F.goff = (const int32_t*)(d + o_goff);
  F.xb = (const FdXBlock*)(d + o_xb);
  F.rot = (const FdRotItem*)(d + o_rot);
  F.xoff = (const int32_t*)(d + o_xoff);
  F.acc = (uint16_t*)(d + o_acc);
  F.xpart = (float*)(d + o_xpart);
  F.xcnt = (int32_t*)(d + o_xcnt);
  F.xdone = (uint32_t*)(d + o_xdone);
  F.xpart_bytes = (uint32_t)xpart_bytes;
  F.part = S > 1 ? (float*)(d + o_part) : nullptr;
  F.cnt = (int32_t*)(d + o_cnt);
  F.err = (int32_t*)(d + o_err);
  F.acc_bytes = (uint32_t)acc_bytes;
  F.part_bytes = (uint32_t)part_bytes;
  F.fwd = 0;
  // SCUTE_FD_FORCE_WAIT_FAIL=1 (tests of the failure report): every wait
  // looks for a forward number no arrival reaches and gives up after a few
  // polls, so each wave still finishes; the output of such a forward is not
  // valid and scute_batch_wait_failures reports it
  if (env_int("SCUTE_FD_FORCE_WAIT_FAIL", 0) == 1) {
    F.spin_limit = 16;
    F.wait_bias = 1;
  }
  F.enabled = true;
  return SCUTE_OK;
}

}  // namespace scute
