// Tables of the MFMA decode path (bf16, up to 256 rows per batch).
//
// The base GEMM y = (x W + delta W) (.) s + b is split into column tiles of
// 64 outputs and S slices of the K dimension; the last slice of a tile to
// finish adds the others' partial tiles (kept in a workspace) and writes y
// once. The low-rank work of the expand step ("Where is the cheapest place
// to compute the remaining slots?", paper-daily.com explainer of "Scute:
// Exact Batched Serving for PEFT Adapters Beyond LoRA": the expand works on
// tiles that each belong to one adapter; VeRA's shared B is applied to every
// VeRA row of the batch at once) is cut into items of up to four 16-rank
// MFMA steps:
//   own item   (row group g, adapter segment, 64 ranks) against B'
//   VeRA item  (row group g, 64 ranks) against the shared B_sh
// Each K slice of a tile takes a share of both kinds, split between its two
// K-half waves of each column block, and every item becomes a list of 16-rank
// steps that the wave walks in batches.
// The prologue items (gather of the sorted x rows, rotation, own-term
// shrink, VeRA shrink) are listed here too, with every pointer and token
// resolved; see decode.hip for the kernels.

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

scute_status build_decode_plan(const scute_layer* L, scute_batch* B, hipStream_t st) {
  DecodePlan& D = B->dp;
  D = DecodePlan{};
  const int32_t n = B->n;
  const int64_t d_in = L->d_in, d_out = L->d_out;
  // the two-launch decode path (gather / rotation / shrink prologue, then
  // the GEMM): SCUTE_DECODE=2
  // (route variants always plan here)
  const uint32_t route = B->flags & ROUTE_MASK;
  if (!route && (env_int("SCUTE_DECODE", DECODE_DEFAULT) != 2 || (B->flags & SCUTE_PLAN_DETERMINISTIC)))
    return SCUTE_OK;
  const bool rot_in_pro = !(route & SCUTE_PLAN_ROUTE_ROTATE_PASS);
  const bool own_fused = !(route & SCUTE_PLAN_ROUTE_EXPAND_PASS);
  const bool vera_fused = !(route & (SCUTE_PLAN_ROUTE_EXPAND_PASS | SCUTE_PLAN_ROUTE_VERA_PASS));
  if (L->act != SCUTE_BF16 || n <= 0 || n > 256) return SCUTE_OK;
  // the route variants' rotation pass has one delta block
  if (B->rproj && route) return SCUTE_OK;
  // K parts of the shrinks: at most 8 of 1024 (own) and 16 of 512 (VeRA)
  if (d_in % 128 != 0 || d_in > 8192 || d_out % 64 != 0) return SCUTE_OK;
  // W is addressed through a buffer range with 32-bit offsets
  if (d_in * d_out * 2 >= ((int64_t)1 << 32)) return SCUTE_OK;
  if (B->n_vera > 0 && (L->r_v % 32 != 0 || d_in % 256 != 0)) return SCUTE_OK;
  for (int32_t i = 0; i < B->nseg(); ++i) {
    const SlotEntry& E = L->table[B->seg[3 * i]];
    if ((E.flags & F_TERM) && (E.rank % 8 != 0)) return SCUTE_OK;
  }

  D.MG = (n + 31) / 32;
  D.g_rot = (B->n_rot + 31) / 32;
  // two staged groups compile badly (accumulator copies); pad with one row
  // group of unused rows instead
  if (D.MG + D.g_rot == 2) D.MG += 1;
  if (D.MG + D.g_rot > 9) {  // LDS: two ring slots of 32 (MG + g_rot) rows x 256 B + row records
    D = DecodePlan{};
    return SCUTE_OK;
  }
  D.M_pad = 32 * D.MG;
  // rows that rotate per projection: one block of delta rows per projection,
  // and each column tile stages its projection's block (projection ends are
  // multiples of 64, so a tile lies in one projection)
  D.np = B->rproj ? L->n_proj : 1;
  for (int32_t i = 0; i + 1 < MAX_PROJ; ++i)
    D.ptile[i] = i + 1 < D.np ? (int32_t)(L->proj_end[i] / 64) : (int32_t)(d_out / 64);
  D.RT = (B->max_rank + 15) / 16 * 16;
  D.C = (int32_t)(d_out / 64);
  // K slices: none when the column tiles alone nearly fill the chip (every
  // slice costs a partial tile in the workspace); otherwise the fewest (up
  // to 4) that reach one work-group per compute unit. Each slice is split in
  // two K halves of 64-wide stages.
  const int32_t cu = L->num_cu > 0 ? L->num_cu : 256;
  int32_t S = 1;
  if ((int64_t)D.C * 4 < (int64_t)cu * 3)
    while (S < 4 && (int64_t)D.C * S < cu && d_in % ((int64_t)S * 2 * 128) == 0) S *= 2;
  S = env_int("SCUTE_DECODE_SPLITK", S);
  if ((S != 1 && S != 2 && S != 4) || d_in % ((int64_t)S * 128) != 0)
    return fail(SCUTE_E_INVALID, "bad SCUTE_DECODE_SPLITK (1, 2 or 4 dividing d_in / 128)");
  D.S = S;
  D.k_chunk = (int32_t)(d_in / S);

  // ---- counts that size the tables ------------------------------------------
  int32_t n_rot_items = 0, n_sgroups = 0, nvb = 0, njb = 0, SV = 0;
  for (int32_t i = 0; i < B->nseg(); ++i) {
    const int32_t a = B->seg[3 * i], len = B->seg[3 * i + 2];
    const SlotEntry& E = L->table[a];
    if ((E.flags & F_R) && rot_in_pro) n_rot_items += D.np * ((len + 3) / 4) * (int32_t)(d_in / 64);
    if (E.flags & F_TERM) n_sgroups += (len + 3) / 4 * ((E.rank + 3) / 4);
  }
  const int32_t KQ = (int32_t)((d_in + 1023) / 1024);
  if (B->n_vera > 0) {
    nvb = (B->n_vera + 31) / 32;
    njb = L->r_v / 32;
    SV = (int32_t)(d_in / 256);
  }
  const int32_t n_gather = n;
  const int32_t n_pro = n_gather + n_rot_items + KQ * n_sgroups + SV * nvb * njb;
  D.AW = D.RT + (B->n_vera > 0 ? L->r_v : 0);

  // ---- expand steps -----------------------------------------------------------
  // item: the steps of one row group's term over up to 64 ranks (own: one
  // adapter segment's rows of the group against its B'; VeRA: the group's
  // VeRA rows against B_sh)
  struct Item {
    int32_t g, kind, k, nst, rank, lo, hi;
    const uint16_t* ptr;
  };
  std::vector<Item> own_items, vera_items;
  std::vector<int32_t> row_vera(D.M_pad, 0);
  for (int32_t p = 0; p < n; ++p) {
    const int32_t a = B->row_adapter[p];
    if (a >= 0 && (L->table[a].flags & F_VERA)) row_vera[p] = 1;
  }
  for (int32_t i = 0; i < B->nseg(); ++i) {
    const int32_t a = B->seg[3 * i], start = B->seg[3 * i + 1], len = B->seg[3 * i + 2];
    const SlotEntry& E = L->table[a];
    if (!(E.flags & F_TERM) || !own_fused) continue;
    for (int32_t g = start / 32; g * 32 < start + len; ++g) {
      const int32_t lo = std::max(start, 32 * g), hi = std::min(start + len, 32 * g + 32);
      for (int32_t k = 0; k < E.rank; k += 64)
        own_items.push_back({g, 0, k, std::min(4, (E.rank - k + 15) / 16), E.rank, lo, hi,
                             (const uint16_t*)E.B});
    }
  }
  // The VeRA term can run dense when a slice has at most 256 ranks of it and
  // the VeRA rows' groups fit the LDS buffer the kernel stages them in, 128
  // ranks at a time (32 (gv1 - gv0) rows of 256 bytes, at most 256 rows).
  if (B->n_vera > 0 && vera_fused) {
    int32_t pmin = n, pmax = -1;
    for (int32_t v : B->vera_pos) {
      pmin = std::min(pmin, v);
      pmax = std::max(pmax, v);
    }
    const int32_t gv0 = pmin / 32, gv1 = pmax / 32 + 1;
    const int32_t nks = L->r_v / 16, nkmax = (nks + S - 1) / S;
    const int32_t rows = 32 * (gv1 - gv0);
    const int64_t slot_bytes = (int64_t)8192 * (D.MG + D.g_rot);
    // worth it once a slice has 16 or more VeRA rank steps (otherwise the
    // steps take about one batch); SCUTE_DECODE_DENSE_VERA=1 / 0 forces it
    // on (where it fits) / off
    const int32_t mode = env_int("SCUTE_DECODE_DENSE_VERA", -1);
    const bool fits = nkmax <= 16 && rows <= 256 && (int64_t)rows * 256 <= slot_bytes;
    if (fits && (mode == 1 || (mode == -1 && (gv1 - gv0) * nkmax >= 16))) {
      D.gv0 = gv0;
      D.gv1 = gv1;
    }
  }
  if (B->n_vera > 0 && vera_fused && D.gv1 == D.gv0) {
    for (int32_t g = 0; g < D.MG; ++g) {
      bool any = false;
      for (int32_t p = 32 * g; p < std::min(n, 32 * g + 32); ++p) any |= row_vera[p] != 0;
      if (!any) continue;
      for (int32_t k = 0; k < L->r_v; k += 64)
        vera_items.push_back({g, STEP_VERA, k, std::min(4, (L->r_v - k) / 16), L->r_v, 32 * g,
                              32 * g + 32, (const uint16_t*)L->B_sh});
    }
  }
  // Each row group's items spread over the S slices, largest first, each to
  // the slice with the fewest of the group's steps so far. In the main
  // kernel one wave runs a group's steps of its slice: the own items' steps,
  // then the VeRA items' steps.
  const int32_t MG = D.MG;
  std::vector<std::vector<Item>> per((size_t)S * MG * 2);  // [(k MG + g) 2 + vera]
  for (int32_t g = 0; g < MG; ++g) {
    std::vector<Item> items;
    for (const Item& it : own_items)
      if (it.g == g) items.push_back(it);
    for (const Item& it : vera_items)
      if (it.g == g) items.push_back(it);
    std::stable_sort(items.begin(), items.end(),
                     [](const Item& p, const Item& q) { return p.nst > q.nst; });
    std::vector<int64_t> load(S, 0);
    for (const Item& it : items) {
      const int32_t k = (int32_t)(std::min_element(load.begin(), load.end()) - load.begin());
      per[((size_t)k * MG + g) * 2 + (it.kind == STEP_VERA ? 1 : 0)].push_back(it);
      load[k] += it.nst;
    }
  }
  std::vector<DecStep> steps;
  std::vector<int32_t> goff;
  for (size_t q = 0; q < per.size(); ++q) {
    goff.push_back((int32_t)steps.size());
    for (const Item& it : per[q])
      for (int32_t st = 0; st < it.nst; ++st) {
        DecStep d{};
        d.gk = it.kind | (it.g << 8);
        d.kk = it.k + 16 * st;
        d.rank = it.rank;
        d.lohi = it.lo | (it.hi << 16);
        d.bp = it.ptr;
        steps.push_back(d);
      }
  }
  goff.push_back((int32_t)steps.size());
  D.n_steps = (int32_t)steps.size();

  // ---- one device allocation: tables, then zeroed workspaces -------------------
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t r = o;
    o += al256(bytes);
    return r;
  };
  const size_t o_rows = take(sizeof(DecRow) * (size_t)D.M_pad);
  const size_t o_pro = take(sizeof(DecProItem) * (size_t)n_pro + 16);
  const size_t o_vrows = take(sizeof(DecVeraRow) * 32 * (size_t)nvb + 16);
  const size_t o_steps = take(sizeof(DecStep) * steps.size() + 16);
  const size_t o_goff = take(sizeof(int32_t) * goff.size());
  const size_t o_ones = take(4 * (size_t)d_out);
  // route tables: rotation pass items, expand pass chunks
  std::vector<FdRotItem> rot;
  std::vector<RtChunk> chunks;
  int32_t rot_blk = -1;
  for (int32_t i = 0; i < B->nseg(); ++i) {
    const int32_t a = B->seg[3 * i], start = B->seg[3 * i + 1], len = B->seg[3 * i + 2];
    const SlotEntry& E = L->table[a];
    if ((E.flags & F_R) && !rot_in_pro) rot_blk = rot_blk == -1 ? E.blk : (rot_blk == E.blk ? rot_blk : 0);
    const bool exp_rows = (route & SCUTE_PLAN_ROUTE_EXPAND_PASS) &&
                          ((E.flags & (F_B | F_TERM)) ||
                           ((E.flags & F_S) && !(route & SCUTE_PLAN_ROUTE_SEPARATE_S)));
    if (exp_rows)
      for (int32_t r0 = 0; r0 < len; r0 += 16) chunks.push_back(RtChunk{start + r0, std::min(16, len - r0), a, 0});
  }
  if (rot_blk != 8 && rot_blk != 16 && rot_blk != 32 && rot_blk != 64) rot_blk = 0;
  const int64_t rot_cols = rot_blk == 64 ? 256 : 512;
  if (!rot_in_pro)
    for (int32_t i = 0; i < B->nseg(); ++i) {
      const int32_t a = B->seg[3 * i], start = B->seg[3 * i + 1], len = B->seg[3 * i + 2];
      const SlotEntry& E = L->table[a];
      if (!(E.flags & F_R)) continue;
      for (int32_t r0 = 0; r0 < len; r0 += 4)
        for (int64_t c0 = 0; c0 < d_in; c0 += rot_cols) {
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
  const size_t o_rot = take(sizeof(FdRotItem) * rot.size() + 16);
  const size_t o_chunks = take(sizeof(RtChunk) * chunks.size() + 16);
  const size_t tables = o;
  const size_t o_zeros = take(4 * (size_t)d_out);
  const size_t acc_bytes = 4 * (size_t)D.M_pad * D.AW;
  const size_t part_bytes = S > 1 ? 4 * (size_t)S * D.C * D.M_pad * 64 : 0;
  const size_t xs_bytes = 2 * (size_t)(D.M_pad + 32 * D.g_rot * D.np) * d_in;
  if (part_bytes >= ((size_t)1 << 31) || acc_bytes >= ((size_t)1 << 31)) {
    D = DecodePlan{};  // buffer offsets are 32-bit
    return SCUTE_OK;
  }
  const size_t o_xs = take(xs_bytes);
  const size_t o_acc0 = take(acc_bytes), o_acc1 = take(acc_bytes);
  const size_t o_part = take(part_bytes), o_cnt = take(4 * (size_t)D.C);
  const size_t o_srows = take((route & SCUTE_PLAN_ROUTE_SEPARATE_S) ? 4 * (size_t)n * d_out : 0);
  const size_t total = o;

  hipError_t e = hipMalloc(&B->fast_dev, total);
  if (e != hipSuccess) return hip_fail(e, "hipMalloc(decode plan)");
  uint8_t* d = (uint8_t*)B->fast_dev;
  const float* ones = (const float*)(d + o_ones);
  const float* zeros = (const float*)(d + o_zeros);

  // ---- per-row tables ----------------------------------------------------------
  std::vector<DecRow> rows(D.M_pad, DecRow{ones, ones, zeros, -1, 0});
  for (int32_t p = 0; p < n; ++p) {
    rows[p].tok = B->perm[p];
    const int32_t a = B->row_adapter[p];
    if (a < 0) continue;
    const SlotEntry& E = L->table[a];
    // (the expand pass route applies s and b after the GEMM; the VeRA pass
    // routes add the VeRA term after it)
    if ((E.flags & F_S) && own_fused) rows[p].s = E.s;
    if ((E.flags & F_B) && own_fused) rows[p].b = E.b;
    if ((E.flags & F_VERA) && vera_fused) {
      rows[p].e = E.ve;
      rows[p].flags = 1;
    }
  }

  // ---- prologue items -----------------------------------------------------------
  std::vector<DecProItem> pro;
  pro.reserve(n_pro);
  auto toks = [&](DecProItem& it) {
    for (int32_t r = 0; r < 4; ++r) it.tok[r] = B->perm[it.p0 + std::min(r, it.n - 1)];
  };
  for (int32_t p0 = 0; p0 < n; ++p0) {
    DecProItem it{};
    it.type = PRO_GATHER;
    it.p0 = p0;
    it.n = 1;
    toks(it);
    pro.push_back(it);
  }
  std::vector<DecProItem> shrink_groups;
  for (int32_t i = 0; i < B->nseg(); ++i) {
    const int32_t a = B->seg[3 * i], start = B->seg[3 * i + 1], len = B->seg[3 * i + 2];
    const SlotEntry& E = L->table[a];
    // (projection pj's delta rows start 32 g_rot pj rows after the first
    // block; an adapter with one rotation uses it for every projection)
    if ((E.flags & F_R) && rot_in_pro)
      for (int32_t pj = 0; pj < D.np; ++pj)
        for (int32_t r0 = 0; r0 < len; r0 += 4)
          for (int64_t c0 = 0; c0 < d_in; c0 += 64) {
            DecProItem it{};
            it.type = PRO_ROT;
            it.p0 = start + r0;
            it.n = std::min(4, len - r0);
            it.k = (int32_t)c0;
            toks(it);
            it.p0 += 32 * D.g_rot * pj;
            it.ptr = (const uint16_t*)E.P + ((E.flags & F_RPROJ) ? (size_t)pj * d_in * E.blk : 0);
            it.blk = E.blk;
            pro.push_back(it);
          }
    if (E.flags & F_TERM)
      for (int32_t r0 = 0; r0 < len; r0 += 4)
        for (int32_t k = 0; k < E.rank; k += 4) {
          DecProItem it{};
          it.type = PRO_SHRINK;
          it.p0 = start + r0;
          it.n = std::min(4, len - r0);
          it.k = k | (std::min(4, E.rank - k) << 16);
          toks(it);
          it.ptr = (const uint16_t*)E.A;
          shrink_groups.push_back(it);
        }
  }
  for (int32_t kq = 0; kq < KQ; ++kq)
    for (DecProItem it : shrink_groups) {
      it.blk = kq;
      pro.push_back(it);
    }
  std::vector<DecVeraRow> vrows;
  if (B->n_vera > 0) {
    for (int32_t kv = 0; kv < SV; ++kv)
      for (int32_t vb = 0; vb < nvb; ++vb)
        for (int32_t jb = 0; jb < njb; ++jb) {
          DecProItem it{};
          it.type = PRO_VSHRINK;
          it.p0 = vb;
          it.n = jb;
          it.k = kv;
          pro.push_back(it);
        }
    vrows.resize(32 * (size_t)nvb);
    for (size_t v = 0; v < vrows.size(); ++v) {
      const bool real = v < (size_t)B->n_vera;
      const int32_t p = B->vera_pos[real ? v : 0];
      vrows[v].vd = L->table[B->row_adapter[p]].vd;
      vrows[v].tok = B->perm[p];
      vrows[v].p = real ? p : -1;
    }
  }
  // heaviest items first: they start on separate compute units
  std::stable_sort(pro.begin(), pro.end(), [](const DecProItem& p, const DecProItem& q) {
    auto rank = [](int32_t t) { return t == PRO_VSHRINK ? 0 : t == PRO_SHRINK ? 1 : t == PRO_ROT ? 2 : 3; };
    return rank(p.type) < rank(q.type);
  });
  D.n_pro = (int32_t)pro.size();
  D.n_vitems = SV * nvb * njb;
  D.nvb = nvb;
  D.njb = njb;
  // the kernel derives a VeRA item's (kv, vb, jb) from its index
  bool order_ok = D.n_pro == n_pro;
  for (int32_t i = 0; order_ok && i < D.n_vitems; ++i) {
    const DecProItem& it = pro[i];
    order_ok = it.type == PRO_VSHRINK && it.k == i / (nvb * njb) && it.p0 == (i / njb) % nvb &&
               it.n == i % njb;
  }
  if (!order_ok) {
    (void)hipFree(B->fast_dev);
    B->fast_dev = nullptr;
    D = DecodePlan{};
    return fail(SCUTE_E_STATE, "decode plan: prologue item count mismatch");
  }

  std::vector<uint8_t> h(tables, 0);
  memcpy(h.data() + o_rows, rows.data(), sizeof(DecRow) * rows.size());
  if (!pro.empty()) memcpy(h.data() + o_pro, pro.data(), sizeof(DecProItem) * pro.size());
  if (!vrows.empty()) memcpy(h.data() + o_vrows, vrows.data(), sizeof(DecVeraRow) * vrows.size());
  if (!steps.empty()) memcpy(h.data() + o_steps, steps.data(), sizeof(DecStep) * steps.size());
  memcpy(h.data() + o_goff, goff.data(), sizeof(int32_t) * goff.size());
  if (!rot.empty()) memcpy(h.data() + o_rot, rot.data(), sizeof(FdRotItem) * rot.size());
  if (!chunks.empty()) memcpy(h.data() + o_chunks, chunks.data(), sizeof(RtChunk) * chunks.size());
  for (int64_t j = 0; j < d_out; ++j) {
    const float one = 1.0f;
    memcpy(h.data() + o_ones + 4 * j, &one, 4);
  }

  // workspaces start at zero: rows of xs past n and delta rows past n_rot
  // (staged but never written), both shrink sum buffers, and the arrival
  // counters
  e = hipMemsetAsync(d + tables, 0, total - tables, st);
  if (e == hipSuccess) e = hipMemcpyAsync(d, h.data(), tables, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    (void)hipFree(B->fast_dev);
    B->fast_dev = nullptr;
    D = DecodePlan{};
    return hip_fail(e, "upload decode plan");
  }
  D.rows = (const DecRow*)(d + o_rows);
  D.pro_items = (const DecProItem*)(d + o_pro);
  D.vrows = B->n_vera ? (const DecVeraRow*)(d + o_vrows) : nullptr;
  D.steps = (const DecStep*)(d + o_steps);
  D.goff = (const int32_t*)(d + o_goff);
  D.zeros = zeros;
  D.xs = (uint16_t*)(d + o_xs);
  D.acc32[0] = (float*)(d + o_acc0);
  D.acc32[1] = (float*)(d + o_acc1);
  D.part = S > 1 ? (float*)(d + o_part) : nullptr;
  D.cnt = (int32_t*)(d + o_cnt);
  D.acc_bytes = (uint32_t)acc_bytes;
  D.part_bytes = (uint32_t)part_bytes;
  D.fwd = 0;
  D.route = route;
  D.rot = rot.empty() ? nullptr : (const FdRotItem*)(d + o_rot);
  D.n_rot_items = (int32_t)rot.size();
  D.rot_blk = rot_blk;
  D.chunks = chunks.empty() ? nullptr : (const RtChunk*)(d + o_chunks);
  D.n_chunks = (int32_t)chunks.size();
  D.S_rows = (route & SCUTE_PLAN_ROUTE_SEPARATE_S) ? (float*)(d + o_srows) : nullptr;
  D.enabled = true;
  return SCUTE_OK;
}

}  // namespace scute
