// Tables of the MFMA decode path (bf16, up to 256 rows per batch).
//
// The base GEMM y = (x W + delta W) (.) s + b is split into column tiles of
// 64 outputs and S slices of the K dimension; the last slice of a tile to
// finish adds the others' partial products (kept in a workspace) and writes
// y once. The low-rank work of the expand step ("Where is
// the cheapest place to compute the remaining slots?", paper-daily.com
// explainer of "Scute: Exact Batched Serving for PEFT Adapters Beyond LoRA":
// the expand works on tiles that each belong to one adapter; VeRA's shared
// B is applied to every VeRA row of the batch at once) is cut into items:
//   own item   (row group g, adapter, 16 ranks): one 32x32x16 MFMA step
//   VeRA item  (row group g): r_v / 16 MFMA steps against the shared B_sh,
//              then each row scaled by its adapter's e
// and the items of every column tile are spread over its S slices.
// The prologue items (rotation, own-term shrink, VeRA shrink) are listed
// here too; see decode.hip for the kernels.

#include <string.h>

#include <algorithm>

#include "internal.h"

namespace scute {

namespace {

enum : int32_t { PRO_ROT = 0, PRO_SHRINK = 1, PRO_VSHRINK = 2 };
enum : int32_t { EXP_OWN = 0, EXP_VERA = 1 };

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
  if (env_int("SCUTE_DECODE", 1) == 0) return SCUTE_OK;
  if (L->act != SCUTE_BF16 || n <= 0 || n > 256) return SCUTE_OK;
  if (d_in % 128 != 0 || d_out % 64 != 0) return SCUTE_OK;
  if (B->n_vera > 0 && (L->r_v % 32 != 0 || d_in % 512 != 0)) return SCUTE_OK;
  for (int32_t i = 0; i < B->nseg(); ++i) {
    const SlotEntry& E = L->table[B->seg[3 * i]];
    if ((E.flags & F_TERM) && (E.rank % 8 != 0)) return SCUTE_OK;
  }

  D.MG = (n + 31) / 32;
  D.g_rot = (B->n_rot + 31) / 32;
  // two staged groups compile badly (accumulator copies); pad with one row
  // group of unused rows instead
  if (D.MG + D.g_rot == 2) D.MG += 1;
  if (D.MG + D.g_rot > 9) {  // two LDS buffers of 32 (MG + g_rot) rows x 256 B + row tables
    D = DecodePlan{};
    return SCUTE_OK;
  }
  D.M_pad = 32 * D.MG;
  D.RT = (B->max_rank + 15) / 16 * 16;
  D.C = (int32_t)(d_out / 64);
  // K slices: none when the column tiles alone nearly fill the chip (every
  // slice costs a partial product of the whole tile in the workspace);
  // otherwise the fewest that reach one work-group per compute unit. Each
  // slice is split in two K halves of 64-wide stages.
  const int32_t cu = L->num_cu > 0 ? L->num_cu : 256;
  int32_t S = 1;
  if ((int64_t)D.C * 4 < (int64_t)cu * 3)
    while ((int64_t)D.C * S < cu && d_in % ((int64_t)S * 2 * 128) == 0) S *= 2;
  S = env_int("SCUTE_DECODE_SPLITK", S);
  if (S < 1 || d_in % ((int64_t)S * 128) != 0)
    return fail(SCUTE_E_INVALID, "bad SCUTE_DECODE_SPLITK");
  D.S = S;
  D.k_chunk = (int32_t)(d_in / S);

  // ---- per-row tables (pointer tables padded to 256 rows) --------------------
  std::vector<int32_t> row_tok(D.M_pad, -1);
  std::vector<const float*> row_s(256, nullptr), row_b(256, nullptr), row_ve(256, nullptr);
  for (int32_t p = 0; p < n; ++p) {
    row_tok[p] = B->perm[p];
    int32_t a = B->row_adapter[p];
    if (a < 0) continue;
    const SlotEntry& E = L->table[a];
    if (E.flags & F_S) row_s[p] = E.s;
    if (E.flags & F_B) row_b[p] = E.b;
    if (E.flags & F_VERA) row_ve[p] = E.ve;
  }

  // ---- prologue items -------------------------------------------------------
  //   rotation: (first row, rows <= 4, first of 64 columns)
  //   own shrink: (group of <= 4 rows x <= 4 ranks, K part of 1024)
  //   VeRA shrink: (32-row block of VeRA rows, 32-row block of A_sh, K slice of 512)
  std::vector<int4> pro, sgroups;
  for (int32_t i = 0; i < B->nseg(); ++i) {
    const int32_t a = B->seg[3 * i], start = B->seg[3 * i + 1], len = B->seg[3 * i + 2];
    const SlotEntry& E = L->table[a];
    if (E.flags & F_R)
      for (int32_t r0 = 0; r0 < len; r0 += 4)
        for (int64_t c0 = 0; c0 < d_in; c0 += 64)
          pro.push_back(make_int4(PRO_ROT, start + r0, std::min(4, len - r0), (int32_t)c0));
    if (E.flags & F_TERM)
      for (int32_t r0 = 0; r0 < len; r0 += 4)
        for (int32_t k = 0; k < E.rank; k += 4)
          sgroups.push_back(make_int4(start + r0, std::min(4, len - r0), k, std::min(4, E.rank - k)));
  }
  D.KQ = (int32_t)((d_in + 1023) / 1024);
  D.n_sgroups = (int32_t)sgroups.size();
  for (int32_t kq = 0; kq < D.KQ; ++kq)
    for (int32_t gi = 0; gi < D.n_sgroups; ++gi) pro.push_back(make_int4(PRO_SHRINK, gi, kq, 0));
  if (B->n_vera > 0) {
    D.nvb = (B->n_vera + 31) / 32;
    D.njb = L->r_v / 32;
    D.SV = (int32_t)(d_in / 512);
    for (int32_t kv = 0; kv < D.SV; ++kv)
      for (int32_t vb = 0; vb < D.nvb; ++vb)
        for (int32_t jb = 0; jb < D.njb; ++jb) pro.push_back(make_int4(PRO_VSHRINK, vb, jb, kv));
  }
  D.n_pro = (int32_t)pro.size();

  // ---- expand items, spread over the S K-slices -----------------------------
  // item: (type | row group << 8, first rank, 16-rank steps (<= 4) | B row
  // length << 8, first row | end row << 16), plus the B pointer
  struct Item {
    int4 v;
    const uint16_t* ptr;
    int32_t cost;
  };
  std::vector<Item> items;
  for (int32_t i = 0; i < B->nseg(); ++i) {
    const int32_t a = B->seg[3 * i], start = B->seg[3 * i + 1], len = B->seg[3 * i + 2];
    const SlotEntry& E = L->table[a];
    if (!(E.flags & F_TERM)) continue;
    for (int32_t g = start / 32; g * 32 < start + len; ++g) {
      int32_t lo = std::max(start, 32 * g), hi = std::min(start + len, 32 * g + 32);
      for (int32_t k = 0; k < E.rank; k += 64) {
        int32_t nst = std::min(4, (E.rank - k + 15) / 16);
        items.push_back({make_int4(EXP_OWN | (g << 8), k, nst | (E.rank << 8), lo | (hi << 16)),
                         (const uint16_t*)E.B, nst});
      }
    }
  }
  if (B->n_vera > 0) {
    for (int32_t g = 0; g < D.MG; ++g) {
      bool any = false;
      for (int32_t p = 32 * g; p < std::min(n, 32 * g + 32); ++p) any |= row_ve[p] != nullptr;
      if (!any) continue;
      for (int32_t k = 0; k < L->r_v; k += 64) {
        int32_t nst = std::min(4, (L->r_v - k) / 16);
        items.push_back({make_int4(EXP_VERA | (g << 8), k, nst | (L->r_v << 8),
                                   (32 * g) | ((32 * g + 32) << 16)),
                         (const uint16_t*)L->B_sh, nst + 2});
      }
    }
  }
  std::stable_sort(items.begin(), items.end(),
                   [](const Item& p, const Item& q) { return p.cost > q.cost; });
  std::vector<std::vector<Item>> per(S);
  std::vector<int64_t> load(S, 0);
  for (const Item& it : items) {
    int32_t best = (int32_t)(std::min_element(load.begin(), load.end()) - load.begin());
    per[best].push_back(it);
    load[best] += it.cost;
  }
  std::vector<int4> exp;
  std::vector<const uint16_t*> exp_ptr;
  std::vector<int32_t> exp_off(S + 1, 0);
  for (int32_t k = 0; k < S; ++k) {
    exp_off[k] = (int32_t)exp.size();
    for (const Item& it : per[k]) {
      exp.push_back(it.v);
      exp_ptr.push_back(it.ptr);
    }
  }
  exp_off[S] = (int32_t)exp.size();
  D.n_exp = (int32_t)exp.size();

  // ---- one device allocation: tables, then workspaces -----------------------
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t r = o;
    o += al256(bytes);
    return r;
  };
  const size_t o_tok = take(4 * (size_t)D.M_pad);
  const size_t o_s = take(8 * 256), o_b = take(8 * 256), o_ve = take(8 * 256);
  const size_t o_pro = take(16 * pro.size() + 16), o_exp = take(16 * exp.size() + 16);
  const size_t o_ptr = take(8 * exp_ptr.size() + 8);
  const size_t o_off = take(4 * exp_off.size());
  const size_t o_sg = take(16 * sgroups.size() + 16);
  const size_t o_ones = take(4 * (size_t)d_out);
  const size_t tables = o;
  const size_t o_tb = take(2 * (size_t)D.M_pad * D.RT);
  const size_t o_ub = take(B->n_vera ? 2 * (size_t)D.M_pad * L->r_v : 0);
  const size_t o_delta = take(2 * (size_t)32 * D.g_rot * d_in);
  const size_t o_vpart = take(4 * (size_t)D.SV * D.nvb * D.njb * 1024);  // K slices of 256
  const size_t o_vcnt = take(4 * (size_t)D.nvb * D.njb);
  const size_t o_part = take(S > 1 ? 4 * (size_t)S * D.C * 2 * D.MG * 16 * 64 : 0);
  const size_t o_cnt = take(4 * (size_t)D.C);
  const size_t o_spart = take(4 * (size_t)D.KQ * D.n_sgroups * 16);
  const size_t o_scnt = take(4 * (size_t)D.n_sgroups);
  const size_t total = o;

  std::vector<uint8_t> h(tables, 0);
  memcpy(h.data() + o_tok, row_tok.data(), 4 * row_tok.size());
  memcpy(h.data() + o_s, row_s.data(), 8 * row_s.size());
  memcpy(h.data() + o_b, row_b.data(), 8 * row_b.size());
  memcpy(h.data() + o_ve, row_ve.data(), 8 * row_ve.size());
  if (!pro.empty()) memcpy(h.data() + o_pro, pro.data(), 16 * pro.size());
  if (!exp.empty()) memcpy(h.data() + o_exp, exp.data(), 16 * exp.size());
  if (!exp_ptr.empty()) memcpy(h.data() + o_ptr, exp_ptr.data(), 8 * exp_ptr.size());
  memcpy(h.data() + o_off, exp_off.data(), 4 * exp_off.size());
  if (!sgroups.empty()) memcpy(h.data() + o_sg, sgroups.data(), 16 * sgroups.size());
  for (int64_t j = 0; j < d_out; ++j) {
    const float one = 1.0f;
    memcpy(h.data() + o_ones + 4 * j, &one, 4);
  }

  hipError_t e = hipMalloc(&B->fast_dev, total);
  if (e != hipSuccess) return hip_fail(e, "hipMalloc(decode plan)");
  uint8_t* d = (uint8_t*)B->fast_dev;
  // workspaces start at zero: rows of delta past n_rot, ranks of tb past each
  // row's own rank, and the VeRA counters must read as zero
  e = hipMemsetAsync(d + tables, 0, total - tables, st);
  if (e == hipSuccess) e = hipMemcpyAsync(d, h.data(), tables, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    (void)hipFree(B->fast_dev);
    B->fast_dev = nullptr;
    return hip_fail(e, "upload decode plan");
  }
  D.row_tok = (const int32_t*)(d + o_tok);
  D.row_s = (const float* const*)(d + o_s);
  D.row_b = (const float* const*)(d + o_b);
  D.row_ve = (const float* const*)(d + o_ve);
  D.pro_items = (const int4*)(d + o_pro);
  D.exp_items = (const int4*)(d + o_exp);
  D.exp_ptr = (const uint16_t* const*)(d + o_ptr);
  D.exp_off = (const int32_t*)(d + o_off);
  D.ones = (const float*)(d + o_ones);
  D.tb = D.RT ? (uint16_t*)(d + o_tb) : nullptr;
  D.ub = B->n_vera ? (uint16_t*)(d + o_ub) : nullptr;
  D.delta = D.g_rot ? (uint16_t*)(d + o_delta) : nullptr;
  D.vpart = B->n_vera ? (float*)(d + o_vpart) : nullptr;
  D.vcnt = B->n_vera ? (int32_t*)(d + o_vcnt) : nullptr;
  D.part = S > 1 ? (float*)(d + o_part) : nullptr;
  D.cnt = (int32_t*)(d + o_cnt);
  D.sgroups = (const int4*)(d + o_sg);
  D.spart = (float*)(d + o_spart);
  D.scnt = (int32_t*)(d + o_scnt);
  D.enabled = true;
  return SCUTE_OK;
}

}  // namespace scute
