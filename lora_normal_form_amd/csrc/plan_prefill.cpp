// Tables of the MFMA prefill path (bf16, long adapter segments).
//
// The base GEMM y = (x W + delta W) (.) s + b runs on tiles of 128 staged
// rows by 256 output columns over the whole K dimension. The rows of a tile
// come from one adapter segment ("Where is the cheapest place to compute the
// remaining slots?", paper-daily.com explainer of "Scute: Exact Batched
// Serving for PEFT Adapters Beyond LoRA": tiles belong to one adapter), so
// the tile's epilogue applies one s, b, e and one own B' to every row: a
// chunk is up to 128 tokens of a segment, or up to 64 tokens and their 64
// Delta rows when the adapter rotates. The expand runs in the same epilogue
// as extra MFMA steps whose A operand is the chunk's shrink sums.
// The prologue kernel computes the own-term and VeRA shrinks (tiles of 64
// rows x 64 ranks x one K part of 1024, added in fixed point so the sums do
// not depend on the order of the parts) and the rotation Delta = x (R - I).

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

scute_status build_prefill_plan(const scute_layer* L, scute_batch* B, hipStream_t st) {
  PrefillPlan& P = B->pp;
  P = PrefillPlan{};
  const int32_t n = B->n;
  const int64_t d_in = L->d_in, d_out = L->d_out;
  if (env_int("SCUTE_PREFILL", 1) == 0) return SCUTE_OK;
  if (L->act != SCUTE_BF16 || n <= 0) return SCUTE_OK;
  // rows that rotate per projection: each 256-column tile stages its own
  // projection's Delta rows, so the projections must end on tile boundaries
  if (B->rproj)
    for (int32_t i = 0; i + 1 < L->n_proj; ++i)
      if (L->proj_end[i] % 256 != 0) return SCUTE_OK;
  // the main kernel's K loop runs in stages of 64 k (unrolled at compile
  // time for d_in 4096); the prologue's items need d_in % 256 (checked below)
  if (d_in % 64 != 0 || d_out % 256 != 0) return SCUTE_OK;
  // W, x and the Delta rows are addressed through buffer ranges with 32-bit offsets
  if (d_in * d_out * 2 >= ((int64_t)1 << 32) || (int64_t)n * d_in * 2 >= ((int64_t)1 << 32))
    return SCUTE_OK;
  if (B->n_rot > 0 && !B->delta) return SCUTE_OK;
  if (B->n_vera > 0 && L->r_v % 64 != 0) return SCUTE_OK;
  for (int32_t i = 0; i < B->nseg(); ++i) {
    const SlotEntry& E = L->table[B->seg[3 * i]];
    if ((E.flags & F_TERM) && (E.rank % 8 != 0)) return SCUTE_OK;
  }

  P.RT = (B->max_rank + 15) / 16 * 16;
  P.AW = P.RT + (B->n_vera > 0 ? L->r_v : 0);
  P.C = (int32_t)(d_out / 256);

  // ---- chunks ---------------------------------------------------------------
  // segments cover the adapted rows [0, n_adapted); the rows without an
  // adapter follow them
  std::vector<int32_t> segs(B->seg);
  int32_t n_adapted = 0;
  for (int32_t i = 0; i < B->nseg(); ++i) n_adapted = std::max(n_adapted, segs[3 * i + 1] + segs[3 * i + 2]);
  if (n_adapted < n) {
    segs.push_back(-1);
    segs.push_back(n_adapted);
    segs.push_back(n - n_adapted);
  }
  std::vector<PfChunk> chunks;
  std::vector<int32_t> crow;
  for (size_t i = 0; i < segs.size() / 3; ++i) {
    const int32_t a = segs[3 * i], start = segs[3 * i + 1], len = segs[3 * i + 2];
    const SlotEntry* E = a >= 0 ? &L->table[a] : nullptr;
    const bool rot = E && (E->flags & F_R);
    const int32_t step = rot ? 64 : 128;
    for (int32_t r0 = 0; r0 < len; r0 += step) {
      PfChunk c{};
      c.x0 = start + r0;
      c.nx = std::min(step, len - r0);
      c.rows = step;
      c.flags = rot ? PF_ROT : 0;
      c.s = nullptr;  // resolved after the allocation (ones / zeros dummies)
      c.e = nullptr;
      c.b = nullptr;
      if (E) {
        if (E->flags & F_S) c.s = E->s;
        if (E->flags & F_B) c.b = E->b;
        if (E->flags & F_VERA) {
          c.e = E->ve;
          c.flags |= PF_VERA;
        }
        if (E->flags & F_TERM) {
          c.Bp = (const uint16_t*)E->B;
          c.rank = E->rank;
          c.flags |= PF_OWN;
        }
      }
      chunks.push_back(c);
      // staged row sources: x rows by token, Delta rows as -(sorted position) - 1;
      // rows past the chunk's tokens repeat its last one (computed, not stored)
      for (int32_t r = 0; r < 128; ++r) {
        if (rot && r >= 64)
          crow.push_back(-(c.x0 + std::min(r - 64, c.nx - 1)) - 1);
        else
          crow.push_back(B->perm[c.x0 + std::min(r, c.nx - 1)]);
      }
    }
  }
  P.n_chunks = (int32_t)chunks.size();

  // ---- work-group order --------------------------------------------------------
  // Work-groups are dispatched round-robin over the 8 XCDs by linear id, and
  // each XCD has its own L2. Each XCD gets a block of cg column tiles x a
  // share of the chunks (cg chosen so the W and rows one XCD reads are
  // smallest), chunk-major, so the work-groups running together on an XCD
  // share W columns and rows. Every XCD runs whole tiles in multiples of its
  // compute units; the tiles left over are split into P parts of the K
  // dimension (as many as the idle compute units take, up to 4) whose
  // partial tiles meet in a workspace.
  const int32_t X = 8;
  const int32_t cu = L->num_cu > 0 ? L->num_cu : 256;
  const int32_t cpx = std::max(1, cu / X);
  int32_t cg = 1;
  {
    double best = 1e300;
    for (int32_t g = 1; g <= X && g <= P.C; g *= 2) {
      const int32_t rg = X / g;
      const double bytes = (double)((P.C + g - 1) / g) * 256.0 + (double)((P.n_chunks + rg - 1) / rg) * 128.0;
      if (bytes < best) {
        best = bytes;
        cg = g;
      }
    }
  }
  const int32_t rg = X / cg;
  std::vector<std::vector<int4>> full(X);
  std::vector<int4> rest;
  for (int32_t x = 0; x < X; ++x) {
    const int32_t c_lo = P.C * (x % cg) / cg, c_hi = P.C * (x % cg + 1) / cg;
    const int32_t r_lo = P.n_chunks * (x / cg) / rg, r_hi = P.n_chunks * (x / cg + 1) / rg;
    std::vector<int4> lst;
    for (int32_t ci = r_lo; ci < r_hi; ++ci)
      for (int32_t c = c_lo; c < c_hi; ++c) lst.push_back(make_int4(c, ci, -1, 0));
    const size_t nf = lst.size() / cpx * cpx;
    full[x].assign(lst.begin(), lst.begin() + nf);
    rest.insert(rest.end(), lst.begin() + nf, lst.end());
  }
  int32_t parts = 1;
  const int64_t nst = d_in / 64;
  while (parts < 4 && !rest.empty() && (int64_t)rest.size() * parts * 2 <= cu && nst % (parts * 2) == 0)
    parts *= 2;
  parts = env_int("SCUTE_PREFILL_PARTS", parts);
  if ((parts != 1 && parts != 2 && parts != 4) || nst % parts != 0)
    return fail(SCUTE_E_INVALID, "bad SCUTE_PREFILL_PARTS (1, 2 or 4 dividing d_in / 64)");
  std::vector<int4> items;
  for (size_t j = 0;; ++j) {
    bool any = false;
    for (int32_t x = 0; x < X; ++x)
      if (j < full[x].size()) {
        items.push_back(full[x][j]);
        any = true;
      }
    if (!any) break;
  }
  for (size_t t = 0; t < rest.size(); ++t)
    for (int32_t q = 0; q < parts; ++q)
      items.push_back(make_int4(rest[t].x, rest[t].y, parts > 1 ? q : -1, (int32_t)t));
  P.n_items = (int32_t)items.size();
  P.P = parts;
  P.n_split = parts > 1 ? (int32_t)rest.size() : 0;

  // ---- prologue items ---------------------------------------------------------
  // shrink tiles of 64 rows x 64 ranks over one K part of 1024 (own: per
  // segment; VeRA: over the table of VeRA rows), then rotation tiles of 32
  // rows x 256 columns
  const int32_t KP = (int32_t)((d_in + 1023) / 1024);  // the last part may be shorter
  std::vector<PfProItem> pro;
  int32_t n_tiles = 0;  // shrink tiles (each with an arrival counter)
  for (int32_t i = 0; i < B->nseg(); ++i) {
    const int32_t a = B->seg[3 * i], start = B->seg[3 * i + 1], len = B->seg[3 * i + 2];
    const SlotEntry& E = L->table[a];
    if (E.flags & F_TERM)
      for (int32_t r0 = 0; r0 < len; r0 += 64)
        for (int32_t k = 0; k < E.rank; k += 64, ++n_tiles)
          for (int32_t kp = 0; kp < KP; ++kp)
            pro.push_back(PfProItem{PP_SHRINK, start + r0, std::min(64, len - r0),
                                    k | (std::min(64, E.rank - k) << 16), (const uint16_t*)E.A, kp,
                                    n_tiles});
  }
  int32_t nvb = 0;
  std::vector<DecVeraRow> vrows;
  if (B->n_vera > 0) {
    nvb = (B->n_vera + 63) / 64;
    for (int32_t vb = 0; vb < nvb; ++vb)
      for (int32_t k = 0; k < L->r_v; k += 64, ++n_tiles)
        for (int32_t kp = 0; kp < KP; ++kp)
          pro.push_back(PfProItem{PP_VSHRINK, vb, 64, k | (64 << 16), nullptr, kp, n_tiles});
    vrows.resize(64 * (size_t)nvb);
    for (size_t v = 0; v < vrows.size(); ++v) {
      const bool real = v < (size_t)B->n_vera;
      const int32_t p = B->vera_pos[real ? v : 0];
      vrows[v].vd = L->table[B->row_adapter[p]].vd;
      vrows[v].tok = B->perm[p];
      vrows[v].p = real ? p : -1;
    }
  }
  for (int32_t i = 0; i < B->nseg(); ++i) {
    const int32_t a = B->seg[3 * i], start = B->seg[3 * i + 1], len = B->seg[3 * i + 2];
    const SlotEntry& E = L->table[a];
    // (one Delta block of n_rot rows per projection when a row rotates per
    // projection: pad is the block's first row; an adapter with one rotation
    // uses it for every projection)
    if (E.flags & F_R)
      for (int32_t pj = 0; pj < (B->rproj ? L->n_proj : 1); ++pj)
        for (int32_t r0 = 0; r0 < len; r0 += 32)
          for (int64_t c0 = 0; c0 < d_in; c0 += 256)
            pro.push_back(PfProItem{PP_ROT, start + r0, std::min(32, len - r0), (int32_t)c0,
                                    (const uint16_t*)E.P + ((E.flags & F_RPROJ) ? (size_t)pj * d_in * E.blk : 0),
                                    E.blk, pj * B->n_rot});
  }
  P.n_pro = (int32_t)pro.size();
  // the prologue's items work in slices (shrinks) and column runs
  // (rotation) of 256
  if (P.n_pro > 0 && d_in % 256 != 0) {
    P = PrefillPlan{};
    return SCUTE_OK;
  }

  // ---- one device allocation: tables, then the shrink sums ----------------------
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t r = o;
    o += al256(bytes);
    return r;
  };
  const size_t o_chunks = take(sizeof(PfChunk) * chunks.size());
  const size_t o_items = take(sizeof(int4) * items.size());
  const size_t o_crow = take(4 * crow.size());
  const size_t o_pro = take(sizeof(PfProItem) * pro.size() + 16);
  const size_t o_vrows = take(sizeof(DecVeraRow) * vrows.size() + 16);
  const size_t o_ones = take(4 * (size_t)d_out);
  const size_t tables = o;
  const size_t o_zeros = take(4 * (size_t)d_out);
  const size_t tpart_bytes = (size_t)n_tiles * KP * 64 * 64 * 4;
  if (tpart_bytes >= ((size_t)1 << 31)) {
    P = PrefillPlan{};  // buffer offsets are 32-bit
    return SCUTE_OK;
  }
  const size_t o_tpart = take(tpart_bytes);
  const size_t tbf_bytes = 2 * (size_t)n * P.AW;
  const size_t o_tbf = take(tbf_bytes), o_tcnt = take(4 * (size_t)n_tiles + 4);
  const size_t part_bytes = (size_t)P.n_split * parts * 32 * 256 * 16;
  if (part_bytes >= ((size_t)1 << 31)) {
    P = PrefillPlan{};
    return SCUTE_OK;
  }
  const size_t o_part = take(part_bytes), o_cnt = take(4 * (size_t)P.n_split + 4);
  const size_t total = o;

  hipError_t e = hipMalloc(&B->pf_dev, total);
  if (e != hipSuccess) return hip_fail(e, "hipMalloc(prefill plan)");
  uint8_t* d = (uint8_t*)B->pf_dev;
  const float* ones = (const float*)(d + o_ones);
  const float* zeros = (const float*)(d + o_zeros);
  for (PfChunk& c : chunks) {
    if (!c.s) c.s = ones;
    if (!c.e) c.e = ones;
    if (!c.b) c.b = zeros;
  }

  std::vector<uint8_t> h(tables, 0);
  memcpy(h.data() + o_chunks, chunks.data(), sizeof(PfChunk) * chunks.size());
  memcpy(h.data() + o_items, items.data(), sizeof(int4) * items.size());
  memcpy(h.data() + o_crow, crow.data(), 4 * crow.size());
  if (!pro.empty()) memcpy(h.data() + o_pro, pro.data(), sizeof(PfProItem) * pro.size());
  if (!vrows.empty()) memcpy(h.data() + o_vrows, vrows.data(), sizeof(DecVeraRow) * vrows.size());
  for (int64_t j = 0; j < d_out; ++j) {
    const float one = 1.0f;
    memcpy(h.data() + o_ones + 4 * j, &one, 4);
  }
  e = hipMemsetAsync(d + tables, 0, total - tables, st);
  if (e == hipSuccess) e = hipMemcpyAsync(d, h.data(), tables, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    (void)hipFree(B->pf_dev);
    B->pf_dev = nullptr;
    P = PrefillPlan{};
    return hip_fail(e, "upload prefill plan");
  }
  P.chunks = (const PfChunk*)(d + o_chunks);
  P.crow = (const int32_t*)(d + o_crow);
  P.pro_items = (const PfProItem*)(d + o_pro);
  P.vrows = B->n_vera ? (const DecVeraRow*)(d + o_vrows) : nullptr;
  P.items = (const int4*)(d + o_items);
  P.part = (float*)(d + o_part);
  P.cnt = (int32_t*)(d + o_cnt);
  P.part_bytes = (uint32_t)part_bytes;
  P.tpart = (float*)(d + o_tpart);
  P.tpart_bytes = (uint32_t)tpart_bytes;
  P.tbf = (uint16_t*)(d + o_tbf);
  P.tcnt = (int32_t*)(d + o_tcnt);
  P.tbf_bytes = (uint32_t)tbf_bytes;
  P.enabled = true;
  return SCUTE_OK;
}

}  // namespace scute
