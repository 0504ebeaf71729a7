// Batch planner (segment builder) and the per-batch cost model.
//
// Planner: the expand of batched LoRA works on tiles that each belong to one
// adapter, and rows look up their tenant's VeRA vectors and rotation ("Where
// is the cheapest place to compute the remaining slots?", paper-daily.com
// explainer of "Scute: Exact Batched Serving for PEFT Adapters Beyond
// LoRA"). Tokens arrive in any order, so the plan is a stable sort of token
// indices by (row class, adapter id): rows with a rotation slot first, then
// rows with a shared VeRA term, then every other adapted row, then rows with
// no adapter. Runs of one adapter in that order are the segments.
//
// Cost model: adapter work is memory-bound, so its cost is counted in bytes;
// added time = extra bytes / bandwidth + extra launches x launch cost (same
// section of the explainer). Bytes count each needed byte once: x and W in
// the activation dtype, y in float32, each touched adapter's stored factors,
// the shared VeRA pair once if any row uses it. Intermediates are excluded.

#include <string.h>

#include <algorithm>

#include "internal.h"

using namespace scute;

namespace {

int row_class(const SlotEntry& E) {
  if (E.flags & F_R) return 0;
  if (E.flags & F_VERA) return 1;
  return 2;
}

void free_batch_memory(scute_batch* B) {
  const int dev = B->device;
  if (dev >= 0) {
    int prev = -1;
    (void)hipGetDevice(&prev);
    if (prev != dev) (void)hipSetDevice(dev);
    if (B->dev) (void)hipFree(B->dev);
    if (B->ws) (void)hipFree(B->ws);
    if (B->fast_dev) (void)hipFree(B->fast_dev);
    if (B->pf_dev) (void)hipFree(B->pf_dev);
    if (B->fd_dev) (void)hipFree(B->fd_dev);
    if (prev != dev && prev >= 0) (void)hipSetDevice(prev);
  }
  B->dev = B->ws = B->fast_dev = B->pf_dev = B->fd_dev = nullptr;
}

}  // namespace

extern "C" scute_status scute_plan_batch(scute_layer* L, const int32_t* token_adapter, int32_t n,
                                         void* stream, scute_batch** out) {
  return scute_plan_batch_flags(L, token_adapter, n, 0, stream, out);
}

extern "C" scute_status scute_plan_batch_flags(scute_layer* L, const int32_t* token_adapter, int32_t n,
                                               uint32_t flags, void* stream, scute_batch** out) {
  try {
    if (!L || !out) return fail(SCUTE_E_INVALID, "scute_plan_batch: null argument");
    *out = nullptr;
    if (flags & ~((uint32_t)SCUTE_PLAN_DETERMINISTIC | ROUTE_MASK))
      return fail(SCUTE_E_INVALID, "scute_plan_batch_flags: unknown flag bits");
    if ((flags & SCUTE_PLAN_ROUTE_SEPARATE_S) && !(flags & SCUTE_PLAN_ROUTE_EXPAND_PASS))
      return fail(SCUTE_E_INVALID, "scute_plan_batch_flags: ROUTE_SEPARATE_S needs ROUTE_EXPAND_PASS");
    if ((flags & SCUTE_PLAN_DETERMINISTIC) && (flags & ROUTE_MASK))
      return fail(SCUTE_E_INVALID, "scute_plan_batch_flags: route variants are not deterministic");
    if ((flags & ROUTE_MASK) && L->device < 0)
      return fail(SCUTE_E_UNSUPPORTED, "scute_plan_batch_flags: route variants need a device layer");
    if (n < 0 || n > (1 << 22)) return fail(SCUTE_E_SHAPE, "scute_plan_batch: n must be in [0, 2^22]");
    if (n > 0 && !token_adapter) return fail(SCUTE_E_INVALID, "scute_plan_batch: token_adapter is null");
    for (int32_t t = 0; t < n; ++t) {
      int32_t a = token_adapter[t];
      if (a < -1 || a >= L->max_adapters)
        return fail(SCUTE_E_INVALID, "scute_plan_batch: token " + std::to_string(t) +
                                         " has adapter id out of range");
      if (a >= 0 && !(L->table[a].flags & F_LOADED))
        return fail(SCUTE_E_STATE, "scute_plan_batch: token " + std::to_string(t) +
                                       " names adapter " + std::to_string(a) + " which is not loaded");
    }
    auto* B = new scute_batch();
    B->layer = L;
    B->device = L->device;
    B->epoch = L->epoch;
    B->n = n;
    B->flags = flags;
    B->perm.resize(n);
    for (int32_t t = 0; t < n; ++t) B->perm[t] = t;
    auto key = [&](int32_t t) -> int64_t {
      int32_t a = token_adapter[t];
      int64_t cls = a < 0 ? 3 : row_class(L->table[a]);
      return cls * ((int64_t)1 << 32) + (a < 0 ? 0 : a);
    };
    std::stable_sort(B->perm.begin(), B->perm.end(),
                     [&](int32_t p, int32_t q) { return key(p) < key(q); });
    B->row_adapter.resize(n);
    std::vector<char> touched(L->max_adapters, 0);
    for (int32_t p = 0; p < n; ++p) {
      int32_t a = token_adapter[B->perm[p]];
      B->row_adapter[p] = a;
      if (a < 0) continue;
      const SlotEntry& E = L->table[a];
      if (E.flags & F_R) B->n_rot = p + 1;
      if (E.flags & F_RPROJ) B->rproj = true;
      if (E.flags & F_VERA) B->vera_pos.push_back(p);
      if ((E.flags & F_TERM) && E.rank > B->max_rank) B->max_rank = E.rank;
      if (!touched[a]) {
        touched[a] = 1;
        B->n_touched++;
      }
      if (p == 0 || B->row_adapter[p - 1] != a) {
        B->seg.push_back(a);
        B->seg.push_back(p);
        B->seg.push_back(1);
      } else {
        B->seg.back()++;
      }
    }
    B->n_vera = (int32_t)B->vera_pos.size();

    if (L->device >= 0 && n > 0) {
      int prev = -1;
      (void)hipGetDevice(&prev);
      if (prev != L->device) (void)hipSetDevice(L->device);
      auto restore = [&] {
        if (prev != L->device && prev >= 0) (void)hipSetDevice(prev);
      };
      hipStream_t s = (hipStream_t)stream;
      // int tables: perm, row_adapter, seg, vera_pos (each 256-B aligned)
      auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
      size_t o_perm = 0, o_ra = o_perm + al(4 * (size_t)n), o_seg = o_ra + al(4 * (size_t)n);
      size_t o_vp = o_seg + al(4 * B->seg.size() + 4);
      size_t tot = o_vp + al(4 * B->vera_pos.size() + 4);
      hipError_t e = hipMalloc(&B->dev, tot);
      if (e != hipSuccess) {
        restore();
        delete B;
        return hip_fail(e, "hipMalloc(plan)");
      }
      std::vector<uint8_t> h(tot, 0);
      memcpy(h.data() + o_perm, B->perm.data(), 4 * (size_t)n);
      memcpy(h.data() + o_ra, B->row_adapter.data(), 4 * (size_t)n);
      if (!B->seg.empty()) memcpy(h.data() + o_seg, B->seg.data(), 4 * B->seg.size());
      if (!B->vera_pos.empty()) memcpy(h.data() + o_vp, B->vera_pos.data(), 4 * B->vera_pos.size());
      uint8_t* d = (uint8_t*)B->dev;
      B->d_perm = (int32_t*)(d + o_perm);
      B->d_row_adapter = (int32_t*)(d + o_ra);
      B->d_seg = (int32_t*)(d + o_seg);
      B->d_vera_pos = (int32_t*)(d + o_vp);
      e = hipMemcpyAsync(B->dev, h.data(), tot, hipMemcpyHostToDevice, s);
      if (e == hipSuccess) e = hipStreamSynchronize(s);
      // workspaces
      size_t es = dtype_size(L->act);
      // (one delta block per projection when a row rotates per projection)
      size_t w_delta = al((size_t)(B->rproj ? L->n_proj : 1) * B->n_rot * L->d_in * es);
      size_t w_t = al((size_t)n * B->max_rank * 4);
      size_t w_u = B->n_vera ? al((size_t)n * L->r_v * 4) : 0;
      size_t wtot = w_delta + w_t + w_u;
      if (e == hipSuccess && wtot > 0) {
        e = hipMalloc(&B->ws, wtot);
        if (e == hipSuccess) {
          uint8_t* w = (uint8_t*)B->ws;
          B->delta = B->n_rot ? w : nullptr;
          B->t = B->max_rank ? (float*)(w + w_delta) : nullptr;
          B->u = B->n_vera ? (float*)(w + w_delta + w_t) : nullptr;
        }
      }
      if (e != hipSuccess) {
        restore();
        free_batch_memory(B);
        delete B;
        return hip_fail(e, "plan upload / workspace");
      }
      scute_status ds = SCUTE_OK;
      if (flags & ROUTE_MASK) {
        ds = build_decode_plan(L, B, s);
        if (ds == SCUTE_OK && !B->dp.enabled)
          ds = fail(SCUTE_E_UNSUPPORTED, "scute_plan_batch_flags: route variants need a batch the "
                                         "two-launch decode path takes (bf16, up to 256 rows)");
      } else {
        ds = build_fdecode_plan(L, B, s);
        if (ds == SCUTE_OK && !B->fp.enabled) ds = build_decode_plan(L, B, s);
        if (ds == SCUTE_OK && !B->fp.enabled && !B->dp.enabled) ds = build_prefill_plan(L, B, s);
      }
      restore();
      if (ds != SCUTE_OK) {
        free_batch_memory(B);
        delete B;
        return ds;
      }
    }
    *out = B;
    return SCUTE_OK;
  } catch (const std::bad_alloc&) {
    return fail(SCUTE_E_NOMEM, "scute_plan_batch: host allocation failed");
  } catch (...) {
    return fail(SCUTE_E_INVALID, "scute_plan_batch: unexpected error");
  }
}

extern "C" scute_status scute_batch_destroy(scute_batch* B) {
  if (!B) return SCUTE_OK;
  free_batch_memory(B);
  delete B;
  return SCUTE_OK;
}

extern "C" scute_status scute_batch_info_get(const scute_batch* B, scute_batch_info* out) {
  if (!B || !out) return fail(SCUTE_E_INVALID, "scute_batch_info_get: null argument");
  out->n = B->n;
  out->n_segments = B->nseg();
  out->n_rot_rows = B->n_rot;
  out->n_vera_rows = B->n_vera;
  out->max_rank = B->max_rank;
  out->path = (B->fp.enabled || B->dp.enabled) ? 1 : (B->pp.enabled ? 2 : 0);
  return SCUTE_OK;
}

// The fused decode path's error flag: its cross-work-group waits are
// bounded, and a wait that gives up sets the flag instead of hanging.
extern "C" scute_status scute_batch_wait_failures(const scute_batch* B, int32_t reset, int32_t* out) {
  if (!B || !out) return fail(SCUTE_E_INVALID, "scute_batch_wait_failures: null argument");
  *out = 0;
  if (!B->fp.enabled || !B->fp.err) return SCUTE_OK;
  int prev = -1;
  (void)hipGetDevice(&prev);
  if (prev != B->device) (void)hipSetDevice(B->device);
  int32_t v = 0;
  hipError_t e = hipMemcpy(&v, B->fp.err, 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess && reset) {
    const int32_t zero = 0;
    e = hipMemcpy(B->fp.err, &zero, 4, hipMemcpyHostToDevice);
  }
  if (prev != B->device && prev >= 0) (void)hipSetDevice(prev);
  if (e != hipSuccess) return hip_fail(e, "scute_batch_wait_failures");
  *out = v != 0;
  return SCUTE_OK;
}

extern "C" scute_status scute_batch_read(const scute_batch* B, int32_t* perm, int32_t* seg) {
  if (!B) return fail(SCUTE_E_INVALID, "scute_batch_read: batch is null");
  if (perm && B->n) memcpy(perm, B->perm.data(), 4 * (size_t)B->n);
  if (seg && !B->seg.empty()) memcpy(seg, B->seg.data(), 4 * B->seg.size());
  return SCUTE_OK;
}

extern "C" scute_status scute_cost_model(const scute_layer* L, const scute_batch* B,
                                         scute_cost* out) {
  if (!L || !B || !out) return fail(SCUTE_E_INVALID, "scute_cost_model: null argument");
  if (B->layer != L) return fail(SCUTE_E_STATE, "scute_cost_model: plan belongs to another layer");
  if (B->epoch != L->epoch) return fail(SCUTE_E_STATE, "scute_cost_model: plan is stale");
  memset(out, 0, sizeof(*out));
  const double es = (double)dtype_size(L->act);
  const double n = B->n, din = (double)L->d_in, dout = (double)L->d_out;
  double adapter = 0.0, flops_extra = 0.0, gemm_side = 0.0, pro_side = 0.0, exp_flops = 0.0;
  bool any_pro = false;
  bool any_vera = false;
  std::vector<char> seen(L->max_adapters, 0);
  for (int32_t p = 0; p < B->n; ++p) {
    int32_t a = B->row_adapter[p];
    if (a < 0) continue;
    const SlotEntry& E = L->table[a];
    const AdapterStore& S = L->store[a];
    if (!seen[a]) {
      seen[a] = 1;
      for (int i = 0; i < 7; ++i) adapter += (double)S.len[i];
      gemm_side += (double)(S.len[SCUTE_SLOT_B] + S.len[SCUTE_SLOT_S] + S.len[SCUTE_SLOT_BIAS] +
                            S.len[SCUTE_SLOT_VE]);
      pro_side += (double)(S.len[SCUTE_SLOT_A] + S.len[SCUTE_SLOT_VD] + S.len[SCUTE_SLOT_P]);
    }
    if (E.flags & (F_TERM | F_VERA | F_R)) any_pro = true;
    if (E.flags & F_TERM) {
      flops_extra += 2.0 * (din * E.rank + E.rank * dout);
      exp_flops += 2.0 * E.rank * dout;
    }
    if (E.flags & F_VERA) {
      any_vera = true;
      flops_extra += 2.0 * (din * L->r_v + L->r_v * dout);
      exp_flops += 2.0 * L->r_v * dout;
    }
    // (x R_p for every projection p when the adapter rotates per projection)
    if (E.flags & F_R) flops_extra += 2.0 * din * E.blk * ((E.flags & F_RPROJ) ? L->n_proj : 1);
  }
  if (any_vera) adapter += (double)L->r_v * (din + dout) * es;
  const double xwy = n * din * es + din * dout * es + n * dout * 4.0;
  if (B->n) {
    out->gemm_bytes = xwy + gemm_side + (any_vera ? (double)L->r_v * dout * es : 0.0);
    out->prologue_bytes =
        any_pro ? n * din * es + pro_side + (any_vera ? (double)L->r_v * din * es : 0.0) : 0.0;
  }
  out->bytes = (B->n ? xwy : 0.0) + adapter;
  out->adapter_bytes = adapter;
  out->base_flops = 2.0 * n * din * dout;
  out->flops = out->base_flops + flops_extra;
  out->gemm_flops = out->base_flops + exp_flops;
  out->prologue_flops = flops_extra - exp_flops;
  out->launches = forward_launch_count(L, B);
  out->n_tokens = B->n;
  out->n_segments = B->nseg();
  out->n_rot_rows = B->n_rot;
  out->n_vera_rows = B->n_vera;
  out->n_touched = B->n_touched;
  return SCUTE_OK;
}
