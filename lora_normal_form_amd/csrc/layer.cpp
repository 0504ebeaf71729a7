// Layer context, adapter loading and the load-time slot fold.
//
// Fold rule ("Which slots can be merged at load?", paper-daily.com explainer
// of "Scute: Exact Batched Serving for PEFT Adapters Beyond LoRA"): a slot
// next to a factor the adapter owns merges into that factor once at load,
// e.g. (xA) (.) d = x (A diag(d)); a slot whose neighbours are all shared
// (the base W, the shared VeRA pair) stays live and is applied every step.
// DoRA's rescale factor is computed here from W ("How does Scute plug into
// vLLM?": s = learned length / norm of each column of W + cAB).
// All fold arithmetic is fp64 on the host; results are rounded once to the
// storage type (activation dtype for matrices, float32 for live vectors).

#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <thread>

#include "internal.h"

namespace scute {

static thread_local std::string g_last_error;

scute_status fail(scute_status code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

scute_status hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string("HIP error in ") + what + ": " + hipGetErrorString(e);
  return e == hipErrorOutOfMemory ? SCUTE_E_NOMEM : SCUTE_E_HIP;
}

size_t dtype_size(int32_t dt) {
  switch (dt) {
    case SCUTE_F32: return 4;
    case SCUTE_BF16: return 2;
    case SCUTE_F64: return 8;
    default: return 0;
  }
}

// ---------------------------------------------------------------------------
// element conversion
// ---------------------------------------------------------------------------

static inline double bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

// Round a double to bf16 with round-to-nearest-even on the 45 dropped
// mantissa bits of the binary64 pattern (exact inside bf16's normal range).
static inline uint16_t double_to_bf16(double v) {
  if (!isfinite(v)) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
  }
  uint64_t b;
  memcpy(&b, &v, 8);
  uint64_t lsb = (b >> 45) & 1u;
  b = (b + ((1ull << 44) - 1) + lsb) & ~((1ull << 45) - 1);
  double r;
  memcpy(&r, &b, 8);
  float f = (float)r;  // exact: r has at most 8 significant bits
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static inline double load_elem(const void* p, int32_t dt, size_t i) {
  switch (dt) {
    case SCUTE_F64: return ((const double*)p)[i];
    case SCUTE_F32: return (double)((const float*)p)[i];
    default: return bf16_to_double(((const uint16_t*)p)[i]);
  }
}

static void to_host_vector(const void* p, int32_t dt, size_t n, std::vector<double>& out) {
  out.resize(n);
  for (size_t i = 0; i < n; ++i) out[i] = load_elem(p, dt, i);
}

static void store_act(void* dst, int32_t act, size_t i, double v) {
  if (act == SCUTE_BF16)
    ((uint16_t*)dst)[i] = double_to_bf16(v);
  else
    ((float*)dst)[i] = (float)v;
}

// ---------------------------------------------------------------------------
// fp64 helpers of the fold
// ---------------------------------------------------------------------------

// Solve M X = Rhs (n x n, row-major) by Gaussian elimination with partial
// pivoting. Returns false if M is singular.
static bool solve_dense(int n, std::vector<double>& M, std::vector<double>& Rhs) {
  for (int col = 0; col < n; ++col) {
    int piv = col;
    for (int r = col + 1; r < n; ++r)
      if (fabs(M[(size_t)r * n + col]) > fabs(M[(size_t)piv * n + col])) piv = r;
    if (M[(size_t)piv * n + col] == 0.0) return false;
    if (piv != col) {
      for (int j = 0; j < n; ++j) {
        std::swap(M[(size_t)piv * n + j], M[(size_t)col * n + j]);
        std::swap(Rhs[(size_t)piv * n + j], Rhs[(size_t)col * n + j]);
      }
    }
    double inv = 1.0 / M[(size_t)col * n + col];
    for (int r = col + 1; r < n; ++r) {
      double f = M[(size_t)r * n + col] * inv;
      if (f == 0.0) continue;
      for (int j = col; j < n; ++j) M[(size_t)r * n + j] -= f * M[(size_t)col * n + j];
      for (int j = 0; j < n; ++j) Rhs[(size_t)r * n + j] -= f * Rhs[(size_t)col * n + j];
    }
  }
  for (int col = n - 1; col >= 0; --col) {
    double inv = 1.0 / M[(size_t)col * n + col];
    for (int j = 0; j < n; ++j) Rhs[(size_t)col * n + j] *= inv;
    for (int r = 0; r < col; ++r) {
      double f = M[(size_t)r * n + col];
      if (f == 0.0) continue;
      for (int j = 0; j < n; ++j) Rhs[(size_t)r * n + j] -= f * Rhs[(size_t)col * n + j];
    }
  }
  return true;
}

template <class F>
static void parallel_for(int64_t n, F&& fn) {
  unsigned hw = std::thread::hardware_concurrency();
  int64_t nt = std::max<int64_t>(1, std::min<int64_t>({(int64_t)(hw ? hw : 4), 16, n}));
  if (nt <= 1) {
    fn(0, n);
    return;
  }
  std::vector<std::thread> th;
  int64_t chunk = (n + nt - 1) / nt;
  for (int64_t t = 0; t < nt; ++t) {
    int64_t lo = t * chunk, hi = std::min(n, lo + chunk);
    if (lo >= hi) break;
    th.emplace_back([&fn, lo, hi] { fn(lo, hi); });
  }
  for (auto& t : th) t.join();
}

// DoRA: s_j = m_j / || column j of (W + cAB) || (row-vector orientation;
// in buffer layout, column j of the formula is row j of W [d_out][d_in]).
static void dora_scale(const void* W, int32_t dt, int64_t d_in, int64_t d_out, int32_t r,
                       double c, const std::vector<double>& A, const std::vector<double>& B,
                       const std::vector<double>& m, std::vector<double>& s) {
  s.assign(d_out, 0.0);
  parallel_for(d_out, [&](int64_t lo, int64_t hi) {
    std::vector<double> col(d_in);
    for (int64_t j = lo; j < hi; ++j) {
      for (int64_t i = 0; i < d_in; ++i) col[i] = load_elem(W, dt, (size_t)j * d_in + i);
      for (int32_t k = 0; k < r; ++k) {
        double cb = c * B[(size_t)j * r + k];
        const double* a = &A[(size_t)k * d_in];
        for (int64_t i = 0; i < d_in; ++i) col[i] += cb * a[i];
      }
      double ss = 0.0;
      for (int64_t i = 0; i < d_in; ++i) ss += col[i] * col[i];
      s[j] = m[j] / sqrt(ss);
    }
  });
}

// ---------------------------------------------------------------------------
// device guard: run with the layer's device current, restore afterwards
// ---------------------------------------------------------------------------

struct DeviceGuard {
  int prev = -1;
  bool active = false;
  explicit DeviceGuard(int dev) {
    if (dev >= 0 && hipGetDevice(&prev) == hipSuccess) {
      active = true;
      if (prev != dev) (void)hipSetDevice(dev);
    }
  }
  ~DeviceGuard() {
    if (active) (void)hipSetDevice(prev);
  }
};

}  // namespace scute

using namespace scute;

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" const char* scute_last_error(void) { return g_last_error.c_str(); }

extern "C" const char* scute_version(void) { return "scute-mi355x 0.1 (gfx950)"; }

extern "C" scute_status scute_layer_create(int32_t device, int64_t d_in, int64_t d_out,
                                           int32_t act_dtype, int32_t max_adapters,
                                           scute_layer** out) {
  try {
    if (!out) return fail(SCUTE_E_INVALID, "scute_layer_create: out is null");
    *out = nullptr;
    if (d_in <= 0 || d_out <= 0 || d_in > (1 << 20) || d_out > (1 << 20))
      return fail(SCUTE_E_SHAPE, "scute_layer_create: d_in and d_out must be in [1, 2^20]");
    if (d_in % 8 != 0 || d_out % 8 != 0)
      return fail(SCUTE_E_SHAPE, "scute_layer_create: d_in and d_out must be multiples of 8");
    if (act_dtype != SCUTE_BF16 && act_dtype != SCUTE_F32)
      return fail(SCUTE_E_INVALID, "scute_layer_create: act_dtype must be SCUTE_BF16 or SCUTE_F32");
    if (max_adapters <= 0 || max_adapters > (1 << 20))
      return fail(SCUTE_E_INVALID, "scute_layer_create: max_adapters must be in [1, 2^20]");
    if (device < -1) return fail(SCUTE_E_INVALID, "scute_layer_create: device must be >= -1");
    auto* L = new scute_layer();
    // every layer starts its epochs in a range of its own, so a plan kept past
    // its layer's destruction never passes the staleness check of a new layer
    // allocated at the same address
    static std::atomic<uint64_t> serial{0};
    L->epoch = (serial.fetch_add(1) + 1) << 32;
    L->device = device;
    L->d_in = d_in;
    L->d_out = d_out;
    L->proj_end[0] = d_out;
    L->act = act_dtype;
    L->max_adapters = max_adapters;
    L->table.assign(max_adapters, SlotEntry{});
    L->store.assign(max_adapters, AdapterStore{});
    if (device >= 0) {
      int ndev = 0;
      hipError_t e = hipGetDeviceCount(&ndev);
      if (e != hipSuccess || device >= ndev) {
        delete L;
        return fail(SCUTE_E_INVALID, "scute_layer_create: no such HIP device");
      }
      DeviceGuard g(device);
      hipDeviceProp_t prop;
      e = hipGetDeviceProperties(&prop, device);
      if (e != hipSuccess) {
        delete L;
        return hip_fail(e, "hipGetDeviceProperties");
      }
      L->num_cu = prop.multiProcessorCount;
      size_t tb = sizeof(SlotEntry) * (size_t)max_adapters;
      e = hipMalloc((void**)&L->table_dev, tb);
      if (e != hipSuccess) {
        delete L;
        return hip_fail(e, "hipMalloc(slot table)");
      }
      e = hipMemset(L->table_dev, 0, tb);
      if (e != hipSuccess) {
        (void)hipFree(L->table_dev);
        delete L;
        return hip_fail(e, "hipMemset(slot table)");
      }
      // the no-allocation forward's scratch address on this device
      scute_status ns = noalloc_setup(device);
      if (ns != SCUTE_OK) {
        (void)hipFree(L->table_dev);
        delete L;
        return ns;
      }
    }
    *out = L;
    return SCUTE_OK;
  } catch (const std::bad_alloc&) {
    return fail(SCUTE_E_NOMEM, "scute_layer_create: host allocation failed");
  } catch (...) {
    return fail(SCUTE_E_INVALID, "scute_layer_create: unexpected error");
  }
}

static void free_store(scute_layer* L, AdapterStore& st) {
  if (!st.mem) return;
  if (L->device >= 0)
    (void)hipFree(st.mem);
  else
    free(st.mem);
  st = AdapterStore{};
}

extern "C" scute_status scute_layer_destroy(scute_layer* L) {
  if (!L) return SCUTE_OK;
  DeviceGuard g(L->device);
  for (auto& st : L->store) free_store(L, st);
  if (L->table_dev) (void)hipFree(L->table_dev);
  for (auto& ev : L->prof_pending) {
    (void)hipEventSynchronize(ev.stop);
    L->prof_pool.push_back(ev.start);
    L->prof_pool.push_back(ev.stop);
  }
  for (hipEvent_t e : L->prof_pool) (void)hipEventDestroy(e);
  delete L;
  return SCUTE_OK;
}

extern "C" scute_status scute_set_vera_shared(scute_layer* L, const void* A_sh,
                                              const void* B_sh, int32_t r_v) {
  if (!L) return fail(SCUTE_E_INVALID, "scute_set_vera_shared: layer is null");
  if (!A_sh || !B_sh) return fail(SCUTE_E_INVALID, "scute_set_vera_shared: null matrix");
  if (r_v <= 0 || r_v > 4096)
    return fail(SCUTE_E_SHAPE, "scute_set_vera_shared: r_v must be in [1, 4096]");
  if (((uintptr_t)A_sh | (uintptr_t)B_sh) & 15)
    return fail(SCUTE_E_INVALID, "scute_set_vera_shared: matrices must be 16-byte aligned");
  if (L->n_vera_loaded > 0 && r_v != L->r_v)
    return fail(SCUTE_E_STATE, "scute_set_vera_shared: VeRA adapters are loaded with another r_v");
  if (L->n_vera_loaded > 0)
    return fail(SCUTE_E_STATE, "scute_set_vera_shared: unload VeRA adapters first");
  L->A_sh = A_sh;
  L->B_sh = B_sh;
  L->r_v = r_v;
  L->epoch++;
  return SCUTE_OK;
}

namespace {

struct FoldOut {
  int32_t flags = 0, rank = 0, blk = 0;
  std::vector<uint8_t> A, B, P;      // act dtype bytes
  std::vector<float> s, b, vd, ve;   // float32
};

// One rotation slot, (R - I)^T per block in the activation dtype, into dst
// (d_in blk elements): R given directly, or as the Cayley transform of the
// skew blocks Q ("The big picture": OFT's rotation is a Cayley transform).
scute_status fold_rotation(const scute_layer* L, int32_t dt, int32_t blk, const void* src, bool cayley,
                           uint8_t* dst) {
  const int64_t nb = L->d_in / blk;
  std::vector<double> M((size_t)blk * blk), X((size_t)blk * blk);
  for (int64_t kb = 0; kb < nb; ++kb) {
    const size_t base = (size_t)kb * blk * blk;
    if (cayley) {
      // R = (I - Q)^-1 (I + Q)
      for (int32_t i = 0; i < blk; ++i)
        for (int32_t j = 0; j < blk; ++j) {
          double q = load_elem(src, dt, base + (size_t)i * blk + j);
          double id = (i == j) ? 1.0 : 0.0;
          M[(size_t)i * blk + j] = id - q;
          X[(size_t)i * blk + j] = id + q;
        }
      if (!solve_dense(blk, M, X))
        return fail(SCUTE_E_INVALID, "scute_load_adapter: I - Q is singular");
    } else if (src) {
      for (int32_t i = 0; i < blk * blk; ++i) X[i] = load_elem(src, dt, base + i);
    } else {  // identity
      for (int32_t i = 0; i < blk; ++i)
        for (int32_t j = 0; j < blk; ++j) X[(size_t)i * blk + j] = (i == j) ? 1.0 : 0.0;
    }
    // stored transposed, (R - I)^T: element [kb][j][i] = (R - I)[kb][i][j],
    // so one output column's block entries are contiguous
    for (int32_t i = 0; i < blk; ++i)
      for (int32_t j = 0; j < blk; ++j)
        store_act(dst, L->act, base + (size_t)j * blk + i, X[(size_t)i * blk + j] - ((i == j) ? 1.0 : 0.0));
  }
  return SCUTE_OK;
}

scute_status fold_adapter(const scute_layer* L, const scute_adapter_desc* D, const void* W_host,
                          FoldOut& F) {
  const int64_t d_in = L->d_in, d_out = L->d_out;
  const int32_t dt = D->dtype, act = L->act;
  const size_t es = dtype_size(act);
  if (dtype_size(dt) == 0) return fail(SCUTE_E_INVALID, "scute_load_adapter: bad desc dtype");
  const int meth = D->method;
  if (meth < SCUTE_LORA || meth > SCUTE_NORMAL_FORM)
    return fail(SCUTE_E_INVALID, "scute_load_adapter: unknown method");
  std::vector<double> tmp;

  auto need = [&](const void* p, const char* what) -> scute_status {
    if (!p) return fail(SCUTE_E_INVALID, std::string("scute_load_adapter: missing array ") + what);
    return SCUTE_OK;
  };
  auto vec_f32 = [&](const void* p, size_t n, std::vector<float>& dst, double scale) {
    dst.resize(n);
    for (size_t i = 0; i < n; ++i) dst[i] = (float)(scale * load_elem(p, dt, i));
  };

  // ---- own low-rank term: A' = c A diag(d), B' = B diag(e) ----------------
  bool term = (meth == SCUTE_LORA || meth == SCUTE_DORA ||
               (meth == SCUTE_NORMAL_FORM && D->rank > 0));
  std::vector<double> A64, B64, s64;
  if (term) {
    if (D->rank <= 0 || D->rank > 1024)
      return fail(SCUTE_E_SHAPE, "scute_load_adapter: rank must be in [1, 1024]");
    scute_status st;
    if ((st = need(D->A, "A")) || (st = need(D->B, "B"))) return st;
    F.rank = D->rank;
    const int32_t r = D->rank;
    to_host_vector(D->A, dt, (size_t)r * d_in, A64);
    to_host_vector(D->B, dt, (size_t)d_out * r, B64);
    std::vector<double> dvec(r, 1.0), evec(d_out, 1.0);
    if (meth == SCUTE_NORMAL_FORM && D->d) to_host_vector(D->d, dt, r, dvec);
    if (meth == SCUTE_NORMAL_FORM && D->e) to_host_vector(D->e, dt, d_out, evec);
    if (meth == SCUTE_DORA) {
      if (!W_host) return fail(SCUTE_E_INVALID, "scute_load_adapter: DoRA needs W_host");
      if ((st = need(D->m, "m"))) return st;
      std::vector<double> m64;
      to_host_vector(D->m, dt, d_out, m64);
      dora_scale(W_host, dt, d_in, d_out, r, D->c, A64, B64, m64, s64);
      for (int64_t j = 0; j < d_out; ++j)
        if (!isfinite(s64[j]))
          return fail(SCUTE_E_INVALID, "scute_load_adapter: DoRA column of W + cAB has zero norm");
      evec = s64;  // e = s on the low-rank path
      F.flags |= F_S;
      F.s.resize(d_out);
      for (int64_t j = 0; j < d_out; ++j) F.s[j] = (float)s64[j];
    }
    // stored at the rank rounded up to a multiple of 8: the added A' rows and
    // B' columns are zero, so the term is unchanged and every kernel's rank
    // steps cover whole 8-rank pieces
    const int32_t r8 = (r + 7) / 8 * 8;
    F.rank = r8;
    F.A.assign((size_t)r8 * d_in * es, 0);
    F.B.assign((size_t)d_out * r8 * es, 0);
    for (int32_t k = 0; k < r; ++k)
      for (int64_t i = 0; i < d_in; ++i)
        store_act(F.A.data(), act, (size_t)k * d_in + i, D->c * dvec[k] * A64[(size_t)k * d_in + i]);
    for (int64_t j = 0; j < d_out; ++j)
      for (int32_t k = 0; k < r; ++k)
        store_act(F.B.data(), act, (size_t)j * r8 + k, B64[(size_t)j * r + k] * evec[j]);
    F.flags |= F_TERM;
  }

  // ---- base-path slots: s, b ------------------------------------------------
  if (meth == SCUTE_IA3) {
    scute_status st;
    if ((st = need(D->l, "l"))) return st;
    vec_f32(D->l, d_out, F.s, 1.0);
    F.flags |= F_S;
  }
  if (meth == SCUTE_NORMAL_FORM && D->s) {
    vec_f32(D->s, d_out, F.s, 1.0);
    F.flags |= F_S;
  }
  if (D->b) {
    vec_f32(D->b, d_out, F.b, 1.0);
    F.flags |= F_B;
  }

  // ---- shared VeRA term: d and e stay live, c merges into e ---------------
  bool vera = (meth == SCUTE_VERA) || (meth == SCUTE_NORMAL_FORM && (D->vd || D->ve));
  if (vera) {
    if (!L->A_sh || L->r_v <= 0)
      return fail(SCUTE_E_STATE, "scute_load_adapter: shared VeRA pair not set");
    scute_status st;
    if ((st = need(D->vd, "vd")) || (st = need(D->ve, "ve"))) return st;
    double cv = (meth == SCUTE_VERA) ? D->c : 1.0;
    vec_f32(D->vd, L->r_v, F.vd, 1.0);
    vec_f32(D->ve, d_out, F.ve, cv);
    F.flags |= F_VERA;
  }

  // ---- rotation slot: P = R - I ---------------------------------------------
  bool rot = (meth == SCUTE_OFT) || (meth == SCUTE_NORMAL_FORM && D->R);
  if (rot) {
    const int32_t blk = D->blk;
    if (blk <= 0 || blk > 256 || d_in % blk != 0)
      return fail(SCUTE_E_SHAPE, "scute_load_adapter: blk must be in [1, 256] and divide d_in");
    scute_status st;
    if ((st = need(meth == SCUTE_OFT ? D->Q : D->R, meth == SCUTE_OFT ? "Q" : "R"))) return st;
    F.blk = blk;
    F.P.resize((size_t)d_in * blk * es);
    if ((st = fold_rotation(L, dt, blk, meth == SCUTE_OFT ? D->Q : D->R, meth == SCUTE_OFT, F.P.data())))
      return st;
    F.flags |= F_R;
  }
  return SCUTE_OK;
}

}  // namespace

namespace {

// Lay out every folded slot in one allocation (256-byte aligned parts),
// upload it and publish the slot entry.
scute_status store_adapter(scute_layer* L, int32_t id, const FoldOut& F, int32_t method, void* stream) {
  // lay out every slot in one allocation, 256-byte aligned parts
  AdapterStore S;
  const size_t es = dtype_size(L->act);
  size_t lens[7] = {F.A.size(), F.B.size(), F.s.size() * 4, F.b.size() * 4,
                    F.vd.size() * 4, F.ve.size() * 4, F.P.size()};
  size_t off = 0;
  for (int i = 0; i < 7; ++i) {
    S.off[i] = off;
    S.len[i] = lens[i];
    off += (lens[i] + 255) & ~(size_t)255;
  }
  S.bytes = std::max<size_t>(off, 256);
  std::vector<uint8_t> host(S.bytes, 0);
  const void* srcs[7] = {F.A.data(), F.B.data(), F.s.data(), F.b.data(),
                         F.vd.data(), F.ve.data(), F.P.data()};
  for (int i = 0; i < 7; ++i)
    if (lens[i]) memcpy(host.data() + S.off[i], srcs[i], lens[i]);
  (void)es;

  if (L->device >= 0) {
    DeviceGuard g(L->device);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipMalloc(&S.mem, S.bytes);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(adapter)");
    e = hipMemcpyAsync(S.mem, host.data(), S.bytes, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      (void)hipFree(S.mem);
      return hip_fail(e, "upload adapter");
    }
  } else {
    S.mem = malloc(S.bytes);
    if (!S.mem) return fail(SCUTE_E_NOMEM, "scute_load_adapter: host allocation failed");
    memcpy(S.mem, host.data(), S.bytes);
  }

  SlotEntry E{};
  auto part = [&](int i) -> void* { return S.len[i] ? (uint8_t*)S.mem + S.off[i] : nullptr; };
  E.A = part(SCUTE_SLOT_A);
  E.B = part(SCUTE_SLOT_B);
  E.s = (const float*)part(SCUTE_SLOT_S);
  E.b = (const float*)part(SCUTE_SLOT_BIAS);
  E.vd = (const float*)part(SCUTE_SLOT_VD);
  E.ve = (const float*)part(SCUTE_SLOT_VE);
  E.P = part(SCUTE_SLOT_P);
  E.rank = F.rank;
  E.blk = F.blk;
  E.flags = F.flags | F_LOADED;
  E.method = method;

  if (L->device >= 0) {
    DeviceGuard g(L->device);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(L->table_dev + id, &E, sizeof(E), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      (void)hipFree(S.mem);
      return hip_fail(e, "upload slot entry");
    }
  }
  L->table[id] = E;
  L->store[id] = S;
  if (E.flags & F_VERA) L->n_vera_loaded++;
  L->epoch++;
  return SCUTE_OK;
}

// Arguments every load checks: a layer and a descriptor, an id in range
// and not occupied.
scute_status load_checks(const scute_layer* L, int32_t id, const void* D, const char* fn) {
  if (!L || !D) return fail(SCUTE_E_INVALID, std::string(fn) + ": null argument");
  if (id < 0 || id >= L->max_adapters) return fail(SCUTE_E_INVALID, std::string(fn) + ": id out of range");
  if (L->table[id].flags & F_LOADED) return fail(SCUTE_E_STATE, std::string(fn) + ": id is occupied");
  return SCUTE_OK;
}

}  // namespace

extern "C" scute_status scute_load_adapter(scute_layer* L, int32_t id, const scute_adapter_desc* D,
                                           const void* W_host, void* stream) {
  try {
    scute_status st = load_checks(L, id, D, "scute_load_adapter");
    if (st != SCUTE_OK) return st;
    FoldOut F;
    st = fold_adapter(L, D, W_host, F);
    if (st != SCUTE_OK) return st;
    return store_adapter(L, id, F, D->method, stream);
  } catch (const std::bad_alloc&) {
    return fail(SCUTE_E_NOMEM, "scute_load_adapter: host allocation failed");
  } catch (...) {
    return fail(SCUTE_E_INVALID, "scute_load_adapter: unexpected error");
  }
}

// A normal-form adapter with one rotation per projection of the layer: the
// descriptor's other slots fold as for scute_load_adapter, and the P slot
// holds n_proj rotations, (R_p - I)^T per block, one after another (a null
// R_p is the identity, stored as zeros). "How does Scute plug into vLLM?"
// (explainer): OFT gives the q, k and v projections their own rotations.
extern "C" scute_status scute_load_adapter_proj(scute_layer* L, int32_t id, const scute_adapter_desc* D,
                                                const void* const* R_proj, const void* W_host,
                                                void* stream) {
  try {
    scute_status st = load_checks(L, id, D, "scute_load_adapter_proj");
    if (st != SCUTE_OK) return st;
    if (L->n_proj < 2)
      return fail(SCUTE_E_STATE, "scute_load_adapter_proj: the layer has no projections");
    if (D->method != SCUTE_NORMAL_FORM || D->R)
      return fail(SCUTE_E_INVALID, "scute_load_adapter_proj: desc must be NORMAL_FORM with R null");
    if (!R_proj) return fail(SCUTE_E_INVALID, "scute_load_adapter_proj: R_proj is null");
    const int32_t blk = D->blk;
    if (blk <= 0 || blk > 256 || L->d_in % blk != 0)
      return fail(SCUTE_E_SHAPE, "scute_load_adapter_proj: blk must be in [1, 256] and divide d_in");
    if (dtype_size(D->dtype) == 0) return fail(SCUTE_E_INVALID, "scute_load_adapter_proj: bad desc dtype");
    FoldOut F;
    st = fold_adapter(L, D, W_host, F);
    if (st != SCUTE_OK) return st;
    const size_t one = (size_t)L->d_in * blk * dtype_size(L->act);
    F.blk = blk;
    F.P.assign(one * L->n_proj, 0);
    for (int32_t p = 0; p < L->n_proj; ++p)
      if ((st = fold_rotation(L, D->dtype, blk, R_proj[p], false, F.P.data() + one * p))) return st;
    F.flags |= F_R | F_RPROJ;
    return store_adapter(L, id, F, D->method, stream);
  } catch (const std::bad_alloc&) {
    return fail(SCUTE_E_NOMEM, "scute_load_adapter_proj: host allocation failed");
  } catch (...) {
    return fail(SCUTE_E_INVALID, "scute_load_adapter_proj: unexpected error");
  }
}

// Output column ranges that may take their own rotation (ends checked:
// increasing, all but the last on 64-column tiles, the last d_out); only
// while no adapter is loaded, so no stored rotation disagrees with them.
extern "C" scute_status scute_layer_set_projections(scute_layer* L, int32_t n_proj, const int64_t* col_end) {
  if (!L || !col_end) return fail(SCUTE_E_INVALID, "scute_layer_set_projections: null argument");
  if (n_proj < 1 || n_proj > MAX_PROJ)
    return fail(SCUTE_E_SHAPE, "scute_layer_set_projections: n_proj must be in [1, 4]");
  for (const SlotEntry& E : L->table)
    if (E.flags & F_LOADED)
      return fail(SCUTE_E_STATE, "scute_layer_set_projections: unload every adapter first");
  int64_t prev = 0;
  for (int32_t i = 0; i < n_proj; ++i) {
    const int64_t e = col_end[i];
    if (e <= prev || e > L->d_out || (i + 1 < n_proj && e % 64 != 0))
      return fail(SCUTE_E_SHAPE,
                  "scute_layer_set_projections: ends must increase, and all but the last be multiples of 64");
    prev = e;
  }
  if (prev != L->d_out) return fail(SCUTE_E_SHAPE, "scute_layer_set_projections: the last end must be d_out");
  L->n_proj = n_proj;
  for (int32_t i = 0; i < MAX_PROJ; ++i) L->proj_end[i] = i < n_proj ? col_end[i] : L->d_out;
  L->epoch++;
  return SCUTE_OK;
}

extern "C" scute_status scute_unload_adapter(scute_layer* L, int32_t id, void* stream) {
  if (!L) return fail(SCUTE_E_INVALID, "scute_unload_adapter: layer is null");
  if (id < 0 || id >= L->max_adapters)
    return fail(SCUTE_E_INVALID, "scute_unload_adapter: id out of range");
  if (!(L->table[id].flags & F_LOADED))
    return fail(SCUTE_E_STATE, "scute_unload_adapter: id is not loaded");
  if (L->device >= 0) {
    DeviceGuard g(L->device);
    hipStream_t s = (hipStream_t)stream;
    SlotEntry E{};
    SCUTE_HIP_CHECK(hipMemcpyAsync(L->table_dev + id, &E, sizeof(E), hipMemcpyHostToDevice, s));
    SCUTE_HIP_CHECK(hipStreamSynchronize(s));
  }
  if (L->table[id].flags & F_VERA) L->n_vera_loaded--;
  free_store(L, L->store[id]);
  L->table[id] = SlotEntry{};
  L->epoch++;
  return SCUTE_OK;
}

extern "C" scute_status scute_adapter_info_get(const scute_layer* L, int32_t id,
                                               scute_adapter_info* out) {
  if (!L || !out) return fail(SCUTE_E_INVALID, "scute_adapter_info_get: null argument");
  if (id < 0 || id >= L->max_adapters)
    return fail(SCUTE_E_INVALID, "scute_adapter_info_get: id out of range");
  const SlotEntry& E = L->table[id];
  out->loaded = (E.flags & F_LOADED) ? 1 : 0;
  out->method = out->loaded ? E.method : -1;
  out->rank = E.rank;
  out->blk = E.blk;
  out->has_R = !!(E.flags & F_R);
  out->has_s = !!(E.flags & F_S);
  out->has_b = !!(E.flags & F_B);
  out->has_term = !!(E.flags & F_TERM);
  out->has_vera = !!(E.flags & F_VERA);
  return SCUTE_OK;
}

extern "C" scute_status scute_read_slot(const scute_layer* L, int32_t id, int32_t slot, void* dst,
                                        int64_t dst_bytes) {
  if (!L || !dst) return fail(SCUTE_E_INVALID, "scute_read_slot: null argument");
  if (id < 0 || id >= L->max_adapters) return fail(SCUTE_E_INVALID, "scute_read_slot: bad id");
  if (slot < 0 || slot > 6) return fail(SCUTE_E_INVALID, "scute_read_slot: bad slot");
  if (!(L->table[id].flags & F_LOADED)) return fail(SCUTE_E_STATE, "scute_read_slot: not loaded");
  const AdapterStore& S = L->store[id];
  if (S.len[slot] == 0) return fail(SCUTE_E_STATE, "scute_read_slot: adapter has no such slot");
  if ((size_t)dst_bytes != S.len[slot])
    return fail(SCUTE_E_SHAPE, "scute_read_slot: dst_bytes must equal the slot size (" +
                                   std::to_string(S.len[slot]) + ")");
  const void* src = (const uint8_t*)S.mem + S.off[slot];
  if (L->device >= 0) {
    DeviceGuard g(L->device);
    SCUTE_HIP_CHECK(hipMemcpy(dst, src, S.len[slot], hipMemcpyDeviceToHost));
  } else {
    memcpy(dst, src, S.len[slot]);
  }
  if (slot == SCUTE_SLOT_P) {
    // storage holds (R - I)^T per block; hand back R - I
    const int32_t blk = L->table[id].blk;
    // (n_proj stacked rotations when the adapter rotates per projection)
    const size_t es = dtype_size(L->act), nb = S.len[slot] / ((size_t)blk * blk * es);
    std::vector<uint8_t> blkbuf((size_t)blk * blk * es);
    for (size_t kb = 0; kb < nb; ++kb) {
      uint8_t* b = (uint8_t*)dst + kb * blk * blk * es;
      memcpy(blkbuf.data(), b, blkbuf.size());
      for (int32_t i = 0; i < blk; ++i)
        for (int32_t j = 0; j < blk; ++j)
          memcpy(b + ((size_t)i * blk + j) * es, blkbuf.data() + ((size_t)j * blk + i) * es, es);
    }
  }
  return SCUTE_OK;
}
