/*
 * scute.h - C ABI of the normal-form batched adapter layer on MI355X (gfx950).
 *
 * The layer computes, for every token t of a batch whose tokens belong to
 * many adapters a = a(t) over one shared base weight W,
 *
 *   y_t = ((x_t R_a) W) (.) s_a + b_a + sum_k c_k (((x_t A_k) (.) d_k) B_k (.) e_k)
 *
 * (row vectors; "The big picture: six extra slots in the LoRA computation",
 * paper-daily.com explainer of "Scute: Exact Batched Serving for PEFT
 * Adapters Beyond LoRA"). LoRA, DoRA, (IA)^3, VeRA and OFT adapters are all
 * written in this normal form ("What problem is it solving?").
 *
 * Buffer conventions (PyTorch nn.Linear layout; the formula uses transposes):
 *   x     [n][d_in]    activation dtype, row-major
 *   W     [d_out][d_in] activation dtype, row-major (K contiguous)
 *   y     [n][d_out]   float32
 *   A     [rank][d_in]   B [d_out][rank]
 *   A_sh  [r_v][d_in]    B_sh [d_out][r_v]
 *   Q, R  [d_in/blk][blk][blk], block kb maps input i -> output j via
 *         out[kb*blk + j] = sum_i in[kb*blk + i] * M[kb][i][j]
 *
 * Errors: every call returns a scute_status; 0 is success. On failure a
 * thread-local message is available from scute_last_error() and the object
 * passed in is left as it was (still usable). No C++ exception crosses this
 * boundary. Device-side faults of asynchronous calls surface at the caller's
 * next synchronisation of the stream.
 *
 * Threading: one layer may run forwards on one stream at a time. Loads and
 * unloads must not overlap a forward on the same layer; the caller
 * serialises them.
 */
#ifndef SCUTE_H
#define SCUTE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t scute_status;

#define SCUTE_OK 0
#define SCUTE_E_INVALID (-1)     /* null pointer or bad argument value        */
#define SCUTE_E_SHAPE (-2)       /* sizes inconsistent with the layer         */
#define SCUTE_E_NOMEM (-3)       /* allocation failed or capacity exhausted   */
#define SCUTE_E_HIP (-4)         /* HIP runtime error                         */
#define SCUTE_E_STATE (-5)       /* wrong state: id occupied / not loaded,
                                    stale plan, shared VeRA pair not set      */
#define SCUTE_E_UNSUPPORTED (-6) /* valid request this build does not serve   */

typedef enum scute_dtype {
  SCUTE_F32 = 0,
  SCUTE_BF16 = 1, /* stored as uint16 bit patterns */
  SCUTE_F64 = 2
} scute_dtype;

typedef enum scute_method {
  SCUTE_LORA = 0,       /* y = xW + b + c (xA) B                                 */
  SCUTE_DORA = 1,       /* y = x W_D + b, W_D = (W + cAB) diag(m / colnorm(W+cAB)) */
  SCUTE_IA3 = 2,        /* y = (xW) (.) l + b  (l on the s slot)                 */
  SCUTE_VERA = 3,       /* y = xW + b + (((x A_sh) (.) d) B_sh) (.) (c e)        */
  SCUTE_OFT = 4,        /* y = (x R) W + b, R = blockdiag(Cayley(Q_k))           */
  SCUTE_NORMAL_FORM = 5 /* slots given directly: R, s, b, one own term, VeRA term */
} scute_method;

typedef struct scute_layer scute_layer;
typedef struct scute_batch scute_batch;

/*
 * One adapter as it comes from its method ("How does Scute plug into vLLM?":
 * the converter rewrites each checkpoint in the normal form at load).
 * Every array is a HOST pointer in `dtype` (SCUTE_F64, SCUTE_F32, or
 * SCUTE_BF16 as uint16). Arrays a method does not use are ignored; an
 * optional array left null takes its identity value (ones, zero, identity).
 */
typedef struct scute_adapter_desc {
  int32_t method; /* scute_method                                            */
  int32_t dtype;  /* element type of the host arrays below                   */
  int32_t rank;   /* rank r of the own low-rank term (LoRA, DoRA, NORMAL_FORM
                     with A and B); 0 = no own term                          */
  int32_t blk;    /* block size of Q (OFT) or R (NORMAL_FORM); divides d_in  */
  double c;       /* scalar c: of the own term (LoRA, DoRA, NORMAL_FORM), or
                     of the shared term (VeRA; the pages' VeRA uses c = 1)   */
  const void* A;  /* [rank][d_in]   own down factor                          */
  const void* B;  /* [d_out][rank]  own up factor                            */
  const void* d;  /* [rank]   NORMAL_FORM own-term d (null: ones)            */
  const void* e;  /* [d_out]  NORMAL_FORM own-term e (null: ones)            */
  const void* m;  /* [d_out]  DoRA learned column lengths                    */
  const void* l;  /* [d_out]  (IA)^3 vector                                  */
  const void* vd; /* [r_v]    VeRA d (VERA; NORMAL_FORM shared term)         */
  const void* ve; /* [d_out]  VeRA e                                         */
  const void* Q;  /* [d_in/blk][blk][blk] OFT skew-symmetric blocks          */
  const void* R;  /* [d_in/blk][blk][blk] NORMAL_FORM rotation blocks        */
  const void* s;  /* [d_out]  NORMAL_FORM s (null: ones)                     */
  const void* b;  /* [d_out]  shift b, any method (null: zero)               */
} scute_adapter_desc;

/* Per-batch algorithmic cost (the byte / FLOP model; "Where is the cheapest
 * place to compute the remaining slots?": adapter work is priced in bytes,
 * added time = extra bytes / bandwidth + extra launches x launch cost). */
typedef struct scute_cost {
  double bytes;         /* x + W + y + every touched adapter's stored factors
                           + shared VeRA pair once if any VeRA row           */
  double adapter_bytes; /* bytes minus x, W and y                            */
  double flops;         /* 2 n d_in d_out + own terms + VeRA terms + rotations */
  double base_flops;    /* 2 n d_in d_out                                    */
  int32_t launches;     /* kernel launches per forward                       */
  int32_t n_tokens;
  int32_t n_segments;   /* runs of one adapter after the stable sort         */
  int32_t n_rot_rows;   /* rows with a rotation slot (OFT)                   */
  int32_t n_vera_rows;  /* rows with a shared VeRA term                      */
  int32_t n_touched;    /* distinct adapters with at least one token         */
  /* the same bytes split by the step that needs them (x counted in both):  */
  double gemm_bytes;     /* base GEMM + expand: x, W, y, B', s, b, VeRA e, B_sh */
  double prologue_bytes; /* rotation + shrink: x, A', P, VeRA d, A_sh          */
  /* the flops split the same way:                                           */
  double gemm_flops;     /* 2 n d_in d_out + expands (t B', u B_sh)           */
  double prologue_flops; /* shrinks (x A', x A_sh) + rotations (x P)          */
} scute_cost;

/* Create a layer context for one (d_in, d_out, activation dtype, device).
 * device >= 0: HIP device ordinal; every forward runs there.
 * device == -1: host-only context (fold, plan and cost model only; the
 *   forward returns SCUTE_E_UNSUPPORTED). Used to test host logic without a
 *   GPU.
 * act_dtype: SCUTE_BF16 (bf16 inputs, fp32 accumulate) or SCUTE_F32.
 * max_adapters: adapter ids run 0 .. max_adapters-1.
 * The library owns everything it allocates; release with scute_layer_destroy. */
scute_status scute_layer_create(int32_t device, int64_t d_in, int64_t d_out,
                                int32_t act_dtype, int32_t max_adapters,
                                scute_layer** out);

/* Free the layer and every adapter it holds. The caller must have
 * synchronised every stream that used it. Plans built for it become invalid
 * and must still be destroyed. Null is accepted. */
scute_status scute_layer_destroy(scute_layer* layer);

/* Set the shared VeRA pair ("Which slots can be merged at load?": VeRA's A
 * and B are shared by every VeRA tenant, so d and e stay live; "How does
 * Scute plug into vLLM?": VeRA keeps a reference to the shared matrices).
 * A_sh [r_v][d_in] and B_sh [d_out][r_v] are DEVICE pointers in the
 * activation dtype, BORROWED: the caller keeps them alive and unchanged
 * while the layer is used. Must precede loading any adapter with a VeRA
 * term; may be replaced only while no VeRA adapter is loaded.
 * Host-only layers accept host pointers (not dereferenced). */
scute_status scute_set_vera_shared(scute_layer* layer, const void* A_sh,
                                   const void* B_sh, int32_t r_v);

/* Load adapter `id`: fold its slots ("Which slots can be merged at load?":
 * a slot next to a factor the adapter owns merges into it, a slot next to
 * shared W or the shared VeRA pair stays live), in fp64 on the host, then
 * store the folded factors in library-owned device memory:
 *   own term:  A' = c A diag(d), B' = B diag(e)  (activation dtype)
 *   DoRA:      s = m / colnorm(W + cAB) stays live on the base path and
 *              also folds into B' (e = s), c folds into A'
 *   (IA)^3:    s = l live     VeRA: d, c e live     OFT: P = R - I
 *   s, b, VeRA d and e are stored in float32.
 * W_host ([d_out][d_in] in desc->dtype, HOST pointer) is read only for
 * DoRA and may be null otherwise. `stream` orders the uploads (null: the
 * default stream); the call returns after they complete.
 * Errors: SCUTE_E_STATE if `id` is occupied or the VeRA pair is missing,
 * SCUTE_E_SHAPE for a bad rank / block size, SCUTE_E_INVALID for a missing
 * array, SCUTE_E_NOMEM if device memory runs out. */
scute_status scute_load_adapter(scute_layer* layer, int32_t id,
                                const scute_adapter_desc* desc,
                                const void* W_host, void* stream);

/* Split the layer's output columns into n_proj projections (at most 4) that
 * share x and are computed by one GEMM over the stacked weight, e.g. q, k
 * and v ("How does Scute plug into vLLM?", paper-daily.com explainer of
 * "Scute: Exact Batched Serving for PEFT Adapters Beyond LoRA": OFT gives
 * each projection its own input rotation, which is why Scute splits the
 * q / k / v GEMM when OFT is present; with this call one GEMM keeps them).
 * col_end[i] (HOST array) is the end column of projection i: increasing,
 * every end but the last a multiple of 64, the last equal to d_out.
 * Only while no adapter is loaded (SCUTE_E_STATE otherwise); plans built
 * before become stale. n_proj = 1 with col_end[0] = d_out undoes it.
 * Errors: SCUTE_E_SHAPE for bad ends or n_proj, SCUTE_E_INVALID for null. */
scute_status scute_layer_set_projections(scute_layer* layer, int32_t n_proj,
                                         const int64_t* col_end);

/* Load adapter `id` like scute_load_adapter, with one rotation per
 * projection of the layer: desc->method must be SCUTE_NORMAL_FORM with
 * desc->R null, and R_proj[p] (HOST pointer, [d_in/blk][blk][blk] in
 * desc->dtype, blk = desc->blk) is the rotation of projection p's input;
 * a null R_proj[p] is the identity. Output columns of projection p compute
 * ((x R_p) W) (.) s + b + the adapter's terms. Each P_p = R_p - I is stored
 * like the single rotation slot, the n_proj of them one after another
 * (scute_read_slot of SCUTE_SLOT_P returns n_proj d_in blk elements).
 * Batches with such rows run the two-launch decode path (bf16, up to 256
 * rows), the prefill path (bf16, when every projection ends on a multiple
 * of 256) or the generic kernels (so does scute_layer_forward_noalloc).
 * Errors: SCUTE_E_STATE if the layer has one projection or `id` is
 * occupied, SCUTE_E_INVALID for another method, a non-null desc->R or a
 * null R_proj, SCUTE_E_SHAPE for a bad block size; otherwise as
 * scute_load_adapter. */
scute_status scute_load_adapter_proj(scute_layer* layer, int32_t id,
                                     const scute_adapter_desc* desc,
                                     const void* const* R_proj,
                                     const void* W_host, void* stream);

/* Unload adapter `id` and free its memory after `stream` drains.
 * SCUTE_E_STATE if `id` is not loaded. Plans built before become stale. */
scute_status scute_unload_adapter(scute_layer* layer, int32_t id, void* stream);

/* Build the batch plan from a HOST array token_adapter[n] (-1: base path
 * only): a stable sort of tokens by adapter so that every run of rows
 * belongs to one adapter ("Where is the cheapest place...": each tile of
 * the expand belongs to one adapter; each row looks up its tenant's VeRA
 * vectors and rotation). Rows with a rotation slot come first, then rows
 * with a shared VeRA term, then the rest, each group ordered by adapter id
 * and token index. The plan is library-owned, sized workspaces included,
 * and may be reused for any number of forwards with the same assignment
 * until the layer's adapters change. n may be 0.
 * Errors: SCUTE_E_STATE if a token names an id that is not loaded. */
scute_status scute_plan_batch(scute_layer* layer, const int32_t* token_adapter,
                              int32_t n, void* stream, scute_batch** out);

/* Plan flags for scute_plan_batch_flags. */
typedef enum scute_plan_flag {
  /* every forward with the plan gives the same bits for the same inputs:
   * decode-size batches run the fused MFMA path, whose K slices and shrink
   * slices are added in a fixed order with no float atomics (the other
   * paths already add in a fixed order) */
  SCUTE_PLAN_DETERMINISTIC = 1,
  /* Route variants of the two-launch decode path, for the route comparison
   * and time model of "Where is the cheapest place to compute the remaining
   * slots?" (the default route fuses every step into the GEMM's prologue and
   * epilogue). Any of them plans the batch on that path (SCUTE_E_UNSUPPORTED
   * if it does not take the batch); results equal the default route's up to
   * the order of fp32 additions. */
  /* the GEMM writes x W only; s (applied inside the pass), b and the own
   * low-rank term follow in an expand pass, the VeRA term in its own pass */
  SCUTE_PLAN_ROUTE_EXPAND_PASS = 2,
  /* with EXPAND_PASS: s applied by a pass of its own before the expand
   * (s copied to every row, then multiplied into the output) */
  SCUTE_PLAN_ROUTE_SEPARATE_S = 4,
  /* the VeRA term in a pass of its own after the GEMM (whole batch, the
   * shared B_sh read once per 32 VeRA rows) */
  SCUTE_PLAN_ROUTE_VERA_PASS = 8,
  /* the OFT rotation in a pass of its own before the prologue */
  SCUTE_PLAN_ROUTE_ROTATE_PASS = 16
} scute_plan_flag;

/* scute_plan_batch with flags (a bitwise or of scute_plan_flag; 0 gives
 * scute_plan_batch). Errors as scute_plan_batch, plus SCUTE_E_INVALID for an
 * unknown flag bit, SEPARATE_S without EXPAND_PASS, or DETERMINISTIC with a
 * route bit, and SCUTE_E_UNSUPPORTED when a route bit is set and the batch
 * does not fit the two-launch decode path. */
scute_status scute_plan_batch_flags(scute_layer* layer, const int32_t* token_adapter,
                                    int32_t n, uint32_t flags, void* stream,
                                    scute_batch** out);

/* Free a plan (after the streams that used it are synchronised). Null ok.
 * The plan records its device when it is built, so it may be freed before
 * or after its layer. */
scute_status scute_batch_destroy(scute_batch* batch);

/* The forward pass on `stream` (null: default stream), asynchronous.
 * x [n][d_in] and W [d_out][d_in] are DEVICE pointers in the activation
 * dtype; y [n][d_out] is a DEVICE float32 pointer that is fully written.
 * All three are borrowed for the call. Every step runs in this library's
 * HIP kernels: OFT rotation, base GEMM with the s / b epilogue, own-term
 * shrink and expand, and the whole-batch shared VeRA term ("How does Scute
 * plug into vLLM?": four steps, the rotation before the GEMM).
 * Range: inputs must be finite; every intermediate (rotation, shrink
 * sums, GEMM partials, expand) is held in float32 (the shrink sums and
 * rotation output are rounded to the activation dtype once as MFMA
 * operands), so any input scale whose products and sums stay inside the
 * float32 range is served; there is no fixed-point stage.
 * Errors: SCUTE_E_STATE if the plan is stale or from another layer,
 * SCUTE_E_UNSUPPORTED on a host-only layer, SCUTE_E_INVALID for null or
 * misaligned pointers (16-byte alignment required). */
scute_status scute_layer_forward(scute_layer* layer, const scute_batch* batch,
                                 const void* x, const void* W, float* y,
                                 void* stream);

/* Bytes of the static device scratch that scute_layer_forward_noalloc uses
 * (one copy per device, held until the process ends). */
#define SCUTE_NOALLOC_SCRATCH_BYTES (16u << 20)

/* The forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * it needs no plan and allocates nothing. token_adapter is a DEVICE int32
 * array [n] (-1: base path only); x, W and y are as in scute_layer_forward.
 * The batch runs in token order on the generic kernels (the same arithmetic
 * as scute_layer_forward's generic path); the rotation output and shrink
 * sums live in the library's static scratch of SCUTE_NOALLOC_SCRATCH_BYTES
 * on the layer's device, which holds n * d_in * dtype_size (only when a
 * loaded adapter rotates) + n * max loaded rank * 4 + n * r_v * 4 (only when
 * a VeRA adapter is loaded) bytes, each part rounded up to 256. Every call on
 * a device shares that scratch and overwrites what it reads, so calls that
 * overlap on one device race: order them on one stream. Ids are checked on
 * the device: a row whose id is out of range or not loaded gets NaN.
 * Errors: SCUTE_E_SHAPE if n is outside [0, 65535] or the batch needs more
 * scratch than there is; SCUTE_E_INVALID for null or misaligned pointers
 * (16-byte x, W, y; 4-byte token_adapter); SCUTE_E_STATE if a VeRA adapter
 * is loaded and the shared pair is not set; SCUTE_E_UNSUPPORTED on a
 * host-only layer or a device index past 63. An adapter loaded with
 * scute_load_adapter_proj makes the rotation output one block of n rows
 * per projection (counted in the scratch a batch needs). */
scute_status scute_layer_forward_noalloc(scute_layer* layer, const int32_t* token_adapter,
                                         int32_t n, const void* x, const void* W, float* y,
                                         void* stream);

/* The FFN gate after the up projection: h = silu(g) (.) u element-wise, with
 * silu(z) = z / (1 + exp(-z)), the gate activation of the Llama models the
 * pages evaluate on. (IA)^3 multiplies the FFN intermediate
 * sigma(x W_g) (.) (x W_u) by l; products reorder, so l is the s slot of the
 * up projection ("The big picture: six extra slots in the LoRA
 * computation"), u is that layer's output and g the gate projection's.
 * g, u, h: DEVICE float32 arrays of `count` elements, h may be u; 16-byte
 * aligned. Errors: SCUTE_E_INVALID for null or misaligned pointers or
 * count < 0; SCUTE_E_HIP if the launch fails. */
scute_status scute_silu_gate(const float* g, const float* u, float* h, int64_t count, void* stream);

/* Algorithmic bytes / FLOPs / launches of one forward with this plan. */
scute_status scute_cost_model(const scute_layer* layer, const scute_batch* batch,
                              scute_cost* out);

/* ---- introspection (tests, debugging) ---------------------------------- */

typedef enum scute_slot {
  SCUTE_SLOT_A = 0,  /* folded A' [rank8][d_in]       activation dtype */
  SCUTE_SLOT_B = 1,  /* folded B' [d_out][rank8]      activation dtype
                        (rank8: the rank rounded up to a multiple of 8;
                        the added rows of A' and columns of B' are zero) */
  SCUTE_SLOT_S = 2,  /* live s [d_out]                float32          */
  SCUTE_SLOT_BIAS = 3, /* b [d_out]                   float32          */
  SCUTE_SLOT_VD = 4, /* VeRA d [r_v]                  float32          */
  SCUTE_SLOT_VE = 5, /* VeRA e, c folded [d_out]      float32          */
  SCUTE_SLOT_P = 6   /* R - I [d_in/blk][blk][blk]    activation dtype
                        (kept transposed per block on the device;
                        scute_read_slot returns R - I itself)         */
} scute_slot;

typedef struct scute_adapter_info {
  int32_t loaded;
  int32_t method;
  int32_t rank;  /* stored rank: the own term's rank rounded up to 8 (0: none) */
  int32_t blk;
  int32_t has_R, has_s, has_b, has_term, has_vera;
} scute_adapter_info;

scute_status scute_adapter_info_get(const scute_layer* layer, int32_t id,
                                    scute_adapter_info* out);

/* Copy one stored slot of adapter `id` to HOST memory `dst` of `dst_bytes`
 * bytes (must be exactly the slot's size). SCUTE_E_STATE if the adapter
 * does not hold that slot. */
scute_status scute_read_slot(const scute_layer* layer, int32_t id, int32_t slot,
                             void* dst, int64_t dst_bytes);

typedef struct scute_batch_info {
  int32_t n;
  int32_t n_segments;
  int32_t n_rot_rows;  /* rows 0 .. n_rot_rows-1 of the sorted order rotate */
  int32_t n_vera_rows;
  int32_t max_rank;
  int32_t path;        /* kernels the forward will run: 0 generic, 1 MFMA decode, 2 MFMA prefill */
} scute_batch_info;

scute_status scute_batch_info_get(const scute_batch* batch, scute_batch_info* out);

/* Whether a forward of this plan had a cross-work-group wait give up
 * (*out = 1) since the plan was built or last reset (*out = 0 otherwise).
 * Only the fused decode path waits across work-groups; its waits are bounded
 * (about 2^20 polls) and a wait that gives up records the failure and lets
 * the kernel finish instead of hanging, so that forward's output is not
 * valid. Call after synchronising the stream the forwards ran on; the read
 * is a blocking device-to-host copy. reset != 0 clears the flag afterwards.
 * Errors: SCUTE_E_INVALID for null pointers, SCUTE_E_HIP if the copy fails.
 * Plans on other paths always report 0. */
scute_status scute_batch_wait_failures(const scute_batch* batch, int32_t reset, int32_t* out);

/* Copy the plan's tables to HOST memory:
 *   perm[n]            token index at each sorted position
 *   seg[3*n_segments]  (adapter id, first sorted position, length) per run
 * Either pointer may be null. */
scute_status scute_batch_read(const scute_batch* batch, int32_t* perm, int32_t* seg);

/* ---- kernel timing (instrumentation) ------------------------------------ */

/* When enabled, every forward on this layer records a HIP event pair around
 * each of its kernel launches, on the forward's stream. Timings accumulate
 * per kernel name until read. Costs a little launch overhead; off by default. */
scute_status scute_profile_enable(scute_layer* layer, int32_t enable);

typedef struct scute_kernel_time {
  char name[32];     /* kernel role, e.g. "gemm"                           */
  int32_t launches;  /* launches timed since the last read                 */
  double total_ms;   /* summed event-to-event time of those launches       */
} scute_kernel_time;

/* Wait for the recorded events, write up to `capacity` per-kernel totals to
 * HOST memory `out`, set *count to the number of kernel names, and reset
 * the totals. */
scute_status scute_profile_read(scute_layer* layer, scute_kernel_time* out, int32_t capacity,
                                int32_t* count);

/* Launch `count` empty kernels (one wave each) back to back on `stream`
 * (null: default stream) on the current device, for the launch-cost term of
 * the time model in "Where is the cheapest place to compute the remaining
 * slots?" (added time = extra bytes / bandwidth + extra launches x launch
 * cost): the caller times them with events. Errors: SCUTE_E_INVALID if
 * count < 0; SCUTE_E_HIP if a launch fails. */
scute_status scute_launch_empty(int32_t count, void* stream);

/* Thread-local message of the last failed call on this thread ("" if none). */
const char* scute_last_error(void);

/* Library version string. */
const char* scute_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SCUTE_H */
