// Internal definitions shared by the host runtime and the HIP kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/scute.h"

namespace scute {

// flags of one adapter's live-slot entry
enum : int32_t {
  F_LOADED = 1,
  F_R = 2,     // rotation slot (P = R - I stored)
  F_S = 4,     // live s
  F_B = 8,     // shift b
  F_TERM = 16, // own low-rank term (A', B')
  F_VERA = 32, // shared VeRA term (d, e live)
  F_RPROJ = 64, // one rotation per projection: P holds n_proj stacked (R_p - I)
};

// Projections of a layer: output column ranges that share x and W's rows
// but may each take their own input rotation (q, k and v over one stacked
// weight). proj_end[i] is the end of projection i; at most 4.
constexpr int32_t MAX_PROJ = 4;

// Device-visible live-slot entry of one adapter (struct of pointers into
// the adapter's library-owned storage). Unused pointers are null.
struct SlotEntry {
  const void* A;   // A' [rank][d_in]   act dtype
  const void* B;   // B' [d_out][rank]  act dtype
  const void* P;   // R - I [d_in/blk][blk][blk] act dtype
  const float* s;  // [d_out]
  const float* b;  // [d_out]
  const float* vd; // [r_v]
  const float* ve; // [d_out]
  int32_t rank;
  int32_t blk;
  int32_t flags;
  int32_t method;
};

struct AdapterStore {
  void* mem = nullptr;  // one allocation holding every slot (device or host)
  size_t bytes = 0;
  size_t off[7] = {0, 0, 0, 0, 0, 0, 0};  // offsets per scute_slot
  size_t len[7] = {0, 0, 0, 0, 0, 0, 0};  // byte sizes per scute_slot
};

}  // namespace scute

namespace scute {
struct ProfEvent {
  int32_t kind;
  hipEvent_t start, stop;
};
}  // namespace scute

struct scute_layer {
  int32_t device = -1;
  int64_t d_in = 0, d_out = 0;
  int32_t act = SCUTE_BF16;
  int32_t max_adapters = 0;
  int32_t n_proj = 1;                   // output column ranges (scute_layer_set_projections)
  int64_t proj_end[scute::MAX_PROJ] = {0, 0, 0, 0};
  std::vector<scute::SlotEntry> table;  // host mirror
  std::vector<scute::AdapterStore> store;
  scute::SlotEntry* table_dev = nullptr;
  const void* A_sh = nullptr;
  const void* B_sh = nullptr;
  int32_t r_v = 0;
  int32_t n_vera_loaded = 0;
  uint64_t epoch = 1;  // bumps on every load / unload
  int32_t num_cu = 0;
  // facts of the loaded adapters for the token-order forward, as of na_epoch
  uint64_t na_epoch = 0;
  int32_t na_max_rank = 0;
  bool na_rot = false;
  bool na_rproj = false;  // some loaded adapter rotates per projection
  // kernel timing (scute_profile_enable)
  bool profiling = false;
  std::vector<scute::ProfEvent> prof_pending;
  std::vector<hipEvent_t> prof_pool;
  std::vector<std::string> prof_names;
  std::vector<double> prof_ms;
  std::vector<int32_t> prof_count;
};

namespace scute {

// Tables and workspaces of the MFMA decode path (bf16, small batches).
// Row of a decode batch (sorted position) as the main kernel's epilogue
// reads it: the factor vectors of the row's adapter, with shared dummies
// (ones for s and e, zeros for b) where the slot is absent, so every row is
// handled by the same branch-free code. 32 bytes.
struct DecRow {
  const float* s;   // live s, or ones
  const float* e;   // VeRA e, or ones
  const float* b;   // shift b, or zeros
  int32_t tok;      // token written by the row, -1 past n
  int32_t flags;    // 1: the row has a VeRA term
};

// Prologue work item (one per wave), pointers and tokens resolved at plan
// time. 48 bytes.
//   gather:      p0 = sorted row, tok[0] = its token
//   rotation:    p0, n, tok as above, k = first of 64 columns,
//                ptr = (R - I)^T blocks, blk = block size
//   own shrink:  p0, n, tok as above, k = first rank | ranks (<= 4) << 16,
//                ptr = A', blk = K part (1024 wide)
//   VeRA shrink: p0 = block of 32 VeRA rows, n = block of 32 ranks,
//                k = K slice (256 wide)
enum : int32_t { PRO_ROT = 0, PRO_SHRINK = 1, PRO_VSHRINK = 2, PRO_GATHER = 3 };
// One 16-rank step of the decode main kernel's expand: an MFMA step over
// ranks [kk, kk + 16) of one row group's own term (t B' against the
// adapter's B') or shared VeRA term (u B_sh). 32 bytes.
//   gk   kind (STEP_VERA) | group << 8
//   kk   first rank of the step; rank = length of a B row (the term's rank)
//   lohi sorted rows [lo, hi) of the group the step contributes to
//   bp   B' of the adapter, or B_sh
enum : int32_t { STEP_VERA = 1 };
struct DecStep {
  int32_t gk, kk, rank, lohi;
  const uint16_t* bp;
  int64_t pad;
};
struct DecProItem {
  int32_t type, p0, n, k;
  int32_t tok[4];
  const uint16_t* ptr;
  int32_t blk, pad;
};

// VeRA row of a decode batch: d of its adapter, its token and sorted
// position (-1 on padding rows, which repeat a valid token and d). 16 bytes.
struct DecVeraRow {
  const float* vd;
  int32_t tok;
  int32_t p;
};

struct FdRotItem;
// Route-pass chunk: sorted rows p0 .. p0 + n - 1 (n <= 16) of adapter a.
struct RtChunk {
  int32_t p0, n, a, pad;
};

struct DecodePlan {
  bool enabled = false;
  int32_t MG = 0;       // row groups of 32 covering the n sorted rows
  int32_t g_rot = 0;    // row groups of delta rows (rotated rows first)
  int32_t M_pad = 0;    // 32 * MG
  int32_t RT = 0;       // own-term ranks per row in the shrink buffer (max rank, to 16)
  int32_t AW = 0;       // shrink buffer row: RT own ranks, then r_v VeRA ranks
  int32_t S = 1;        // K slices of the base GEMM (1, 2 or 4)
  int32_t C = 0;        // column tiles of 64 outputs
  int32_t k_chunk = 0;  // d_in / S
  int32_t n_pro = 0;    // prologue work items
  // the first n_vitems prologue items are the VeRA shrinks, item
  // (kv nvb + vb) njb + jb covering K slice kv, VeRA rows 32 vb.., ranks 32 jb..
  int32_t n_vitems = 0, nvb = 0, njb = 0;
  int32_t n_steps = 0;
  // dense VeRA expand: row groups [gv0, gv1) hold every VeRA row; slice k
  // multiplies their shrink sums over its share of the r_v / 16 rank steps
  // (staged in LDS) instead of VeRA steps (gv1 == gv0: no dense expand)
  int32_t gv0 = 0, gv1 = 0;
  // [2 S MG + 1] step ranges: slice k, row group g (q = k MG + g) has own
  // steps [goff[2q], goff[2q+1]) and VeRA steps [goff[2q+1], goff[2q+2])
  const int32_t* goff = nullptr;
  const DecRow* rows = nullptr;          // [M_pad]
  const DecProItem* pro_items = nullptr; // [n_pro]
  const DecVeraRow* vrows = nullptr;     // [32 nvb]
  const DecStep* steps = nullptr;        // [n_steps]
  const float* zeros = nullptr;          // [d_out] of 0.0f
  uint16_t* xs = nullptr;     // [M_pad + 32 g_rot np][d_in] bf16: sorted x rows, then delta rows
                              // of each projection in turn
  int32_t np = 1;             // delta row blocks (the layer's projections when a row's
                              // adapter rotates per projection, else 1)
  int32_t ptile[MAX_PROJ - 1] = {0, 0, 0};  // first column tile of projections 1.. (C past the last)
  float* acc32[2] = {nullptr, nullptr};  // per parity: [M_pad][AW] fp32 shrink sums
  float* part = nullptr;      // [S][C][M_pad][64] split-K partial tiles (S > 1)
  int32_t* cnt = nullptr;     // [C] arrival counters (kept at zero)
  uint32_t acc_bytes = 0, part_bytes = 0;
  // forwards launched with this plan; the shrink sums alternate between the
  // two acc32 buffers, and each forward's prologue clears the other one
  mutable uint32_t fwd = 0;
  // route variant (SCUTE_PLAN_ROUTE_* bits; 0: everything fused)
  uint32_t route = 0;
  const FdRotItem* rot = nullptr;  // rotation pass items (ROTATE_PASS)
  int32_t n_rot_items = 0, rot_blk = 0;
  const RtChunk* chunks = nullptr;  // expand pass chunks (EXPAND_PASS)
  int32_t n_chunks = 0;
  float* S_rows = nullptr;          // [n][d_out] s copied to every row (SEPARATE_S)
};

// ---- fused decode path (fdecode.hip / plan_fdecode.cpp) --------------------
// Staged x row of a decode batch (sorted position): the factor vectors of the
// row's adapter (shared ones / zeros where a slot is absent, so every row runs
// the same branch-free code), the y row it writes and the x row it stages.
// 48 bytes.
enum : int32_t { FR_S = 1, FR_E = 2, FR_B = 4, FR_VERA = 8 };
struct FdRow {
  const float* s;  // live s, or ones
  const float* e;  // VeRA e, or ones
  const float* b;  // shift b, or zeros
  const float* d;  // VeRA d, or zeros
  int32_t tok;     // y row written (-1: padding row)
  int32_t src;     // x row staged (padding rows repeat a valid token)
  int32_t flags;   // FR_* of the live slots
  int32_t rank;    // rank of the row's own term (0: none)
};
// One 16-rank step of an own term's expand: ranks [kk, kk + 16) of the
// term of rank `rank`, for sorted rows [lo, hi) of row group g, against
// B' = bp. 32 bytes.
struct FdStep {
  int32_t kk, rank, lo, hi;
  const uint16_t* bp;
  int32_t g, pad;
};
// Shrink block: 32 rank rows (rows of adapters' A', or of the shared A_sh)
// multiplied with the x rows of one row group in the GEMM's K loop. Rank row
// m's sums go to column col[m] of the shrink buffer for the sorted rows in
// [lohi[m] & 0xFFFF, lohi[m] >> 16) (own ranks) or for every VeRA row of the
// group (vera). 768 bytes.
struct FdXBlock {
  const uint16_t* arow[32];
  int32_t col[32];   // -1: unused rank row
  int32_t lohi[32];
  int32_t g, vera;
  int32_t pad[62];
};
// Rotation item: rows p0 .. p0 + n - 1 (n <= 4, one adapter; tokens tok[])
// by the item's columns from c0, P = (R - I)^T blocks of size blk. 48 bytes.
struct FdRotItem {
  int32_t p0, n, c0, blk;
  int32_t tok[4];
  const uint16_t* P;
  int64_t pad;
};

struct FdPlan {
  bool enabled = false;
  int32_t MG = 0, g_rot = 0, MGT = 0, M_pad = 0;
  int32_t S = 1, C = 0, NST = 0;   // K slices, 128-column tiles, 64-k stages per slice
  int32_t CG = 0;                  // column tiles of the grid (C, or more to carry every shrink block)
  int32_t RT = 0, AW = 0;          // shrink buffer row: RT own ranks, then r_v VeRA ranks
  int32_t gv0 = 0, gv1 = 0;        // row groups holding VeRA rows
  int32_t n_rot_items = 0;
  int32_t rot_blk = 0;             // block size of every rotation item (8..64), or 0: mixed
  int32_t rot_cols = 0;            // columns per rotation item (256 for blocks of 64, else 512)
  int32_t n_xb = 0;                // shrink blocks (block j rides on wave j / CG of tile j % CG)
  const FdRow* rows = nullptr;     // [M_pad]
  const FdStep* steps = nullptr;   // own expand steps by row group
  const int32_t* goff = nullptr;   // [MG + 1]: group g's steps [goff[g], goff[g+1])
  const int32_t* xoff = nullptr;   // [MG + 1]: group g's shrink blocks [xoff[g], xoff[g+1])
  const FdXBlock* xb = nullptr;    // [n_xb]
  const FdRotItem* rot = nullptr;  // [n_rot_items]
  uint16_t* acc = nullptr;         // [M_pad][AW] finished shrink sums, rounded to bf16
  float* xpart = nullptr;          // [n_xb][S][4 KB] the slices' partial shrink tiles
  int32_t* xcnt = nullptr;         // [n_xb] block arrival counters (never reset)
  uint32_t* xdone = nullptr;       // [n_xb] forward number whose sums the block holds
  float* part = nullptr;           // [C][S][MG][4][4 KB] split-K partial pieces
  int32_t* cnt = nullptr;          // [C][MG][4] arrival counters (never reset)
  int32_t* err = nullptr;          // bounded waits that gave up (scute_batch_wait_failures)
  int32_t spin_limit = 1 << 20;    // polls before a wait gives up
  uint32_t wait_bias = 0;          // 1: the waits look for a forward that never comes (tests)
  uint32_t acc_bytes = 0, part_bytes = 0, xpart_bytes = 0;
  mutable uint32_t fwd = 0;        // forwards launched with this plan
};

// Chunk of a prefill batch: the rows of one adapter segment (or of rows
// without an adapter) that one row tile of the prefill GEMM covers: up to 128
// tokens, or up to 64 tokens followed by their 64 Delta rows when the adapter
// rotates (the Delta rows fold into the token rows in registers); always 128
// staged rows. Every live slot is uniform over the chunk; absent factor
// vectors point at shared ones (s, e) and zeros (b). 64 bytes.
struct PfChunk {
  int32_t x0;          // sorted position of the chunk's first token
  int32_t nx;          // tokens in the chunk
  int32_t rows;        // token rows held by the tile (128, or 64 with rotation)
  int32_t flags;       // PF_* below
  const float* s;      // live s, or ones
  const float* e;      // VeRA e, or ones
  const float* b;      // shift b, or zeros
  const uint16_t* Bp;  // own B' [d_out][rank], or null
  int32_t rank;        // own rank (0 without an own term)
  int32_t pad[3];
};
enum : int32_t { PF_OWN = 1, PF_VERA = 2, PF_ROT = 4 };

// Prologue item of the prefill path (one work-group of 4 waves each):
//   shrink:      rows p0 .. p0 + n - 1 (sorted positions, n <= 64) x own
//                ranks (k & 0xFFFF) .. + (k >> 16) (<= 64) of A' = ptr, over
//                K part blk (1024 wide)
//   VeRA shrink: VeRA rows 64 p0 .. + 63 (of the VeRA row table) x ranks
//                (k & 0xFFFF) .. + 63 of A_sh over K part blk, scaled by d
//   (shrinks: pad = the tile's arrival counter)
//   rotation:    Delta rows p0 .. p0 + n - 1 (n <= 32) x columns k .. k + 255,
//                ptr = (R - I)^T blocks of size blk
// 32 bytes.
enum : int32_t { PP_SHRINK = 0, PP_VSHRINK = 1, PP_ROT = 2 };
struct PfProItem {
  int32_t type, p0, n, k;
  const uint16_t* ptr;
  int32_t blk, pad;
};

struct PrefillPlan {
  bool enabled = false;
  int32_t n_chunks = 0;
  int32_t C = 0;        // column tiles of 256 outputs
  // work-groups of the main kernel: {column tile, chunk, K part (-1: the
  // whole K), exchange slot}; whole tiles first, then P parts of each tile
  // of the remainder
  const int4* items = nullptr;
  int32_t n_items = 0;
  int32_t P = 1;        // K parts of a split tile (1, 2 or 4)
  int32_t n_split = 0;  // split tiles
  float* part = nullptr;      // [n_split][P][32][256] f32x4 partial tiles
  int32_t* cnt = nullptr;     // [n_split] arrival counters (kept at zero)
  uint32_t part_bytes = 0;
  int32_t RT = 0;       // own-term ranks per row in the shrink buffer (max rank, to 16)
  int32_t AW = 0;       // shrink buffer row: RT own ranks, then r_v VeRA ranks
  int32_t n_pro = 0;    // prologue work items
  const PfChunk* chunks = nullptr;        // [n_chunks]
  const int32_t* crow = nullptr;          // [n_chunks][128] staged row sources
  const PfProItem* pro_items = nullptr;  // shrinks, rotation
  const DecVeraRow* vrows = nullptr;     // [64 nvb]
  // [shrink tiles][K parts][64 x 64] fp32 partial shrink tiles, added in
  // part order by the last part of a tile to arrive
  float* tpart = nullptr;
  uint32_t tpart_bytes = 0;
  uint16_t* tbf = nullptr;    // [n][AW] the finished sums in bf16 (the expand's A operand)
  int32_t* tcnt = nullptr;    // [shrink tiles] arrival counters of the K parts (kept at zero)
  uint32_t tbf_bytes = 0;
};

}  // namespace scute

struct scute_batch {
  uint32_t flags = 0;  // scute_plan_flag bits
  const scute_layer* layer = nullptr;  // compared only: the layer may be destroyed first
  int32_t device = -1;                 // device of the allocations below (-1: none)
  uint64_t epoch = 0;
  int32_t n = 0;
  int32_t n_rot = 0;      // sorted positions [0, n_rot) carry a rotation
  int32_t n_vera = 0;     // rows with a VeRA term
  int32_t max_rank = 0;   // largest own-term rank among touched adapters
  int32_t n_touched = 0;
  bool rproj = false;     // some row's adapter rotates per projection (F_RPROJ)
  // host tables
  std::vector<int32_t> perm;         // [n] token at sorted position
  std::vector<int32_t> row_adapter;  // [n] adapter of sorted position (-1)
  std::vector<int32_t> seg;          // [3 * nseg] (adapter, start, len)
  std::vector<int32_t> vera_pos;     // [n_vera] sorted positions with VeRA
  // device copies (one allocation) and workspaces
  void* dev = nullptr;
  int32_t* d_perm = nullptr;
  int32_t* d_row_adapter = nullptr;
  int32_t* d_seg = nullptr;
  int32_t* d_vera_pos = nullptr;
  void* ws = nullptr;         // workspace allocation
  void* delta = nullptr;      // [np][n_rot][d_in] act dtype: x (R_p - I), np = the layer's
                              // projections when rproj, else 1
  float* t = nullptr;         // [n][max_rank]  own-term shrink
  float* u = nullptr;         // [n][r_v] VeRA shrink scaled by d (rows with VeRA)
  void* fast_dev = nullptr;   // decode-path tables + workspaces (one allocation)
  scute::DecodePlan dp;
  void* pf_dev = nullptr;     // prefill-path tables + workspaces (one allocation)
  scute::PrefillPlan pp;
  void* fd_dev = nullptr;     // fused decode tables + workspaces (one allocation)
  scute::FdPlan fp;
  int32_t nseg() const { return (int32_t)(seg.size() / 3); }
};

namespace scute {

// error reporting (thread-local message)
scute_status fail(scute_status code, const std::string& msg);
scute_status hip_fail(hipError_t e, const char* what);
#define SCUTE_HIP_CHECK(expr)                                   \
  do {                                                          \
    hipError_t _e = (expr);                                     \
    if (_e != hipSuccess) return ::scute::hip_fail(_e, #expr);  \
  } while (0)

size_t dtype_size(int32_t dt);

// no-allocation forward (forward.hip): takes the device address of its
// static scratch on `device` (current), once per device
scute_status noalloc_setup(int32_t device);

// forward launcher (forward.hip)
scute_status launch_forward(scute_layer* L, const scute_batch* B, const void* x,
                            const void* W, float* y, hipStream_t stream,
                            int32_t* launches_out);
int32_t forward_launch_count(const scute_layer* L, const scute_batch* B);

// Decode path selection (environment SCUTE_DECODE, read when a batch is
// planned): 0 = generic kernels only, 1 = the fused single-kernel path
// (fdecode.hip), 2 = the two-launch path (decode.hip). Unset: the fused path
// for batches of at least FUSED_MIN_GROUPS staged row groups in which no row
// has an own low-rank term, the two-launch path (DECODE_DEFAULT) otherwise.
// Measured on MI355X: with 7 or more row groups the two-launch kernel keeps
// only a 2-slot ring of 64-column tiles, while the fused kernel's
// 128-column tiles feed four column blocks from each staged row; the fused
// kernel's extra work is its in-loop shrink blocks, which own terms add per
// adapter (256 (IA)^3 / VeRA rows: 86 against 91 us at 4096 -> 14336, 73
// against 91 us at 11008; 256 LoRA rows: 95 against 83 us).
constexpr int DECODE_DEFAULT = 2;
constexpr int FUSED_MIN_GROUPS = 7;

// decode path (decode.hip / plan.cpp)
scute_status build_decode_plan(const scute_layer* L, scute_batch* B, hipStream_t st);
scute_status launch_decode(scute_layer* L, const scute_batch* B, const void* x, const void* W,
                           float* y, hipStream_t st, int32_t* launches);

// fused decode path (fdecode.hip / plan_fdecode.cpp)
scute_status build_fdecode_plan(const scute_layer* L, scute_batch* B, hipStream_t st);
scute_status launch_fdecode(scute_layer* L, const scute_batch* B, const void* x, const void* W,
                            float* y, hipStream_t st, int32_t* launches);

// route passes of the decode path (routes.hip)
constexpr uint32_t ROUTE_MASK = SCUTE_PLAN_ROUTE_EXPAND_PASS | SCUTE_PLAN_ROUTE_SEPARATE_S |
                                SCUTE_PLAN_ROUTE_VERA_PASS | SCUTE_PLAN_ROUTE_ROTATE_PASS;
int32_t decode_route_launches(const scute_batch* B);
scute_status launch_route_rotate(scute_layer* L, const scute_batch* B, const void* x, hipStream_t st,
                                 int32_t* nl);
scute_status launch_route_passes(scute_layer* L, const scute_batch* B, float* y, const float* acc,
                                 hipStream_t st, int32_t* nl);

// rotation pass (rotate.hip): items of up to 4 rows by 512 columns (256 for
// blocks of 64); blk the block size shared by every item, or 0 for mixed
// sizes (scalar form)
scute_status launch_rotate_items(const FdRotItem* items, int32_t n_items, int32_t blk, const uint16_t* x,
                                 uint16_t* dx, int32_t d_in, hipStream_t st);

// prefill path (prefill.hip / plan_prefill.cpp)
scute_status build_prefill_plan(const scute_layer* L, scute_batch* B, hipStream_t st);
scute_status launch_prefill(scute_layer* L, const scute_batch* B, const void* x, const void* W,
                            float* y, hipStream_t st, int32_t* launches);

// Arguments of the decode path's prologue kernel (decode.hip).
struct ProArgs {
  const uint16_t* x;
  const DecProItem* items;
  int32_t n_items;
  int32_t n_vitems, nvb, njb;  // VeRA shrink items first, indexed arithmetically
  const DecVeraRow* vrows;  // [32 nvb]
  const uint16_t* A_sh;     // [r_v][d_in]
  uint16_t* xs;             // [M_pad + 32 g_rot][d_in] sorted x rows, then delta rows
  float* acc;               // [M_pad][AW] this forward's shrink sums (zero on entry)
  float* acc_next;          // the other buffer, cleared for the next forward
  uint32_t acc_words;       // M_pad * AW (a multiple of 4)
  int32_t M_pad, AW, RT;
  int32_t d_in;
};
void launch_prologue(const ProArgs& pa, int grid, hipStream_t st, hipEvent_t e0, hipEvent_t e1);

// Kernel timing: when the layer has profiling on, bracket each launch with a
// HIP event pair on the launch stream.
// in_launch: the launch records the pair itself (hipExtLaunchKernelGGL with
// ev_start() / ev_stop()), so the pair times the kernel's execution, as a
// kernel trace does, without the dispatch around it.
struct ProfScope {
  scute_layer* L;
  hipStream_t st;
  ProfEvent ev{};
  bool on = false, in_launch = false;
  ProfScope(scute_layer* L_, hipStream_t st_, const char* name, bool in_launch_ = false)
      : L(L_), st(st_), in_launch(in_launch_) {
    if (!L->profiling) return;
    int32_t kind = -1;
    for (size_t i = 0; i < L->prof_names.size(); ++i)
      if (L->prof_names[i] == name) kind = (int32_t)i;
    if (kind < 0) {
      kind = (int32_t)L->prof_names.size();
      L->prof_names.push_back(name);
      L->prof_ms.push_back(0.0);
      L->prof_count.push_back(0);
    }
    ev.kind = kind;
    for (hipEvent_t* e : {&ev.start, &ev.stop}) {
      if (!L->prof_pool.empty()) {
        *e = L->prof_pool.back();
        L->prof_pool.pop_back();
      } else if (hipEventCreate(e) != hipSuccess) {
        return;
      }
    }
    on = in_launch || hipEventRecord(ev.start, st) == hipSuccess;
  }
  hipEvent_t ev_start() const { return on ? ev.start : nullptr; }
  hipEvent_t ev_stop() const { return on ? ev.stop : nullptr; }
  ~ProfScope() {
    if (!on) return;
    if (in_launch || hipEventRecord(ev.stop, st) == hipSuccess) L->prof_pending.push_back(ev);
  }
};

}  // namespace scute
