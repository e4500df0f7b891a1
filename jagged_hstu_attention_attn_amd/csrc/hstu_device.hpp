// hstu_device.hpp -- shared definitions of the gfx950 jagged HSTU attention
// kernels: tile sizes, sequence/mask geometry, work-list layout, kernel
// argument blocks.
//
// Mask geometry.  The four rules named on the "HSTU-MUSA" page (section
// "Mathematical Equivalence") plus the causal indicator of the teaching
// equation ("HSTU tensor by tensor", section "Similar shape, different
// aggregation") reduce, for every query row i, to one contiguous key interval
// [lo_i, hi_i] plus, for candidate rows, the row's own position:
//   prefix rows    i <  c       : [max(0, i-W), c-1]
//   history rows   c <= i < n_h : [max(0, i-W), i]
//   candidate rows i >= n_h     : [max(0, n_h-W), n_h-1]  and  j == i
// (the max(0, . - W) term only when W > 0; p_i = min(i, n_h) is the clamped
// candidate position).  lo_i is nondecreasing in i, which lets a query tile
// bound its key range by its first and last rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

constexpr int kBM = 128;        // query rows per work item: 4 waves x 32 rows
constexpr int kBN = 32;         // keys per staged K/V tile (one 32-key MFMA block)
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kPosMax = 8192;   // longest supported position table
constexpr int kPlanThreads = 1024;
constexpr int kPlanLdsSeqs = 2048;  // batches up to this many sequences plan from LDS
constexpr int kEmptyLo = 0x40000000;  // lower bound of an empty key interval

struct SeqGeom {
  int L;    // tokens in the sequence
  int n_h;  // history tokens (L minus clamped candidates)
  int c;    // bidirectional prefix tokens (clamped to n_h)
  int W;    // max attention length (0 = unlimited)
};

__host__ __device__ inline int clampi(int x, int lo, int hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

__host__ __device__ inline SeqGeom seq_geom(int L, int num_targets, int contextual_len, int W) {
  SeqGeom g;
  g.L = L;
  g.n_h = L - clampi(num_targets, 0, L);
  g.c = clampi(contextual_len, 0, g.n_h);
  g.W = W;
  return g;
}

// Allowed keys of row i: (unsigned)(j - lo) <= (unsigned)span, or j == self_j.
struct RowBounds {
  int lo;
  int span;    // hi - lo; an empty interval is lo = kEmptyLo, span = 0
  int self_j;  // i for candidate rows, -1 otherwise
};

__host__ __device__ inline RowBounds row_bounds(const SeqGeom& g, int i) {
  int lo = 0, hi, p = i, self_j = -1;
  if (i < g.c) {
    hi = g.c - 1;
  } else if (i < g.n_h) {
    hi = i;
  } else {
    hi = g.n_h - 1;
    p = g.n_h;
    self_j = i;
  }
  if (g.W > 0 && p - g.W > lo) lo = p - g.W;
  RowBounds r;
  if (hi < lo) {
    r.lo = kEmptyLo;
    r.span = 0;
  } else {
    r.lo = lo;
    r.span = hi - lo;
  }
  r.self_j = self_j;
  return r;
}

// Key range [jlo, jhi] that rows [i0, i1) (i0 < i1 <= L) can reach.
__host__ __device__ inline void tile_key_range(const SeqGeom& g, int i0, int i1, int& jlo,
                                               int& jhi) {
  const int p0 = i0 < g.n_h ? i0 : g.n_h;
  jlo = (g.W > 0 && p0 - g.W > 0) ? p0 - g.W : 0;
  jhi = i1 - 1;
  if (i0 < g.c && g.c - 1 > jhi) jhi = g.c - 1;
}

// Work list.  The scheduler lists the (sequence, head, query tile) items
// sequence by sequence, the tiles of one (sequence, head) together, deals them
// round-robin to the workgroups of the persistent attention launch and cuts
// the dealt order into equal-cost shares (cost = key tiles plus a fixed
// per-item term), placing consecutive shares on one XCD (the MI355X
// dispatches workgroup g to XCD g % 8; each XCD has its own L2) so that the
// workgroups running side by side work on neighbouring query tiles, which
// share most of their keys and values.  An item a share boundary cuts is
// split along its key tiles into chunks.  The aggregation is a plain sum over
// keys, so every chunk writes its fp32 partial output and the chunk that
// finishes last adds them in chunk order and runs the epilogue.
constexpr int kXcds = 8;
constexpr int kMaxGrid = 1024;      // most workgroups one plan serves
constexpr int kCostOverhead = 6;    // fixed cost of an item, in key tiles
constexpr int kMinChunk = 8;        // fewest key tiles of a chunk of a split item
constexpr int kPlanLdsItems = 4096; // plans of up to this many items stay in LDS
constexpr int kSortBuckets = 16;     // key-tile counts the queue order tells apart
// Unit flag (bit 31 of the chunk word): the unit's query tiles start at the
// history end n_h instead of row 0 (candidates-only plans).
constexpr int kUnitCandRows = int(0x80000000u);
// Plan modes (header word 2): the static plan, one work queue, or one work
// queue per XCD.
constexpr int kPlanStatic = 0, kPlanQueue = 1, kPlanXcdQueues = 2;
constexpr int kHdrXcdCtr = 8;     // header words 8 .. 15: the XCD queues' counters
constexpr int kHdrXcdBound = 16;  // words 16 .. 24: XCD x's units are [w[16 + x], w[17 + x])

// The queue a workgroup of the attention launch takes units from (queue
// modes).  Units [first, end) are shared by n workgroups; the workgroup with
// index w among them starts with unit first + w, and each fetch from counter
// word `ctr` returns how many units its queue has handed out after the first
// n, so its next unit is first + n + that value.  Per-XCD queues serve the
// workgroups g with g % 8 == x (the XCD g runs on).
struct WorkQueue {
  int first, end, n, w, ctr;
};
__device__ inline WorkQueue work_queue(const int32_t* hdr) {
  WorkQueue q;
  if (hdr[2] == kPlanXcdQueues) {
    const int x = (int)blockIdx.x % kXcds;
    q.first = hdr[kHdrXcdBound + x];
    q.end = hdr[kHdrXcdBound + x + 1];
    q.n = ((int)gridDim.x - x + kXcds - 1) / kXcds;
    q.w = (int)blockIdx.x / kXcds;
    q.ctr = kHdrXcdCtr + x;
  } else {
    q.first = 0;
    q.end = hdr[4];
    q.n = (int)gridDim.x;
    q.w = (int)blockIdx.x;
    q.ctr = 3;
  }
  return q;
}

struct PlanLayout {
  size_t hdr_off;      // int32[64]: [0] workgroups the plan was made for,
                       //   [1] 1 for a candidates-only plan, [2] the plan
                       //   mode (kPlan*), [3] the single queue's counter,
                       //   [4] the number of units, [8 .. 24] the XCD
                       //   queues' counters and unit ranges
  size_t units_off;    // int4[2 * units_max]: (seq start, L, n_h, qt*H + h),
                       //   (kt_begin, kt_end, split slot or -1, chunk << 16 | chunks)
  size_t wg_off;       // int32[2 * kMaxGrid]: (first unit, units) per workgroup
  size_t ctr_off;      // int32[slots_max]: arrival counter of each split item
  size_t part_off;     // float[slots_max * slot_floats]: partial outputs of chunks
  size_t seq_off;      // int32[4 * (B + 1)]: per-sequence scratch of large batches
  size_t item_off;     // per-item scratch of large plans: int32 cost[items_max + 1],
                       //   int32 seq[items_max + 1], int64 line[items_max + 1],
                       //   int64 ubase[items_max + 1]
  size_t total;
  int64_t items_max;   // bound on sum_b ceil(L_b / BM) * H
  int64_t units_max;   // items_max + kMaxGrid
  int64_t slots_max;   // 2 * kMaxGrid: chunks of split items
  int64_t slot_floats; // kBM rows x d_v rounded up to 32
};

__host__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The scheduler's compact variant (32-bit cost sums, per-item arrays in LDS)
// serves plans of at most kPlanLdsItems items over fewer than 2^21 tokens:
// then every item costs below 2^16 and every cost sum stays below 2^28.
__host__ inline bool plan_is_compact(int64_t items_max, int64_t total_tokens) {
  return items_max <= kPlanLdsItems && total_tokens < (int64_t(1) << 21);
}

// The scheduler splits only items of at least 2 kMinChunk key tiles, which
// needs a sequence of at least this many tokens: a batch with fewer tokens in
// all never uses the partial-output slots.
constexpr int64_t kMinSplitTokens = (2 * kMinChunk - 1) * kBN + 1;

// Work-list layout.  `splits`: the plan may split items along their keys
// (then it holds 2 kMaxGrid partial-output slots); without, it keeps every
// item whole and holds none.
__host__ inline PlanLayout plan_layout(int64_t num_seqs, int64_t total_tokens, int64_t heads,
                                       int64_t d_v, bool splits) {
  PlanLayout p;
  // sum_b ceil(L_b / BM) <= (N + B*(BM-1)) / BM
  p.items_max = (total_tokens + num_seqs * (kBM - 1)) / kBM * heads;
  p.units_max = p.items_max + kMaxGrid;
  p.slots_max = splits ? 2 * kMaxGrid : 0;
  p.slot_floats = (int64_t)kBM * 32 * ((d_v + 31) / 32);
  const size_t im = (size_t)(p.items_max > 0 ? p.items_max : 1);
  const bool big_b = num_seqs > kPlanLdsSeqs, big_i = !plan_is_compact(p.items_max, total_tokens);
  p.hdr_off = 0;
  p.units_off = 256;
  p.wg_off = align256(p.units_off + 2 * sizeof(int4) * (size_t)p.units_max);
  p.ctr_off = align256(p.wg_off + sizeof(int32_t) * 2 * kMaxGrid);
  p.part_off = align256(p.ctr_off + sizeof(int32_t) * (size_t)p.slots_max);
  p.seq_off = align256(p.part_off + sizeof(float) * (size_t)(p.slots_max * p.slot_floats));
  p.item_off = align256(p.seq_off + (big_b ? sizeof(int32_t) * 4 * (size_t)(num_seqs + 1) : 0));
  p.total = align256(p.item_off +
                     (big_i ? (2 * sizeof(int32_t) + 2 * sizeof(int64_t)) * (im + 1) + 16 : 0));
  return p;
}

struct PlanArgs {
  const int32_t* offsets;
  const int32_t* num_targets;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t contextual_len;
  int32_t max_attn_len;
  int32_t items_max;     // capacity of the item scratch
  int32_t n_wg;          // workgroups of the attention launch (<= kMaxGrid)
  int32_t cand_only;     // 1: only the candidate rows [n_h, L), tiled from n_h
  int32_t no_split;      // 1: keep every item whole (no partial-output slots)
  int32_t transposed;    // 1: items are key tiles walking the query rows they reach
  int32_t* hdr;
  int4* units;
  int32_t* wg;
  int32_t* counters;
  int32_t* seq_scratch;  // used when B > kPlanLdsSeqs
  char* item_scratch;    // used when the items exceed kPlanLdsItems
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* u;
  void* out;
  const int32_t* offsets;
  const int64_t* timestamps;
  const int32_t* num_targets;
  const float* pos_table;
  const float* time_table;
  const int32_t* hdr;        // [0]: workgroups the plan was made for
  const int4* units;
  const int32_t* wg;         // (first unit, units) per planned workgroup
  int32_t* counters;         // arrival counters of split items
  float* partials;           // fp32 partial outputs of split chunks
  int64_t slot_floats;
  int64_t ld_q, ld_k, ld_v, ld_u, ld_out;
  int32_t num_heads;
  int32_t contextual_len;
  int32_t max_attn_len;
  int32_t pos_len;
  int32_t time_len;
  int32_t epilogue;   // 0 = LayerNorm * U, 1 = none
  int32_t pos_clamp;  // position bias of |p_i - p_j|, p = min(position, n_h)
  void* out_raw;      // optional: o / n_scale before the gate, [N, H, d_v]
  int64_t ld_raw;
  float alpha;
  float out_scale;    // ln(2) / n_scale: SiLU values are formed in log2 units
  float ln_eps;
};

// Epilogue variant: LayerNorm over all heads of a token, in place on `out`.
struct LnArgs {
  void* out;
  const void* u;
  int64_t ld_out, ld_u;
  const int32_t* offsets;
  const int32_t* num_targets;
  const int32_t* hdr;    // plan header: [1] != 0 for a candidates-only plan
  int32_t num_seqs;
  int32_t n_tok;
  int32_t width;         // H * d_v
  float eps;
};

// Allowed query rows of key j -- the same rules read by column: a candidate
// key (j >= n_h) is seen by its own row only; any other key by the rows
// [j < c ? 0 : j, hi_j], where hi_j = L - 1 when the key is within the window
// of the history end (W == 0 or j + W >= n_h: the candidates see it, and so
// does every later history row), else j + W.  Same encoding as RowBounds:
// (unsigned)(i - lo) <= span, or i == self_j.
__host__ __device__ inline RowBounds col_bounds(const SeqGeom& g, int j) {
  RowBounds r;
  if (j >= g.n_h) {
    r.lo = kEmptyLo;
    r.span = 0;
    r.self_j = j;
    return r;
  }
  const int lo = j < g.c ? 0 : j;
  const int hi = (g.W == 0 || j + g.W >= g.n_h) ? g.L - 1 : j + g.W;
  r.lo = lo;
  r.span = hi - lo;
  r.self_j = -1;
  return r;
}

// Query rows [ilo, ihi] that keys [j0, j1) (j0 < j1 <= L) can reach: the
// union of their col_bounds.  A history key's interval starts at 0 (prefix
// keys) or at the key and ends at j + W or L - 1, nondecreasing in j; a
// candidate key reaches only its own row.
__host__ __device__ inline void tile_row_range(const SeqGeom& g, int j0, int j1, int& ilo,
                                               int& ihi) {
  if (j0 < g.n_h) {
    ilo = j0 < g.c ? 0 : j0;
    const int jl = (j1 < g.n_h ? j1 : g.n_h) - 1;
    ihi = (g.W == 0 || jl + g.W >= g.n_h) ? g.L - 1 : jl + g.W;
    if (j1 - 1 > ihi) ihi = j1 - 1;   // candidate keys of the tile: their own rows
  } else {
    ilo = j0;
    ihi = j1 - 1;
  }
}

// The range a tile of 128 rows reaches: keys for the forward, or with
// `transposed` (a tile of keys) the query rows, as the key-side passes of
// the backward walk them.
__host__ __device__ inline void tile_range(const SeqGeom& g, int i0, int i1, bool transposed,
                                           int& lo, int& hi) {
  if (transposed) tile_row_range(g, i0, i1, lo, hi);
  else tile_key_range(g, i0, i1, lo, hi);
}

// Backward.  Work is listed as (sequence, 128-token tile) groups, sorted by
// decreasing cost twice: once for the dQ pass (query tiles, cost = key
// steps) and once for the dK/dV pass (key tiles, cost = query steps); item
// v of a pass is group list[v / H], head v % H.
constexpr int kBwdCostBins = 1024;

__host__ inline int64_t bwd_groups_max(int64_t num_seqs, int64_t total_tokens) {
  return (total_tokens + num_seqs * (kBM - 1)) / kBM;
}

struct BwdPlanArgs {
  const int32_t* offsets;
  const int32_t* num_targets;
  int32_t num_seqs;
  int32_t contextual_len;
  int32_t max_attn_len;
  int32_t* hdr;       // [0]: groups
  int32_t* gstart;    // int32[B + 1]: first group of each sequence
  int2* list_q;       // groups by decreasing dQ cost: (sequence, tile)
  int2* list_kv;      // groups by decreasing dK/dV cost
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;          // dLoss / dO (the gate's input gradient)
  void* dq;
  void* dk;
  void* dv;
  const int32_t* offsets;
  const int64_t* timestamps;
  const int32_t* num_targets;
  const float* pos_table;
  const float* time_table;
  double* tab64;             // fp32 kernels: [pos_len + time_len] fp64 table sums
  float* tab_part;           // MFMA kernels: per-workgroup table sums
  const int32_t* hdr;
  const int2* list;
  int64_t ld_q, ld_k, ld_v, ld_do;
  int32_t num_heads;
  int32_t contextual_len;
  int32_t max_attn_len;
  int32_t pos_len;
  int32_t time_len;
  int32_t n_tok;
  float alpha;
  float inv_scale;           // 1 / n_scale
  int32_t pos_clamp;         // position bias of the clamped positions min(p, n_h)
};

struct GateBwdArgs {
  const void* o;             // raw aggregated output (epilogue NONE), ld = ld_o
  const void* u;
  const void* dy;            // dLoss / d(out)
  void* du;
  void* d_o;                 // dLoss / dO, ld = ld_o
  int64_t ld_o, ld_u, ld_dy;
  int32_t n_tok;
  int32_t groups;            // LayerNorm groups per token
  int32_t width;             // values per group
  float eps;
};

struct TabReduceArgs {
  const float* part;         // [n_part][stride]
  float* part2;              // [ceil(n_part / 64)][stride]: row-block sums
  float* dpos;
  float* dtime;
  int32_t n_part;
  int32_t stride;            // pos_len + 64
  int32_t pos_len;
  int32_t time_len;
  float scale;
};

// Launchers (defined in the .hip files).
hipError_t launch_plan(const PlanArgs& a, bool compact, hipStream_t stream);
// start / stop: when not null, events that take the kernel's own start and
// end times (hipExtLaunchKernelGGL).
hipError_t launch_attn(const AttnArgs& a, int dtype, int d_qk, int d_v, int n_wg,
                       hipStream_t stream, hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// Workgroups of the persistent attention launch for this shape on the current
// device (CUs x resident workgroups per CU), or a negative value on error.
int attn_grid(int dtype, int d_qk, int d_v, int pos_len, int time_len, bool clamp);
bool attn_supported(int dtype, int d_qk, int d_v);
// The eight-wave forward for long sequences (attn_fwd_pp.hip): bf16, d_qk =
// d_v = 128; same units, workspace and arguments as launch_attn.
bool attn_pp_supported(int dtype, int d_qk, int d_v);
int attn_pp_grid(int pos_len, int time_len, bool clamp);
hipError_t launch_attn_pp(const AttnArgs& a, int n_wg, hipStream_t stream,
                          hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// The sixteen-row forward (attn_fwd_w16.hip): bf16, d_qk = d_v = 128; eight
// waves of 16 query rows per workgroup, four waves per SIMD; same units,
// workspace and arguments as launch_attn.
// `transposed`: the key-side walk of the backward's value gradient (plan
// made with PlanArgs::transposed; epilogue none; no clamped position bias).
bool attn_w16_supported(int dtype, int d_qk, int d_v);
int attn_w16_grid(int pos_len, int time_len, bool clamp, bool transposed = false);
hipError_t launch_attn_w16(const AttnArgs& a, int n_wg, hipStream_t stream,
                           hipEvent_t start = nullptr, hipEvent_t stop = nullptr,
                           bool transposed = false);
// The thirty-two-row forward (attn_fwd_w32.hip): bf16, d_qk = d_v = 128; four
// waves of two 16-row groups per workgroup, two waves per SIMD; same units,
// workspace and arguments as launch_attn.
bool attn_w32_supported(int dtype, int d_qk, int d_v);
int attn_w32_grid(int pos_len, int time_len, bool clamp);
hipError_t launch_attn_w32(const AttnArgs& a, int n_wg, hipStream_t stream,
                           hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// Batches whose mean sequence length reaches this many tokens take the
// eight-wave kernel (short sequences give it too few key blocks per item to
// fill its pipeline; the four-wave kernel runs two workgroups per CU).
constexpr int kPPMinMeanLen = 512;
// Whether the automatic choice may take the eight-wave kernel at all: off
// while it measures slower than the four-wave kernel on the long batches.
constexpr bool kPPAuto = false;
// Whether the automatic choice takes the sixteen-row kernel where it is built
// (it measures faster than the four-wave kernel on long and short batches).
constexpr bool kW16Auto = true;
int ln_all_heads_max_width(int dtype);
hipError_t launch_ln_all_heads(const LnArgs& a, int dtype, hipStream_t stream);
bool bwd_supported(int dtype, int d_qk, int d_v);
// Shapes whose backward runs the per-token kernels (fp64 table sums) rather
// than the matrix-core passes.
bool bwd_per_token(int dtype, int d_qk, int d_v);
hipError_t launch_bwd_plan(const BwdPlanArgs& a, hipStream_t stream);
hipError_t launch_gate_bwd(const GateBwdArgs& a, int dtype, hipStream_t stream);
// Backward passes: which = 0 (dQ), 1 (dK with the table sums; also dV for
// d = 64), 2 (dV alone, d = 128 only; a no-op otherwise).  bwd_grid gives the
// persistent launch size (CUs x resident workgroups per CU), 0 for a pass
// that does not exist, or a negative value on error; for fp32 n_wg of
// launch_bwd is the number of sequences instead.
int bwd_grid(int dtype, int d_qk, int d_v, int pos_len, int time_len, int which,
             bool clamp = false);
hipError_t launch_bwd(const BwdArgs& a, int dtype, int d_qk, int d_v, int which, int n_wg,
                      hipStream_t stream);
hipError_t launch_tab_reduce(const TabReduceArgs& a, hipStream_t stream);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream);
// dpos[e] = tab64[e], dtime[e] = tab64[pos_len + e], rounded to float.
hipError_t launch_tab64_finish(const double* tab64, float* dpos, float* dtime, int pos_len,
                               int time_len, hipStream_t stream);

}  // namespace hstu
