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
constexpr int kPlanLdsSeqs = 4096;  // batches up to this many sequences plan from LDS
constexpr int kKeyBuckets = 64; // work-estimate buckets of the scheduler
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

// Work-list layout inside the caller's workspace (byte offsets, 256-aligned).
// The scheduler fills one queue of items per XCD (the MI355X has 8 XCDs, each
// with its own L2); items are (sequence, head, query tile).
constexpr int kQueues = 8;

struct PlanLayout {
  size_t hdr_off;      // int32 queue_count[8], queue_start[8]
  size_t items_off;    // int4[items_max]: (seq start, L, n_h, qt*H + h), queue by queue
  size_t gscan_off;    // int32[8*S + 1]: item offsets of the (queue, slot) groups
  size_t seq_off;      // int32[6*B]: per-sequence scratch of the scheduler (large batches)
  size_t total;
  int64_t pairs_max;   // bound on sum_b ceil(L_b / BM)
  int64_t items_max;   // pairs_max * H
  int64_t slots;       // S = ceil(B*H / 8)
};

__host__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ inline PlanLayout plan_layout(int64_t num_seqs, int64_t total_tokens, int64_t heads) {
  PlanLayout p;
  // sum_b ceil(L_b / BM) <= (N + B*(BM-1)) / BM
  p.pairs_max = (total_tokens + num_seqs * (kBM - 1)) / kBM;
  p.items_max = p.pairs_max * heads;
  p.slots = (num_seqs * heads + kQueues - 1) / kQueues;
  p.hdr_off = 0;
  p.items_off = 256;
  p.gscan_off = align256(p.items_off + sizeof(int4) * (size_t)(p.items_max > 0 ? p.items_max : 1));
  p.seq_off = align256(p.gscan_off + sizeof(int32_t) * (size_t)(kQueues * p.slots + 1));
  p.total = align256(p.seq_off + sizeof(int32_t) * (size_t)(6 * num_seqs + 6));
  return p;
}

struct PlanArgs {
  const int32_t* offsets;
  const int32_t* num_targets;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t contextual_len;
  int32_t max_attn_len;
  int32_t items_max;     // capacity of `items`
  int32_t slots;         // S
  int32_t* queue_count;  // [8]
  int32_t* queue_start;  // [8]
  int4* items;
  int32_t* gscan;
  int32_t* seq_scratch;  // [6*B], used when B > kPlanLdsSeqs
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
  const int32_t* queue_count;
  const int32_t* queue_start;
  const int4* items;
  int64_t ld_q, ld_k, ld_v, ld_u, ld_out;
  int32_t num_heads;
  int32_t contextual_len;
  int32_t max_attn_len;
  int32_t pos_len;
  int32_t time_len;
  int32_t epilogue;   // 0 = LayerNorm * U, 1 = none
  float alpha;
  float out_scale;    // ln(2) / n_scale: SiLU values are formed in log2 units
  float ln_eps;
};

// Launchers (defined in the .hip files).
hipError_t launch_plan(const PlanArgs& a, hipStream_t stream);
hipError_t launch_attn(const AttnArgs& a, int dtype, int d_qk, int d_v, int n_wg,
                       hipStream_t stream);
// Workgroups of the persistent attention launch for this shape on the current
// device (CUs x resident workgroups per CU), or a negative value on error.
int attn_grid(int dtype, int d_qk, int d_v, int pos_len, int time_len);
bool attn_supported(int dtype, int d_qk, int d_v);

}  // namespace hstu
