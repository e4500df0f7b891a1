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
constexpr int kBN = 64;         // keys per staged K/V tile (two 32-key MFMA blocks)
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kPosMax = 8192;   // longest supported position table
constexpr int kPlanThreads = 1024;
constexpr int kPlanLdsSeqs = 8192;  // batches up to this many sequences plan from LDS
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
struct PlanLayout {
  size_t count_off;      // int32: number of (sequence, query-tile) pairs
  size_t pairs_off;      // int2[pairs_max]: sorted (b, qt)
  size_t keys_off;       // int32[pairs_max]: bucketed work estimate per pair
  size_t seqstart_off;   // int32[B+1]: first pair of each sequence
  size_t total;
  int64_t pairs_max;
};

__host__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ inline PlanLayout plan_layout(int64_t num_seqs, int64_t total_tokens) {
  PlanLayout p;
  // sum_b ceil(L_b / BM) <= (N + B*(BM-1)) / BM
  p.pairs_max = (total_tokens + num_seqs * (kBM - 1)) / kBM;
  p.count_off = 0;
  p.pairs_off = 256;
  p.keys_off = align256(p.pairs_off + sizeof(int2) * (size_t)(p.pairs_max > 0 ? p.pairs_max : 1));
  p.seqstart_off = align256(p.keys_off + sizeof(int32_t) * (size_t)(p.pairs_max > 0 ? p.pairs_max : 1));
  p.total = align256(p.seqstart_off + sizeof(int32_t) * (size_t)(num_seqs + 1));
  return p;
}

struct PlanArgs {
  const int32_t* offsets;
  const int32_t* num_targets;
  int32_t num_seqs;
  int32_t contextual_len;
  int32_t max_attn_len;
  int32_t pairs_max;     // capacity of pairs/keys (bound from num_seqs, total_tokens)
  int32_t* count;
  int2* pairs;
  int32_t* keys;
  int32_t* seq_start;
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
  const int32_t* count;
  const int2* pairs;
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
hipError_t launch_attn(const AttnArgs& a, int dtype, int d_qk, int d_v, int64_t grid,
                       hipStream_t stream);
bool attn_supported(int dtype, int d_qk, int d_v);

}  // namespace hstu
