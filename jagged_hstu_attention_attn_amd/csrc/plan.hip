// plan.hip -- device-side scheduler for the jagged HSTU attention kernel.
//
// Ragged execution must handle "boundaries, grouping and balance" ("Scaling
// HSTU: ragged execution, candidate amortization and content features",
// section "Variable length is a central systems issue").  Padding is never
// materialised: the scheduler reads the offsets, lists only the query tiles
// that exist and balances them over the persistent attention launch:
//
//   1. items are the (sequence, head, 128-row query tile) triples, sequence
//      by sequence, the tiles of one (sequence, head) together with the last
//      (most expensive) tile first; an item costs the key tiles its mask lets
//      it reach (tile_key_range) plus a fixed term.  A candidates-only plan
//      tiles just the candidate rows [n_h, L) of each sequence, from n_h;
//   2. items are dealt round-robin to n_wg columns (item t * n_wg + c goes to
//      column c in round t) and the columns are laid end to end on one line
//      (the dealt order), which is cut into n_wg shares of equal cost;
//   3. share r runs on workgroup x + 8w with x = r / (n_wg / 8): consecutive
//      shares share an XCD (the MI355X dispatches workgroup g to XCD g % 8
//      and each XCD has its own L2).  With items of equal cost the shares are
//      the columns, so in every round the 64 workgroups of an XCD process 64
//      neighbouring query tiles, whose key/value rows that L2 serves once;
//   4. an item that a share boundary cuts is split there along its key tiles
//      (proportionally, never into chunks under kMinChunk tiles): the
//      pointwise aggregation is a sum over keys, so the chunks' partial
//      outputs add up exactly to the item's output.
//
// Batches whose sequences all fit two query tiles (rows computed) and whose
// items all stay under 2 x kMinChunk key tiles (so none would be split; a
// candidate tile behind a long history reaches more) are planned as a work
// queue instead: the units in decreasing cost
// (a counting sort on their key-tile count), taken by the attention
// workgroups one at a time from a counter, which balances them like
// longest-first list scheduling.
//
// Batches whose items are all small against a workgroup's share (the
// largest costs at most a quarter of it: many windowed tiles, say) are
// planned as one work queue per XCD instead: XCD x takes a contiguous,
// cost-balanced range of the items in list order, so the workgroups of one
// L2 always work on neighbouring tiles, and the range's last items go in
// decreasing cost.
//
// One workgroup of 1024 threads, five phases; the per-item arrays stay in LDS
// up to kPlanLdsItems items.  Everything stays on the device, so the
// caller's stream never synchronises with the host.
#include <type_traits>

#include "attn_common.hpp"
#include "hstu_device.hpp"

namespace hstu {

// Inclusive prefix sum over the 64 lanes of a wave.  32-bit values use
// data-parallel-primitive moves: row shifts by 1, 2, 4, 8 (lanes without a
// source read 0) scan each 16-lane row, then row broadcasts carry lane 15 of
// row 0 into row 1, of row 2 into row 3, and lane 31 into rows 2 and 3.
__device__ inline int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}
__device__ inline int64_t wave_incl_scan(int64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive scan over the kPlanThreads threads of the block; `ws` holds 16
// values; `total` receives the sum over the block.
template <typename V>
__device__ inline V block_excl_scan(V x, V* ws, V& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const V inc = wave_incl_scan(x);
  if (lane == 63) ws[wave] = inc;
  __syncthreads();
  V pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kPlanThreads / 64; ++w) {
    const V s = ws[w];
    if (w < wave) pre += s;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return pre + inc - x;
}

// Chunks of an item spanning cost units [P, P + cost) of a line cut into
// shares of T units.  An item under 2 * kMinChunk tiles (or any item when
// splitting is off) stays whole and goes to the share holding its midpoint.  Otherwise each multiple rT strictly
// inside the span is a candidate cut at tile offset
// t = floor((rT - P) * tiles / cost).  A cut that would
// close a chunk of fewer than kMinChunk tiles instead hands the open chunk to
// share r; a cut that would leave fewer than kMinChunk tiles after it is
// dropped.  f(j, tb, te, r): chunk j covers tile offsets [tb, te) and belongs
// to share r.  Owners never decrease along the line.  Returns the number of
// chunks.
template <typename I, typename F>
__device__ inline int item_chunks(I P, int cost, int tiles, I T, bool may_split, F&& f) {
  using U = typename std::make_unsigned<I>::type;   // products stay below 2^(bits of I)
  if (!may_split || tiles < 2 * kMinChunk) {   // whole: the share holding its midpoint takes it
    f(0, 0, tiles, (int)((P + cost / 2) / T));
    return 1;
  }
  const I r0 = P / T, r1 = (P + cost - 1) / T;
  int j = 0, tb = 0;
  I owner = r0;
  for (I r = r0 + 1; r <= r1; ++r) {
    const int t = (int)((U)(r * T - P) * (U)tiles / (U)cost);
    if (t - tb < kMinChunk) {
      owner = r;   // the open chunk moves to the later share, which holds most of it
    } else if (tiles - t >= kMinChunk) {
      f(j, tb, t, (int)owner);
      ++j;
      tb = t;
      owner = r;
    }
  }
  f(j, tb, tiles, (int)owner);
  return j + 1;
}

// Workgroups of XCD x: g < n_wg with g % 8 == x.
__device__ inline int xcd_wgs(int n_wg, int x) { return (n_wg - x + kXcds - 1) / kXcds; }

// Shares in XCD-major order -> workgroup: share r of XCD x is workgroup x + 8r.
__device__ inline int share_wg(int f, int n_wg) {
  int x = 0, base = 0;
  for (; x < kXcds - 1; ++x) {
    const int wx = xcd_wgs(n_wg, x);
    if (f < base + wx) break;
    base += wx;
  }
  return x + kXcds * (f - base);
}

struct ItemGeo {
  int b, h, qt, kt_lo, kt_hi, n_h;
};

// First query row of a sequence's tiles: 0, or the history end when only the
// candidate rows are computed.
__device__ inline int row_base(int n_h, bool cand_only) { return cand_only ? n_h : 0; }

// Item k of sequence b (head-major, last query tile first).
__device__ inline ItemGeo item_geo_of(int k, int b, const int32_t* base, const int32_t* slen,
                                      const int32_t* hist, int contextual_len,
                                      int max_attn_len, bool cand_only, bool tr) {
  ItemGeo r;
  r.b = b;
  const int L = slen[b], i_b = row_base(hist[b], cand_only);
  const int nq = (L - i_b + kBM - 1) / kBM;
  const int t = k - base[b];
  r.h = t / nq;
  r.qt = nq - 1 - (t - r.h * nq);
  SeqGeom g;
  g.L = L;
  g.n_h = hist[b];
  g.c = clampi(contextual_len, 0, g.n_h);
  g.W = max_attn_len;
  const int i0 = i_b + r.qt * kBM, i1 = min(i0 + kBM, L);
  int jlo, jhi;
  tile_range(g, i0, i1, tr, jlo, jhi);
  r.kt_lo = jlo / kBN;
  r.kt_hi = jhi / kBN;
  r.n_h = g.n_h;
  return r;
}

// Sequence of item k: the last b with base[b] <= k.
__device__ inline int seq_of(int k, const int32_t* base, int B) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (base[mid] <= k) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Dealt order: item i = t * n_wg + c (round t, column c) sits at position
// start(c) + t of the line, columns one after another, where column c holds
// `full` + (c < extra) items.  Returns the item at line position j.
__device__ inline int dealt_item(int j, int n, int n_wg) {
  const int full = n / n_wg, extra = n - full * n_wg;
  const int big = extra * (full + 1);   // positions held by the longer columns
  int c, t;
  if (j < big) {
    c = j / (full + 1);
    t = j - c * (full + 1);
  } else {
    c = extra + (j - big) / full;
    t = j - big - (c - extra) * full;
  }
  return t * n_wg + c;
}

// Inverse of dealt_item: the line position of item k.
__device__ inline int dealt_pos(int k, int n, int n_wg) {
  const int full = n / n_wg, extra = n - full * n_wg;
  const int t = k / n_wg, c = k - t * n_wg;
  return (c < extra ? c * (full + 1) : extra * (full + 1) + (c - extra) * full) + t;
}

// Sequence geometry of sequence b for the mask rules.
__device__ inline SeqGeom seq_geom(int b, const int32_t* slen, const int32_t* hist,
                                   const PlanArgs& a) {
  SeqGeom g;
  g.L = slen[b];
  g.n_h = hist[b];
  g.c = clampi(a.contextual_len, 0, g.n_h);
  g.W = a.max_attn_len;
  return g;
}

// Key tiles [kt_lo, kt_hi] that query tile qt (first row i_b + qt * kBM) can
// reach, as item_geo_of counts them, and its queue-order bucket (0 = the most
// key tiles).  The count and the scatter of the queue order both use it, so
// they agree on every bucket.
__device__ inline int tile_bucket(const SeqGeom& g, int i_b, int qt, bool tr, int& kt_lo,
                                  int& kt_hi) {
  const int i0 = i_b + qt * kBM, i1 = min(i0 + kBM, g.L);
  int jlo, jhi;
  tile_range(g, i0, i1, tr, jlo, jhi);
  kt_lo = jlo / kBN;
  kt_hi = jhi / kBN;
  return kSortBuckets - min(kt_hi - kt_lo + 1, kSortBuckets);
}

// I: type of the cost prefix sums (int when they fit, else int64_t).  LDS:
// the per-item arrays live in LDS (at most kPlanLdsItems items) instead of
// the workspace.
template <typename I, bool LDS>
__global__ __launch_bounds__(kPlanThreads) void hstu_plan_kernel(PlanArgs a) {
  constexpr int kItems = LDS ? kPlanLdsItems : 1;
  constexpr int kShift = 4 * (int)sizeof(I);   // units | split chunks << kShift
  constexpr I kLow = (I(1) << kShift) - 1;
  __shared__ I s_ws[kPlanThreads / 64];
  __shared__ int s_ws32[kPlanThreads / 64];
  __shared__ int s_cnt[kMaxGrid];
  __shared__ int s_seq[4 * (kPlanLdsSeqs + 1)];
  __shared__ int s_cost[kItems + 1];
  __shared__ int s_iseq[kItems];
  __shared__ I s_line[kItems + 1];
  __shared__ I s_ub[kItems + 1];
  __shared__ int2 s_geo[kItems];   // LDS plans: first key tile, qt * H + h of each item
  __shared__ int s_bcnt[kSortBuckets];
  __shared__ int s_long;   // some item needs the static plan
  __shared__ int s_maxc;   // the largest item cost
  __shared__ int s_xb[kXcds + 1];   // per-XCD queues: first item of each XCD's range

  const int tid = threadIdx.x;
  const int B = a.num_seqs, H = a.num_heads, n_wg = a.n_wg;
  const bool cand = a.cand_only != 0;
  const bool tr = a.transposed != 0;
  int32_t* seq = B <= kPlanLdsSeqs ? s_seq : a.seq_scratch;
  const int LD = B <= kPlanLdsSeqs ? kPlanLdsSeqs + 1 : B + 1;
  int32_t* base = seq;            // [B + 1] first item of each sequence
  int32_t* start = seq + LD;      // [B] first token
  int32_t* slen = seq + 2 * LD;   // [B] tokens
  int32_t* hist = seq + 3 * LD;   // [B] history tokens (L minus clamped candidates)

  for (int v = tid; v < kMaxGrid; v += kPlanThreads) s_cnt[v] = 0;
  if (tid == 0) s_long = 0;
  if (tid == 0) s_maxc = 0;
  if (tid < kSortBuckets) s_bcnt[tid] = 0;
  __syncthreads();

  // 1. Per sequence: geometry and the first item (exclusive scan of nq * H).
  int carry = 0;
  for (int b0 = 0; b0 < B; b0 += kPlanThreads) {
    const int b = b0 + tid;
    int cnt = 0;
    if (b < B) {
      const int s0 = a.offsets[b];
      const int L = max(0, a.offsets[b + 1] - s0);
      const int nt = a.num_targets ? a.num_targets[b] : 0;
      start[b] = s0;
      slen[b] = L;
      hist[b] = L - clampi(nt, 0, L);
      cnt = (L - row_base(hist[b], cand) + kBM - 1) / kBM * H;
      if (L - row_base(hist[b], cand) > 2 * kBM) {
        s_long = 1;
      } else if (LDS) {
        const SeqGeom g = seq_geom(b, slen, hist, a);
        const int i_b = row_base(g.n_h, cand);
        int kt_lo, kt_hi;
        for (int qt = 0; i_b + qt * kBM < L; ++qt) {
          atomicAdd(&s_bcnt[tile_bucket(g, i_b, qt, tr, kt_lo, kt_hi)], H);
          if (kt_hi - kt_lo + 1 >= 2 * kMinChunk) s_long = 1;   // the static plan would split it
        }
      }
    }
    int tot;
    const int ex = block_excl_scan(cnt, s_ws32, tot);
    if (b < B) base[b] = carry + ex;
    carry += tot;
  }
  const int n = min(carry, a.items_max);   // never beyond the scratch's capacity

  // Work queue: the units, one per item (none is split), in decreasing cost
  // straight from the counting sort; the attention kernel reads nothing else
  // of the plan in this mode.
  if (LDS && s_long == 0 && n == carry) {
    if (tid < 64) {   // bucket starts: exclusive scan over the buckets
      const int c = tid < kSortBuckets ? s_bcnt[tid] : 0;
      const int inc = wave_incl_scan(c);
      if (tid < kSortBuckets) s_bcnt[tid] = inc - c;
    }
    __syncthreads();
    for (int b = tid; b < B; b += kPlanThreads) {   // ties in any order
      const SeqGeom g = seq_geom(b, slen, hist, a);
      const int i_b = row_base(g.n_h, cand);
      for (int qt = 0; i_b + qt * kBM < g.L; ++qt) {
        int kt_lo, kt_hi;
        const int pos = atomicAdd(&s_bcnt[tile_bucket(g, i_b, qt, tr, kt_lo, kt_hi)], H);
        const int4 ch = make_int4(kt_lo, kt_hi, -1, (cand ? kUnitCandRows : 0) | 1);
        for (int h = 0; h < H; ++h) {
          a.units[2 * (pos + h)] = make_int4(start[b], g.L, g.n_h, qt * H + h);
          a.units[2 * (pos + h) + 1] = ch;
        }
      }
    }
    if (tid == 0) {
      a.hdr[0] = n_wg;
      a.hdr[1] = cand ? 1 : 0;
      a.hdr[2] = kPlanQueue;
      a.hdr[3] = 0;
      a.hdr[4] = n;
    }
    return;
  }

  int* cost = s_cost;
  int* iseq = s_iseq;
  I* line = s_line;
  I* ub = s_ub;
  if constexpr (!LDS) {
    const size_t im = (size_t)a.items_max + 1;
    cost = reinterpret_cast<int*>(a.item_scratch);
    iseq = cost + im;
    line = reinterpret_cast<I*>(a.item_scratch + ((2 * sizeof(int) * im + 15) & ~size_t(15)));
    ub = line + im;
  }
  __syncthreads();

  // 2. Costs in dealt order and their prefix sums (the line).
  I ccarry = 0;
  for (int j0 = 0; j0 < n; j0 += kPlanThreads) {
    const int j = j0 + tid;
    int c = 0;
    if (j < n) {
      const int k = dealt_item(j, n, n_wg);
      const int b = seq_of(k, base, B);
      const ItemGeo g = item_geo_of(k, b, base, slen, hist, a.contextual_len, a.max_attn_len, cand, tr);
      c = g.kt_hi - g.kt_lo + 1 + kCostOverhead;
      cost[j] = c;
      iseq[j] = b;
      if constexpr (LDS) s_geo[j] = make_int2(g.kt_lo, g.qt * H + g.h);
    }
    const int wmax = wave_max(c);   // one LDS atomic per wave
    if ((tid & 63) == 0) atomicMax(&s_maxc, wmax);
    I tot;
    const I ex = block_excl_scan((I)c, s_ws, tot);
    if (j < n) line[j] = ccarry + ex;
    ccarry += tot;
  }
  const I C = ccarry;
  const I T = C > 0 ? (C + n_wg - 1) / n_wg : 1;   // cost of one share
  __syncthreads();

  // Per-XCD work queues, when the largest item costs at most a quarter of a
  // share: XCD x takes a contiguous range of the items in list order, cut
  // where the items' cost midpoints pass x / 8 of the total, and its
  // workgroups take the range's units in that order from one counter.  The
  // workgroups of one L2 then work on neighbouring query tiles of one
  // (sequence, head) at any time, whatever the item costs (the dealt
  // shares drift apart in time when the costs differ, which loses that
  // reuse).  The range's last items, one per workgroup of the XCD, go in
  // decreasing cost, which evens out the end like longest-first list
  // scheduling.  Nothing is split.
  if constexpr (LDS) {
    if (n == carry && (I)s_maxc * 4 <= T) {
      // list-order costs (into `line`) and their exclusive prefix sums (into
      // `ub`), read from the dealt-order arrays at dealt_pos(k)
      if (tid <= kXcds) s_xb[tid] = tid == 0 ? 0 : n;
      I lcarry = 0;
      for (int k0 = 0; k0 < n; k0 += kPlanThreads) {
        const int k = k0 + tid;
        const int c = k < n ? cost[dealt_pos(k, n, n_wg)] : 0;
        I tot;
        const I ex = block_excl_scan((I)c, s_ws, tot);
        if (k < n) {
          line[k] = c;
          ub[k] = lcarry + ex;
        }
        lcarry += tot;
      }
      __syncthreads();
      // XCD x starts at the first item whose cost midpoint is at or past
      // x C / 8: `reached` counts the x in 1 .. 7 with x C <= 4 (2 P + c),
      // P the item's prefix and c its cost
      auto reached = [&](int k) {
        const int64_t m4 = 4 * (2 * (int64_t)ub[k] + (int64_t)line[k]);
        int r = 0;
#pragma unroll
        for (int x = 1; x < kXcds; ++x) r += (int64_t)x * (int64_t)C <= m4 ? 1 : 0;
        return r;
      };
      for (int k = tid; k < n; k += kPlanThreads) {
        const int hi = reached(k), lo = k > 0 ? reached(k - 1) : 0;
        for (int x = lo + 1; x <= hi; ++x) s_xb[x] = k;
      }
      __syncthreads();
      int xb[kXcds];
#pragma unroll
      for (int x = 1; x < kXcds; ++x) xb[x] = s_xb[x];
      for (int k = tid; k < n; k += kPlanThreads) {
        int x = 0;   // the range holding k: the last x with start <= k
#pragma unroll
        for (int y = 1; y < kXcds; ++y) x += xb[y] <= k ? 1 : 0;
        const int r_lo = s_xb[x], r_hi = s_xb[x + 1];
        const int tail = min(xcd_wgs(n_wg, x), r_hi - r_lo);
        const int c = (int)line[k];
        int uix = k;
        if (k >= r_hi - tail) {   // decreasing cost, ties in list order
          int rank = 0;
#pragma unroll 8
          for (int k2 = r_hi - tail; k2 < r_hi; ++k2) {
            const int c2 = (int)line[k2];
            rank += (c2 > c || (c2 == c && k2 < k)) ? 1 : 0;
          }
          uix = r_hi - tail + rank;
        }
        const int j = dealt_pos(k, n, n_wg);
        const int b = iseq[j];
        const int2 gg = s_geo[j];
        a.units[2 * uix] = make_int4(start[b], slen[b], hist[b], gg.y);
        a.units[2 * uix + 1] = make_int4(gg.x, gg.x + c - kCostOverhead - 1, -1,
                                         (cand ? kUnitCandRows : 0) | 1);
      }
      if (tid == 0) {
        a.hdr[0] = n_wg;
        a.hdr[1] = cand ? 1 : 0;
        a.hdr[2] = kPlanXcdQueues;
        a.hdr[3] = 0;
        a.hdr[4] = n;
      }
      if (tid < kXcds) a.hdr[kHdrXcdCtr + tid] = 0;
      if (tid <= kXcds) a.hdr[kHdrXcdBound + tid] = s_xb[tid];
      return;
    }
  }

  // 3. Chunks per item; prefix sums of the units and of the split chunks.
  I ucarry = 0;
  for (int j0 = 0; j0 < n; j0 += kPlanThreads) {
    const int j = j0 + tid;
    I packed = 0;
    if (j < n) {
      const int c = cost[j];
      const int nc = item_chunks(line[j], c, c - kCostOverhead, T, a.no_split == 0,
                                 [](int, int, int, int) {});
      packed = (I)nc | ((I)(nc > 1 ? nc : 0) << kShift);
    }
    I tot;
    const I ex = block_excl_scan(packed, s_ws, tot);
    if (j < n) ub[j] = ucarry + ex;
    ucarry += tot;
  }
  if (tid == 0) ub[n] = ucarry;
  __syncthreads();

  // 4. Units, one per chunk in line order; count the units of every workgroup.
  for (int j = tid; j < n; j += kPlanThreads) {
    const int b = iseq[j];
    int kt_lo, qh;   // the geometry phase 2 found (LDS plans keep it)
    if constexpr (LDS) {
      const int2 gg = s_geo[j];
      kt_lo = gg.x;
      qh = gg.y;
    } else {
      const ItemGeo g = item_geo_of(dealt_item(j, n, n_wg), b, base, slen, hist,
                                    a.contextual_len, a.max_attn_len, cand, tr);
      kt_lo = g.kt_lo;
      qh = g.qt * H + g.h;
    }
    const int4 it = make_int4(start[b], slen[b], hist[b], qh);
    const int u0 = (int)(ub[j] & kLow), slot0 = (int)(ub[j] >> kShift);
    const int nc = (int)(ub[j + 1] & kLow) - u0;
    item_chunks(line[j], cost[j], cost[j] - kCostOverhead, T, a.no_split == 0,
                [&](int c, int tb, int te, int r) {
      a.units[2 * (u0 + c)] = it;
      a.units[2 * (u0 + c) + 1] = make_int4(kt_lo + tb, kt_lo + te - 1, nc > 1 ? slot0 : -1,
                                            (cand ? kUnitCandRows : 0) | (c << 16) | nc);
      atomicAdd(&s_cnt[share_wg(r, n_wg)], 1);
    });
    if (nc > 1) a.counters[slot0] = 0;
  }
  __syncthreads();

  // 5. First unit and unit count of every workgroup (shares in line order).
  int rcarry = 0;
  for (int f0 = 0; f0 < n_wg; f0 += kPlanThreads) {
    const int f = f0 + tid;
    const int v = f < n_wg ? share_wg(f, n_wg) : 0;
    const int cnt = f < n_wg ? s_cnt[v] : 0;
    int tot;
    const int ex = block_excl_scan(cnt, s_ws32, tot);
    if (f < n_wg) {
      a.wg[2 * v] = rcarry + ex;
      a.wg[2 * v + 1] = cnt;
    }
    rcarry += tot;
  }
  if (tid == 0) {
    a.hdr[0] = n_wg;
    a.hdr[1] = cand ? 1 : 0;
    a.hdr[2] = kPlanStatic;
    a.hdr[3] = 0;
    a.hdr[4] = (int)(ucarry & kLow);
  }
}

hipError_t launch_plan(const PlanArgs& a, bool compact, hipStream_t stream) {
  if (compact)
    hipLaunchKernelGGL((hstu_plan_kernel<int, true>), dim3(1), dim3(kPlanThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((hstu_plan_kernel<int64_t, false>), dim3(1), dim3(kPlanThreads), 0, stream,
                       a);
  return hipGetLastError();
}

}  // namespace hstu
