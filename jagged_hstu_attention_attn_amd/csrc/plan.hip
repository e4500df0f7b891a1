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
//      it reach (tile_key_range) plus a fixed term;
//   2. the items are cut into 8 consecutive portions of about equal cost,
//      one per XCD (an item goes to the portion holding its midpoint);
//   3. inside the portion of XCD x the items are dealt round-robin to the
//      W_x workgroups of that XCD, and the dealt order (workgroup 0's items,
//      then workgroup 1's, ...) is cut into W_x shares of equal cost
//      T_x = ceil(C_x / W_x).  With items of equal cost the shares are the
//      dealt columns, so workgroups running side by side process neighbouring
//      query tiles, whose key/value rows their XCD's L2 then serves once;
//   4. an item that a share boundary cuts is split there along its key tiles
//      (proportionally, never into chunks under kMinChunk tiles): the
//      pointwise aggregation is a sum over keys, so the chunks' partial
//      outputs add up exactly to the item's output.
//
// One workgroup of 1024 threads; the per-item arrays stay in LDS up to
// kPlanLdsItems items.  Everything stays on the device, so the caller's
// stream never synchronises with the host.
#include <type_traits>

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
// shares of T units.  Each multiple rT strictly inside the span is a candidate
// cut at tile offset t = floor((rT - P) * tiles / cost).  A cut that would
// close a chunk of fewer than kMinChunk tiles instead hands the open chunk to
// share r; a cut that would leave fewer than kMinChunk tiles after it is
// dropped.  f(j, tb, te, r): chunk j covers tile offsets [tb, te) and belongs
// to share r.  Owners never decrease along the line.  Returns the number of
// chunks.
template <typename I, typename F>
__device__ inline int item_chunks(I P, int cost, int tiles, I T, F&& f) {
  using U = typename std::make_unsigned<I>::type;   // products stay below 2^(bits of I)
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

// Item k of sequence b (head-major, last query tile first).
__device__ inline ItemGeo item_geo_of(int k, int b, const int32_t* base, const int32_t* slen,
                                      const int32_t* hist, int contextual_len,
                                      int max_attn_len) {
  ItemGeo r;
  r.b = b;
  const int L = slen[b], nq = (L + kBM - 1) / kBM;
  const int t = k - base[b];
  r.h = t / nq;
  r.qt = nq - 1 - (t - r.h * nq);
  SeqGeom g;
  g.L = L;
  g.n_h = hist[b];
  g.c = clampi(contextual_len, 0, g.n_h);
  g.W = max_attn_len;
  const int i0 = r.qt * kBM, i1 = min(i0 + kBM, L);
  int jlo, jhi;
  tile_key_range(g, i0, i1, jlo, jhi);
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
  __shared__ int s_xa[kXcds + 1];                 // first item of each XCD's portion
  __shared__ int s_seq[4 * (kPlanLdsSeqs + 1)];
  __shared__ int s_cost[kItems + 1];
  __shared__ int s_order[kItems];
  __shared__ int s_iseq[kItems];
  __shared__ I s_line[kItems + 1];
  __shared__ I s_ub[kItems + 1];

  const int tid = threadIdx.x;
  const int B = a.num_seqs, H = a.num_heads, n_wg = a.n_wg;
  int32_t* seq = B <= kPlanLdsSeqs ? s_seq : a.seq_scratch;
  const int LD = B <= kPlanLdsSeqs ? kPlanLdsSeqs + 1 : B + 1;
  int32_t* base = seq;            // [B + 1] first item of each sequence
  int32_t* start = seq + LD;      // [B] first token
  int32_t* slen = seq + 2 * LD;   // [B] tokens
  int32_t* hist = seq + 3 * LD;   // [B] history tokens (L minus clamped candidates)

  for (int v = tid; v < kMaxGrid; v += kPlanThreads) s_cnt[v] = 0;

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
      cnt = (L + kBM - 1) / kBM * H;
    }
    int tot;
    const int ex = block_excl_scan(cnt, s_ws32, tot);
    if (b < B) base[b] = carry + ex;
    carry += tot;
  }
  const int n = min(carry, a.items_max);   // never beyond the scratch's capacity
  if (tid <= kXcds) s_xa[tid] = n;

  int* cost = s_cost;
  int* order = s_order;
  I* line = s_line;
  I* ub = s_ub;
  if constexpr (!LDS) {
    const size_t im = (size_t)a.items_max + 1;
    cost = reinterpret_cast<int*>(a.item_scratch);
    order = cost + im;
    line = reinterpret_cast<I*>(a.item_scratch + ((2 * sizeof(int) * im + 15) & ~size_t(15)));
    ub = line + im;
  }
  __syncthreads();

  // 2. Item costs and their prefix sums in list order.
  I ccarry = 0;
  for (int k0 = 0; k0 < n; k0 += kPlanThreads) {
    const int k = k0 + tid;
    int c = 0;
    if (k < n) {
      const int b = seq_of(k, base, B);
      const ItemGeo g = item_geo_of(k, b, base, slen, hist, a.contextual_len, a.max_attn_len);
      c = g.kt_hi - g.kt_lo + 1 + kCostOverhead;
      cost[k] = c;
      if constexpr (LDS) s_iseq[k] = b;
    }
    I tot;
    const I ex = block_excl_scan((I)c, s_ws, tot);
    if (k < n) line[k] = ccarry + ex;
    ccarry += tot;
  }
  const I C = ccarry;
  __syncthreads();

  // 3. XCD portions: item k goes to XCD floor(8 * midpoint / C).
  using U = typename std::make_unsigned<I>::type;
  for (int k = tid; k < n; k += kPlanThreads) {
    auto xcd_of = [&](int i) {
      const U m = (U)(2 * line[i] + cost[i]) * (U)(kXcds / 2) / (U)C;
      return (int)(m < (U)kXcds ? m : (U)(kXcds - 1));
    };
    const int xk = xcd_of(k), xp = k > 0 ? xcd_of(k - 1) : -1;
    for (int x = xp + 1; x <= xk; ++x) s_xa[x] = k;
  }
  __syncthreads();

  // 4. Dealt order inside each portion (column-major over the XCD's workgroups).
  for (int k = tid; k < n; k += kPlanThreads) {
    int x = 0;
    while (x < kXcds - 1 && s_xa[x + 1] <= k) ++x;
    const int a0 = s_xa[x], nx = s_xa[x + 1] - a0, W = xcd_wgs(n_wg, x);
    const int i = k - a0, col = i % W, row = i / W;
    const int full = nx / W, extra = nx % W;
    order[a0 + col * full + min(col, extra) + row] = k;
  }
  __syncthreads();

  // 5. Cost prefix sums in dealt order (portions stay where they were).
  ccarry = 0;
  for (int j0 = 0; j0 < n; j0 += kPlanThreads) {
    const int j = j0 + tid;
    const int c = j < n ? cost[order[j]] : 0;
    I tot;
    const I ex = block_excl_scan((I)c, s_ws, tot);
    if (j < n) line[j] = ccarry + ex;
    ccarry += tot;
  }
  if (tid == 0) line[n] = ccarry;
  __syncthreads();

  // 6. Chunks per dealt item; prefix sums of the units and of the split chunks.
  auto share_of = [&](int j, int& x, I& P, I& T) {
    x = 0;
    while (x < kXcds - 1 && s_xa[x + 1] <= j) ++x;
    const I p0 = line[s_xa[x]];
    const I Cx = line[s_xa[x + 1]] - p0;
    const int W = xcd_wgs(n_wg, x);
    P = line[j] - p0;
    T = Cx > 0 ? (Cx + W - 1) / W : 1;
  };
  I ucarry = 0;
  for (int j0 = 0; j0 < n; j0 += kPlanThreads) {
    const int j = j0 + tid;
    I packed = 0;
    if (j < n) {
      int x;
      I P, T;
      share_of(j, x, P, T);
      const int c = cost[order[j]];
      const int nc = item_chunks(P, c, c - kCostOverhead, T, [](int, int, int, int) {});
      packed = (I)nc | ((I)(nc > 1 ? nc : 0) << kShift);
    }
    I tot;
    const I ex = block_excl_scan(packed, s_ws, tot);
    if (j < n) ub[j] = ucarry + ex;
    ucarry += tot;
  }
  if (tid == 0) ub[n] = ucarry;
  __syncthreads();

  // 7. Units, one per chunk in dealt order; count the units of every workgroup.
  for (int j = tid; j < n; j += kPlanThreads) {
    int x;
    I P, T;
    share_of(j, x, P, T);
    const int k = order[j];
    int b;
    if constexpr (LDS) b = s_iseq[k];
    else b = seq_of(k, base, B);
    const ItemGeo g = item_geo_of(k, b, base, slen, hist, a.contextual_len, a.max_attn_len);
    const int4 it = make_int4(start[b], slen[b], g.n_h, g.qt * H + g.h);
    const int u0 = (int)(ub[j] & kLow), slot0 = (int)(ub[j] >> kShift);
    const int nc = (int)(ub[j + 1] & kLow) - u0;
    item_chunks(P, cost[k], g.kt_hi - g.kt_lo + 1, T, [&](int c, int tb, int te, int r) {
      a.units[2 * (u0 + c)] = it;
      a.units[2 * (u0 + c) + 1] =
          make_int4(g.kt_lo + tb, g.kt_lo + te - 1, nc > 1 ? slot0 : -1, (c << 16) | nc);
      atomicAdd(&s_cnt[x + kXcds * r], 1);
    });
    if (nc > 1) a.counters[slot0] = 0;
  }
  __syncthreads();

  // 8. First unit and unit count of every workgroup (shares XCD-major, in
  //    the order their units were written).
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
  if (tid == 0) a.hdr[0] = n_wg;
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
