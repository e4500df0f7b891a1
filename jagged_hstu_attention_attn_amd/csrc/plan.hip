// plan.hip -- device-side scheduler for the jagged HSTU attention kernel.
//
// Splits every sequence into query tiles of kBM rows and orders the
// (sequence, query-tile) pairs by decreasing estimated work, so that the
// hardware dispatcher, which hands out workgroups in index order, starts the
// longest tiles first (longest-processing-time-first list scheduling).  This
// is the "grouping and balance" that ragged execution needs ("Scaling HSTU:
// ragged execution, candidate amortization and content features", section
// "Variable length is a central systems issue").
//
// The work estimate of a pair is the number of kBN-key tiles its rows can
// reach under the mask geometry, plus a constant for loading the queries and
// the epilogue.  Estimates are bucketed on a quarter-octave scale, and the
// sort is a stable counting sort, so pairs of equal bucket keep the natural
// (sequence, tile) order and the result is deterministic.
//
// One workgroup of 1024 threads.  Sequence lengths, candidate counts and the
// first pair of every sequence live in LDS for batches of up to kPlanLdsSeqs
// sequences (larger batches use the workspace copy), so the per-pair work is
// LDS-only after one coalesced pass over offsets.  Everything stays on the
// device: the caller's stream never synchronises with the host.
#include "hstu_device.hpp"

namespace hstu {

__device__ inline int work_bucket(int cost) {
  // floor(log2(cost)) * 4 + next two mantissa bits: nondecreasing in cost.
  const int e = 31 - __builtin_clz((unsigned)cost);
  const int frac = e >= 2 ? ((cost >> (e - 2)) & 3) : ((cost << (2 - e)) & 3);
  const int bkt = 4 * e + frac;
  return bkt < kKeyBuckets - 1 ? bkt : kKeyBuckets - 1;
}

// Largest b in [0, B) with seq_start[b] <= p (seq_start nondecreasing).
__device__ inline int find_seq(const int32_t* seq_start, int B, int p) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seq_start[mid] <= p) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Inclusive sum over the 1024 threads of the block; `ws` holds 16 ints.
__device__ inline int block_inclusive_sum(int x, int* ws) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) ws[wave] = x;
  __syncthreads();
  int pre = 0;
  for (int w = 0; w < wave; ++w) pre += ws[w];
  __syncthreads();
  return x + pre;
}

struct SeqView {
  const int32_t* start;   // [B+1] first pair of each sequence (LDS or workspace)
  const int32_t* len;     // [B] lengths (LDS), or nullptr: read offsets
  const int32_t* nt;      // [B] candidate counts (LDS), or nullptr: read num_targets
};

__device__ inline int pair_key(const PlanArgs& a, const SeqView& sv, int b, int qt) {
  const int L = sv.len ? sv.len[b] : a.offsets[b + 1] - a.offsets[b];
  const int nt = sv.nt ? sv.nt[b] : (a.num_targets ? a.num_targets[b] : 0);
  const SeqGeom g = seq_geom(L, nt, a.contextual_len, a.max_attn_len);
  const int i0 = qt * kBM;
  const int i1 = min(i0 + kBM, L);
  int jlo, jhi;
  tile_key_range(g, i0, i1, jlo, jhi);
  const int cost = jhi / kBN - jlo / kBN + 1 + 2;
  return kKeyBuckets - 1 - work_bucket(cost);   // descending work = ascending key
}

__global__ __launch_bounds__(kPlanThreads) void hstu_plan_kernel(PlanArgs a) {
  __shared__ int s_wsum[kPlanThreads / 64];
  __shared__ int s_total;
  __shared__ int s_hist[kKeyBuckets];
  __shared__ int s_base[kKeyBuckets];
  __shared__ int s_wcnt[kPlanThreads / 64][kKeyBuckets];
  __shared__ int s_start[kPlanLdsSeqs + 1];
  __shared__ int s_len[kPlanLdsSeqs];
  __shared__ int s_nt[kPlanLdsSeqs];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.num_seqs;
  const bool in_lds = B <= kPlanLdsSeqs;
  int32_t* start = in_lds ? s_start : a.seq_start;

  // 1. Lengths, candidate counts, and the first pair of every sequence
  //    (exclusive scan of ceil(L_b / BM)).
  int carry = 0;
  for (int b0 = 0; b0 < B; b0 += kPlanThreads) {
    const int b = b0 + tid;
    int L = 0, nt = 0;
    if (b < B) {
      L = max(0, a.offsets[b + 1] - a.offsets[b]);
      nt = a.num_targets ? a.num_targets[b] : 0;
      if (in_lds) {
        s_len[b] = L;
        s_nt[b] = nt;
      }
    }
    const int nq = (L + kBM - 1) / kBM;
    const int inc = block_inclusive_sum(nq, s_wsum);
    if (b < B) start[b] = carry + inc - nq;
    if (tid == kPlanThreads - 1) s_total = inc;
    __syncthreads();
    carry += s_total;
    __syncthreads();
  }
  // Never more pairs than the work list holds (reached only by offsets that
  // break the documented contract).
  const int Q = min(carry, a.pairs_max);
  if (tid == 0) {
    start[B] = Q;
    *a.count = Q;
  }
  if (tid < kKeyBuckets) s_hist[tid] = 0;
  for (int w = tid; w < (kPlanThreads / 64) * kKeyBuckets; w += kPlanThreads)
    (&s_wcnt[0][0])[w] = 0;
  __syncthreads();
  const SeqView sv{start, in_lds ? s_len : nullptr, in_lds ? s_nt : nullptr};

  // 2. Histogram of work keys.
  for (int p = tid; p < Q; p += kPlanThreads) {
    const int b = find_seq(sv.start, B, p);
    atomicAdd(&s_hist[pair_key(a, sv, b, p - sv.start[b])], 1);
  }
  __syncthreads();

  // 3. Start of every key bucket (exclusive scan over 64 buckets, one wave).
  if (wave == 0) {
    int x = s_hist[lane];
    const int own = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    s_base[lane] = x - own;
  }
  __syncthreads();

  // 4. Stable scatter, 1024 pairs at a time: rank inside the wave from a
  //    ballot match of the key bits, rank across waves from per-wave counts.
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int p0 = 0; p0 < Q; p0 += kPlanThreads) {
    const int p = p0 + tid;
    const bool valid = p < Q;
    int b = 0, qt = 0, key = 0;
    if (valid) {
      b = find_seq(sv.start, B, p);
      qt = p - sv.start[b];
      key = pair_key(a, sv, b, qt);
    }
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
      const uint64_t m = __ballot(valid && ((key >> bit) & 1));
      same &= ((key >> bit) & 1) ? m : ~m;
    }
    const int rank = __popcll(same & lt_mask);
    if (valid && rank == 0) s_wcnt[wave][key] = __popcll(same);
    __syncthreads();
    if (tid < kKeyBuckets) {
      int run = s_base[tid];
      for (int w = 0; w < kPlanThreads / 64; ++w) {
        const int c = s_wcnt[w][tid];
        s_wcnt[w][tid] = run;
        run += c;
      }
      s_base[tid] = run;
    }
    __syncthreads();
    if (valid) a.pairs[s_wcnt[wave][key] + rank] = make_int2(b, qt);
    __syncthreads();
    for (int w = tid; w < (kPlanThreads / 64) * kKeyBuckets; w += kPlanThreads)
      (&s_wcnt[0][0])[w] = 0;
    __syncthreads();
  }
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(hstu_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hstu
