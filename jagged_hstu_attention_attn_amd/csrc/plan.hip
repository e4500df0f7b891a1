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
// One workgroup of 1024 threads; everything stays on the device, so the
// caller's stream never synchronises with the host.
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

__device__ inline int pair_key(const PlanArgs& a, int b, int qt) {
  const int s0 = a.offsets[b];
  const int L = a.offsets[b + 1] - s0;
  const int nt = a.num_targets ? a.num_targets[b] : 0;
  const SeqGeom g = seq_geom(L, nt, a.contextual_len, a.max_attn_len);
  const int i0 = qt * kBM;
  const int i1 = min(i0 + kBM, L);
  int jlo, jhi;
  tile_key_range(g, i0, i1, jlo, jhi);
  const int cost = jhi / kBN - jlo / kBN + 1 + 2;
  // descending work = ascending key
  return kKeyBuckets - 1 - work_bucket(cost);
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

__global__ __launch_bounds__(kPlanThreads) void hstu_plan_kernel(PlanArgs a) {
  __shared__ int s_wsum[kPlanThreads / 64];
  __shared__ int s_total;
  __shared__ int s_hist[kKeyBuckets];
  __shared__ int s_base[kKeyBuckets];
  __shared__ int s_wcnt[kPlanThreads / 64][kKeyBuckets];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.num_seqs;

  // 1. First pair of every sequence: exclusive scan of ceil(L_b / BM).
  int carry = 0;
  for (int b0 = 0; b0 < B; b0 += kPlanThreads) {
    const int b = b0 + tid;
    const int nq = b < B ? max(0, a.offsets[b + 1] - a.offsets[b] + kBM - 1) / kBM : 0;
    const int inc = block_inclusive_sum(nq, s_wsum);
    if (b < B) a.seq_start[b] = carry + inc - nq;
    if (tid == kPlanThreads - 1) s_total = inc;
    __syncthreads();
    carry += s_total;
    __syncthreads();
  }
  // Never more pairs than the work list holds (reached only by offsets that
  // break the documented contract).
  const int Q = min(carry, a.pairs_max);
  if (tid == 0) {
    a.seq_start[B] = Q;
    *a.count = Q;
  }
  if (tid < kKeyBuckets) s_hist[tid] = 0;
  __syncthreads();

  // 2. Work key of every pair, and the histogram of keys.
  for (int p = tid; p < Q; p += kPlanThreads) {
    const int b = find_seq(a.seq_start, B, p);
    const int key = pair_key(a, b, p - a.seq_start[b]);
    a.keys[p] = key;
    atomicAdd(&s_hist[key], 1);
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
  for (int w = tid; w < (kPlanThreads / 64) * kKeyBuckets; w += kPlanThreads)
    (&s_wcnt[0][0])[w] = 0;
  __syncthreads();

  // 4. Stable scatter, 1024 pairs at a time: rank inside the wave from a
  //    ballot match of the key bits, rank across waves from per-wave counts.
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int p0 = 0; p0 < Q; p0 += kPlanThreads) {
    const int p = p0 + tid;
    const bool valid = p < Q;
    const int key = valid ? a.keys[p] : 0;
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
    if (valid) {
      const int b = find_seq(a.seq_start, B, p);
      a.pairs[s_wcnt[wave][key] + rank] = make_int2(b, p - a.seq_start[b]);
    }
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
