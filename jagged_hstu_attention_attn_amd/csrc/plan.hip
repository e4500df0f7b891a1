// plan.hip -- device-side scheduler for the jagged HSTU attention kernel.
//
// Ragged execution must handle "boundaries, grouping and balance" ("Scaling
// HSTU: ragged execution, candidate amortization and content features",
// section "Variable length is a central systems issue").  The scheduler turns
// the jagged batch into work for a persistent attention launch on the 8 XCDs
// of an MI355X:
//
//   1. per sequence: length, candidates, query tiles (kBM rows) and a work
//      estimate L * reach, where reach is L (causal) or the window plus one
//      query tile (max attention length);
//   2. sequences are sorted by decreasing estimate (stable counting sort on a
//      quarter-octave bucket of the estimate);
//   3. (sequence, head) groups, in that order, are dealt to the 8 XCD queues in
//      snake order (0..7, 7..0, ...), which balances the queues' work and puts
//      the largest groups first in every queue;
//   4. each group's query tiles are listed consecutively, most expensive
//      (last) tile first, so that the tiles sharing a group's keys and values
//      run close together on one XCD and hit its L2.
//
// The attention workgroups of one XCD share its queue cyclically.  One workgroup of 1024 threads; everything
// stays on the device, so the caller's stream never synchronises with the host.
#include "hstu_device.hpp"

namespace hstu {

__device__ inline int work_bucket(int cost) {
  // floor(log2(cost)) * 4 + next two mantissa bits: nondecreasing in cost.
  const int e = 31 - __builtin_clz((unsigned)max(cost, 1));
  const int frac = e >= 2 ? ((cost >> (e - 2)) & 3) : ((cost << (2 - e)) & 3);
  const int bkt = 4 * e + frac;
  return bkt < kKeyBuckets - 1 ? bkt : kKeyBuckets - 1;
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

// Group r of the snake deal sits in queue q at slot s; inverse map.
__device__ inline int group_of_slot(int q, int s) {
  return kQueues * s + ((s & 1) ? (kQueues - 1 - q) : q);
}

__global__ __launch_bounds__(kPlanThreads) void hstu_plan_kernel(PlanArgs a) {
  __shared__ int s_wsum[kPlanThreads / 64];
  __shared__ int s_total;
  __shared__ int s_hist[kKeyBuckets];
  __shared__ int s_base[kKeyBuckets];
  __shared__ int s_wcnt[kPlanThreads / 64][kKeyBuckets];
  __shared__ int s_seq[6 * kPlanLdsSeqs];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.num_seqs, H = a.num_heads;
  int32_t* seq = B <= kPlanLdsSeqs ? s_seq : a.seq_scratch;
  const int LD = B <= kPlanLdsSeqs ? kPlanLdsSeqs : B;
  int32_t* len = seq;            // [B] history lengths
  int32_t* nqs = seq + LD;       // [B] query tiles
  int32_t* key = seq + 2 * LD;   // [B] sort key (ascending = decreasing work)
  int32_t* order = seq + 3 * LD; // [B] sequences by decreasing work
  int32_t* start = seq + 4 * LD; // [B] first token
  int32_t* slen = seq + 5 * LD;  // [B] tokens

  // 1. Per-sequence geometry and work estimate; histogram of keys.
  if (tid < kKeyBuckets) s_hist[tid] = 0;
  __syncthreads();
  for (int b = tid; b < B; b += kPlanThreads) {
    const int L = max(0, a.offsets[b + 1] - a.offsets[b]);
    const int nt = a.num_targets ? a.num_targets[b] : 0;
    const SeqGeom g = seq_geom(L, nt, a.contextual_len, a.max_attn_len);
    const int nq = (L + kBM - 1) / kBM;
    const int64_t reach = g.W > 0 ? min(L, g.W + kBM) : L;
    const int64_t cost = (int64_t)L * reach / 64 + nq;
    const int k = kKeyBuckets - 1 - work_bucket((int)min(cost, (int64_t)0x7fffffff));
    len[b] = g.n_h;   // history length (L minus clamped candidates)
    start[b] = a.offsets[b];
    slen[b] = L;
    nqs[b] = nq;
    key[b] = k;
    atomicAdd(&s_hist[k], 1);
  }
  __syncthreads();

  // 2. Stable counting sort of the sequences by key.
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
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int b0 = 0; b0 < B; b0 += kPlanThreads) {
    const int b = b0 + tid;
    const bool valid = b < B;
    const int k = valid ? key[b] : 0;
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
      const uint64_t m = __ballot(valid && ((k >> bit) & 1));
      same &= ((k >> bit) & 1) ? m : ~m;
    }
    const int rank = __popcll(same & lt_mask);
    if (valid && rank == 0) s_wcnt[wave][k] = __popcll(same);
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
    if (valid) order[s_wcnt[wave][k] + rank] = b;
    __syncthreads();
    for (int w = tid; w < (kPlanThreads / 64) * kKeyBuckets; w += kPlanThreads)
      (&s_wcnt[0][0])[w] = 0;
    __syncthreads();
  }

  // 3. Item offsets of the (queue, slot) groups: exclusive scan, queue-major.
  const int G = B * H, S = a.slots, F = kQueues * S;
  int carry = 0;
  for (int f0 = 0; f0 < F; f0 += kPlanThreads) {
    const int f = f0 + tid;
    int cnt = 0;
    if (f < F) {
      const int r = group_of_slot(f / S, f % S);
      if (r < G) cnt = nqs[order[r / H]];
    }
    const int inc = block_inclusive_sum(cnt, s_wsum);
    if (f < F) a.gscan[f] = carry + inc - cnt;
    if (tid == kPlanThreads - 1) s_total = inc;
    __syncthreads();
    carry += s_total;
    __syncthreads();
  }
  const int total = min(carry, a.items_max);   // never beyond the list's capacity
  if (tid == 0) a.gscan[F] = carry;
  __syncthreads();

  // 4. Items: every group's tiles, last (most expensive) tile first.
  for (int f = tid; f < F; f += kPlanThreads) {
    const int r = group_of_slot(f / S, f % S);
    if (r >= G) continue;
    const int b = order[r / H], h = r % H, nq = nqs[b];
    const int base = a.gscan[f];
    const int s0 = start[b], L = slen[b], n_h = len[b];
    for (int t = 0; t < nq && base + t < total; ++t)
      a.items[base + t] = make_int4(s0, L, n_h, (nq - 1 - t) * H + h);
  }

  // 5. Queue bounds.
  if (tid < kQueues) {
    const int s0 = min(a.gscan[tid * S], total);
    const int s1 = min(tid == kQueues - 1 ? carry : a.gscan[(tid + 1) * S], total);
    a.queue_start[tid] = s0;
    a.queue_count[tid] = s1 - s0;
  }
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(hstu_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hstu
