// ln_heads.hip -- epilogue variant: LayerNorm over all heads of a token.
//
// The gate of "HSTU tensor by tensor: SiLU aggregation, temporal bias and
// gating" (section "Similar shape, different aggregation") normalises the
// aggregated values before multiplying by U.  The main kernel normalises each
// (token, head) over d_v; this variant normalises a token's H * d_v values
// together.  A workgroup cannot hold all heads of a token (heads are separate
// work items), so the attention kernel writes the raw outputs O / n_scale
// (epilogue "none") and this pass, one wave per token, reads the token's
// row (heads are consecutive d_v blocks), forms mean and variance with wave
// reductions, and writes (O - mean) * rstd * U back in place.
#include "hstu_device.hpp"

namespace hstu {

typedef float floatx4_ln __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_ln __attribute__((ext_vector_type(8)));

constexpr int kLnChunks = 8;   // 16-byte chunks per lane at most

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// T: element type; EPC: elements per 16-byte chunk.
// When the plan covered the candidate rows only (plan header word 1), rows
// of the history are left alone: they were not computed by this run.
template <typename T, int EPC>
__global__ __launch_bounds__(256) void hstu_ln_all_heads_kernel(LnArgs a) {
  T* out = static_cast<T*>(a.out);
  const T* u = static_cast<const T*>(a.u);
  const int64_t ld_out = a.ld_out, ld_u = a.ld_u;
  const int width = a.width;
  const float eps = a.eps;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.n_tok) return;   // whole waves leave together
  if (a.hdr[1] != 0) {        // candidates-only plan: skip history rows
    int lo = 0, hi = a.num_seqs - 1;   // sequence of token t: last b with offsets[b] <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.offsets[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int L = a.offsets[lo + 1] - a.offsets[lo];
    const int nt = a.num_targets ? clampi(a.num_targets[lo], 0, L) : 0;
    if (t - a.offsets[lo] < L - nt) return;
  }
  const int chunks = width / EPC;
  T* row = out + t * ld_out;
  const T* urow = u + t * ld_u;
  float x[kLnChunks][EPC];
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < kLnChunks; ++c) {
    const int ch = lane + 64 * c;
#pragma unroll
    for (int e = 0; e < EPC; ++e) x[c][e] = 0.0f;
    if (ch < chunks) {
      if constexpr (EPC == 8) {
        const bf16x8_ln v = *reinterpret_cast<const bf16x8_ln*>(row + EPC * ch);
#pragma unroll
        for (int e = 0; e < EPC; ++e) x[c][e] = (float)v[e];
      } else {
        const floatx4_ln v = *reinterpret_cast<const floatx4_ln*>(row + EPC * ch);
#pragma unroll
        for (int e = 0; e < EPC; ++e) x[c][e] = v[e];
      }
#pragma unroll
      for (int e = 0; e < EPC; ++e) sum += x[c][e];
    }
  }
  const float mean = wave_sum(sum) / (float)width;
  float sq = 0.0f;
#pragma unroll
  for (int c = 0; c < kLnChunks; ++c)
    if (lane + 64 * c < chunks) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) sq += (x[c][e] - mean) * (x[c][e] - mean);
    }
  const float rstd = rsqrtf(wave_sum(sq) / (float)width + eps);
#pragma unroll
  for (int c = 0; c < kLnChunks; ++c) {
    const int ch = lane + 64 * c;
    if (ch < chunks) {
      if constexpr (EPC == 8) {
        const bf16x8_ln uu = *reinterpret_cast<const bf16x8_ln*>(urow + EPC * ch);
        bf16x8_ln o;
#pragma unroll
        for (int e = 0; e < EPC; ++e) o[e] = (__bf16)((x[c][e] - mean) * rstd * (float)uu[e]);
        *reinterpret_cast<bf16x8_ln*>(row + EPC * ch) = o;
      } else {
        const floatx4_ln uu = *reinterpret_cast<const floatx4_ln*>(urow + EPC * ch);
        floatx4_ln o;
#pragma unroll
        for (int e = 0; e < EPC; ++e) o[e] = (x[c][e] - mean) * rstd * uu[e];
        *reinterpret_cast<floatx4_ln*>(row + EPC * ch) = o;
      }
    }
  }
}

int ln_all_heads_max_width(int dtype) { return 64 * kLnChunks * (dtype == 1 ? 8 : 4); }

hipError_t launch_ln_all_heads(const LnArgs& a, int dtype, hipStream_t stream) {
  if (a.n_tok <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.n_tok + 3) / 4)), block(256);
  if (dtype == 1)
    hipLaunchKernelGGL((hstu_ln_all_heads_kernel<__bf16, 8>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((hstu_ln_all_heads_kernel<float, 4>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace hstu
