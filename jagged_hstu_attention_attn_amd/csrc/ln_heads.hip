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
#include <type_traits>

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

// T: element type; EPC: elements per 16-byte chunk; NCH: chunks per lane
// (the row width rounded up to a power of two, so registers fit the row).
// When the plan covered the candidate rows only (plan header word 1), rows
// of the history are left alone: they were not computed by this run.
template <typename T, int EPC, int NCH>
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
  // The U chunks are loaded together with the outputs, so the token's two
  // reads overlap instead of waiting for the reductions.
  using Vec = typename std::conditional<EPC == 8, bf16x8_ln, floatx4_ln>::type;
  float x[NCH][EPC];
  Vec uv[NCH];
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
#pragma unroll
    for (int e = 0; e < EPC; ++e) x[c][e] = 0.0f;
    if (ch < chunks) {
      const Vec v = *reinterpret_cast<const Vec*>(row + EPC * ch);
      uv[c] = *reinterpret_cast<const Vec*>(urow + EPC * ch);
#pragma unroll
      for (int e = 0; e < EPC; ++e) x[c][e] = (float)v[e];
#pragma unroll
      for (int e = 0; e < EPC; ++e) sum += x[c][e];
    }
  }
  const float mean = wave_sum(sum) / (float)width;
  float sq = 0.0f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    if (lane + 64 * c < chunks) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) sq += (x[c][e] - mean) * (x[c][e] - mean);
    }
  const float rstd = rsqrtf(wave_sum(sq) / (float)width + eps);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = lane + 64 * c;
    if (ch < chunks) {
      Vec o;
#pragma unroll
      for (int e = 0; e < EPC; ++e) o[e] = (T)((x[c][e] - mean) * rstd * (float)uv[c][e]);
      *reinterpret_cast<Vec*>(row + EPC * ch) = o;
    }
  }
}

int ln_all_heads_max_width(int dtype) { return 64 * kLnChunks * (dtype == 1 ? 8 : 4); }

template <typename T, int EPC>
hipError_t launch_width(const LnArgs& a, const dim3& grid, hipStream_t stream) {
  const int nch = (a.width / EPC + 63) / 64;
  const dim3 block(256);
  if (nch <= 1)
    hipLaunchKernelGGL((hstu_ln_all_heads_kernel<T, EPC, 1>), grid, block, 0, stream, a);
  else if (nch <= 2)
    hipLaunchKernelGGL((hstu_ln_all_heads_kernel<T, EPC, 2>), grid, block, 0, stream, a);
  else if (nch <= 4)
    hipLaunchKernelGGL((hstu_ln_all_heads_kernel<T, EPC, 4>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((hstu_ln_all_heads_kernel<T, EPC, kLnChunks>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_ln_all_heads(const LnArgs& a, int dtype, hipStream_t stream) {
  if (a.n_tok <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.n_tok + 3) / 4));
  return dtype == 1 ? launch_width<__bf16, 8>(a, grid, stream)
                    : launch_width<float, 4>(a, grid, stream);
}

}  // namespace hstu
