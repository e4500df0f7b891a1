// layer.hip -- row LayerNorm of the layer input (no affine), bf16.
//
// The full HSTU layer normalises its input before the U/V/Q/K projection
// ("HSTU tensor by tensor: SiLU aggregation, temporal bias and gating",
// section "Trace four projections": normalised inputs produce the four
// projections).  One wave per token row: the row's `width` values are read
// as 16-byte chunks, mean and variance come from wave reductions, and the
// normalised row is written as bf16 for the projection GEMM.
#include "gemm.hpp"

namespace hstu {

typedef __bf16 l_bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kLnRowChunks = 8;   // 16-byte chunks per lane at most: width <= 4096

__device__ inline float l_wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__global__ __launch_bounds__(256) void hstu_layernorm_rows_kernel(const __bf16* x, int64_t ldx,
                                                                  __bf16* y, int64_t ldy,
                                                                  int rows, int width,
                                                                  float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= rows) return;   // whole waves leave together
  const int chunks = width / 8;
  const __bf16* xr = x + t * ldx;
  __bf16* yr = y + t * ldy;
  float v[kLnRowChunks][8];
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < kLnRowChunks; ++c) {
    const int ch = lane + 64 * c;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[c][e] = 0.0f;
    if (ch < chunks) {
      const l_bf16x8 w = *reinterpret_cast<const l_bf16x8*>(xr + 8 * ch);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[c][e] = (float)w[e];
        sum += v[c][e];
      }
    }
  }
  const float mean = l_wave_sum(sum) / (float)width;
  float sq = 0.0f;
#pragma unroll
  for (int c = 0; c < kLnRowChunks; ++c)
    if (lane + 64 * c < chunks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sq += (v[c][e] - mean) * (v[c][e] - mean);
    }
  const float rstd = rsqrtf(l_wave_sum(sq) / (float)width + eps);
#pragma unroll
  for (int c = 0; c < kLnRowChunks; ++c) {
    const int ch = lane + 64 * c;
    if (ch < chunks) {
      l_bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (__bf16)((v[c][e] - mean) * rstd);
      *reinterpret_cast<l_bf16x8*>(yr + 8 * ch) = o;
    }
  }
}

int layernorm_rows_max_width() { return 64 * kLnRowChunks * 8; }

hipError_t launch_layernorm_rows(const __bf16* x, int64_t ldx, __bf16* y, int64_t ldy, int rows,
                                 int width, float eps, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(hstu_layernorm_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                     stream, x, ldx, y, ldy, rows, width, eps);
  return hipGetLastError();
}

}  // namespace hstu
