// gemm.hpp -- argument block and launchers of the layer's GEMMs and row
// LayerNorm (gemm.hip, layer.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

// C[M, N] = act(A[M, K] * B[N, K]^T + bias[N]) + residual[M, N], bf16 in and
// out, fp32 accumulation.  Pointers are bf16 (passed as __bf16*).
struct GemmArgs {
  const __bf16* A;
  const __bf16* B;
  const __bf16* bias;       // or nullptr
  const __bf16* residual;   // or nullptr
  __bf16* C;
  int64_t lda, ldb, ldc, ldr;   // row strides in elements
  int32_t M, N, K;
  int32_t act_silu;         // 1: SiLU after the bias
};

bool gemm_shape_ok(int M, int N, int K);
hipError_t launch_gemm_bt(const GemmArgs& a, hipStream_t stream);

// y[t, :] = LayerNorm(x[t, :]) over `width` values (no affine), bf16.
hipError_t launch_layernorm_rows(const __bf16* x, int64_t ldx, __bf16* y, int64_t ldy, int rows,
                                 int width, float eps, hipStream_t stream);
int layernorm_rows_max_width();

}  // namespace hstu
