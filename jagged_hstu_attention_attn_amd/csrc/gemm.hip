// gemm.hip -- bf16 MFMA GEMM with fused epilogues for the full HSTU layer.
//
// The layer ("HSTU tensor by tensor: SiLU aggregation, temporal bias and
// gating", sections "Follow the U, V, Q and K branches" and "Trace four
// projections"; the teaching equation of "Similar shape, different
// aggregation") wraps the attention in two projections: one fused U/V/Q/K
// projection of the normalised input followed by SiLU, and an output
// projection plus the residual.  Both are C = A * B^T with
//   A [M, K] bf16 (tokens, token stride lda),
//   B [N, K] bf16 (weights in the [out, in] layout, row stride ldb),
//   C [M, N] bf16 (token stride ldc),
// fp32 accumulation and an epilogue  C = act(A B^T + bias) + residual  with
// act = SiLU or identity, bias bf16 [N] or none, residual bf16 [M, N] or none.
//
// Tiling: a workgroup of 4 waves computes a 128 x 128 block of C; wave (wn,
// wm) holds 64 x 64 of it as 2 x 2 tiles of v_mfma_f32_32x32x16_bf16 with the
// weight rows on the MFMA's M side and the tokens on N, so each lane ends up
// with 16 outputs of one token.  K advances 32 at a time through two LDS
// stages filled by global_load_lds_dwordx4 (16-byte chunks XOR-swizzled by
// row), one stage ahead: 32 KB of LDS and at most 128 registers, so four
// workgroups share a CU and one's loads and epilogue overlap the others'
// matrix work (a tile is only K / 32 stages long).  The epilogue parks the
// fp32 block in LDS 64 token rows at a time (the two stages' space) and
// writes whole rows: every lane finishes 8 consecutive outputs of one token
// (bias, SiLU, residual, bf16) and stores them as one 16-byte chunk, 8 full
// 128-byte lines per wave instruction.
// Requires N % 128 == 0, K % 32 == 0, 16-byte aligned rows; M is arbitrary.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.hpp"

namespace hstu {

typedef __bf16 g_bf16x8 __attribute__((ext_vector_type(8)));
typedef float g_floatx4 __attribute__((ext_vector_type(4)));
typedef float g_floatx16 __attribute__((ext_vector_type(16)));

constexpr int kGB = 128;    // block of C: rows (tokens) and columns (features)
constexpr int kGK = 32;     // K per stage
constexpr int kGThreads = 256;
constexpr int kGXcds = 8;   // XCDs of the MI355X

__device__ inline uint32_t g_lds_off(const void* p) { return (uint32_t)(uintptr_t)p; }
template <typename V>
__device__ inline V g_lds_ld(uint32_t off) {
  return *(__attribute__((address_space(3))) const V*)(uintptr_t)off;
}
template <typename V>
__device__ inline void g_lds_st(uint32_t off, V v) {
  *(__attribute__((address_space(3))) V*)(uintptr_t)off = v;
}
__device__ inline uint64_t g_uni_ptr(const void* p) {
  const uint64_t x = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// HBM -> LDS copy of 16 bytes per lane (lane l lands at lds + 16 l); `base`
// and `lds` uniform.  Waited for with s_waitcnt vmcnt.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void g_lds_copy16(uint64_t base, uint32_t voff, uint32_t lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(m), "v"(voff), "s"(base) : "memory", "m0");
}
#pragma clang diagnostic pop

// Workgroup barrier that waits for this wave's LDS accesses only: the copies
// of the next stage stay in flight (__syncthreads would wait for them too).
__device__ inline void g_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Staged tile: 128 rows x 32 k (64 bytes = 4 chunks per row); physical chunk
// c of row r holds logical chunk c ^ ((r >> 2) & 3): the 16 rows one
// 16-lane phase of a fragment read touches land on 16 different 16-byte
// bank groups.
__device__ inline int g_swz(int r) { return (r >> 2) & 3; }

__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(4))) void
hstu_gemm_bt_kernel(GemmArgs a) {
  __shared__ __align__(16) char smem[2 * 2 * kGB * kGK * 2];   // 2 stages x (W, X) tiles
  static_assert(2 * 2 * kGB * kGK * 2 == 64 * 512, "half the fp32 block fits the stages");
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave >> 1, wm = wave & 1;   // wave's 64 x 64 sub-block: features wn, tokens wm
  // XCD-aware tile order: the MI355X dispatches workgroup g to XCD g % 8,
  // and each XCD has its own L2.  XCD x takes the contiguous tile range
  // [x * per, (x + 1) * per) in token-block-major order, so the N / 128
  // workgroups that read one 128-token block of A run on one XCD, close in
  // time, and its L2 serves that block to all of them.
  const int nN = a.N / kGB, nT = nN * ((a.M + kGB - 1) / kGB);
  const int per = (nT + kGXcds - 1) / kGXcds;
  const int t = (int)(blockIdx.x % kGXcds) * per + (int)(blockIdx.x / kGXcds);
  if (t >= nT) return;
  const int n0 = (t % nN) * kGB, m0 = (t / nN) * kGB;
  const int M = a.M, K = a.K;
  constexpr int kTile = kGB * kGK * 2;   // bytes of one staged 128 x 32 tile
  const uint32_t s0 = g_lds_off(smem);
  auto w_tile = [&](int st) { return s0 + (uint32_t)(st * 2 * kTile); };
  auto x_tile = [&](int st) { return s0 + (uint32_t)(st * 2 * kTile + kTile); };

  const uint64_t wb = g_uni_ptr(reinterpret_cast<const char*>(a.B) + (int64_t)n0 * a.ldb * 2);
  const uint64_t xb = g_uni_ptr(reinterpret_cast<const char*>(a.A) + (int64_t)m0 * a.lda * 2);
  const uint32_t ldb_b = (uint32_t)(a.ldb * 2), lda_b = (uint32_t)(a.lda * 2);
  const int m_last = min(kGB, M - m0) - 1;   // rows past M repeat the last token

  // Stage kb: each wave copies 2 + 2 chunks-of-64-lanes of the two tiles.
  auto issue = [&](int st, int kb) __attribute__((always_inline)) {
    const uint32_t kbyte = (uint32_t)kb * kGK * 2;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int n = s * 4 + wave, m = 64 * n + lane, r = m >> 2, c = m & 3;
      const uint32_t coff = kbyte + 16u * (uint32_t)(c ^ g_swz(r));
      g_lds_copy16(wb, (uint32_t)r * ldb_b + coff, w_tile(st) + 1024u * (uint32_t)n);
      g_lds_copy16(xb, (uint32_t)min(r, m_last) * lda_b + coff, x_tile(st) + 1024u * (uint32_t)n);
    }
  };

  g_floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nkb = K / kGK;
  issue(0, 0);
  for (int kb = 0; kb < nkb; ++kb) {
    const int st = kb & 1;
    if (kb + 1 < nkb) {
      issue(st ^ 1, kb + 1);
      __builtin_amdgcn_s_waitcnt(4 | (7 << 4) | (15 << 8));   // vmcnt(4): stage kb landed
    } else {
      __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
    }
    g_barrier();
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks) {
      g_bf16x8 wf[2], xf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int rw = 64 * wn + 32 * i + l32, rx = 64 * wm + 32 * i + l32;
        const int c = 2 * ks + hh;
        wf[i] = g_lds_ld<g_bf16x8>(w_tile(st) + (uint32_t)(rw * 64 + 16 * (c ^ g_swz(rw))));
        xf[i] = g_lds_ld<g_bf16x8>(x_tile(st) + (uint32_t)(rx * 64 + 16 * (c ^ g_swz(rx))));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], xf[j], acc[i][j], 0, 0, 0);
    }
    g_barrier();   // the stage may be refilled by the next iteration's copies
  }

  // Epilogue, in two halves of 64 tokens (the waves with wm == half park
  // theirs).  acc[i][j][r]: feature 64wn + 32i + 8(r/4) + 4hh + r%4 of token
  // 64wm + 32j + l32.  fp32 half-block C[token][feature] in LDS, 512 bytes
  // per token row, 16-byte chunk c of row t at physical chunk c ^ (t & 15).
  const int oc = tid & 15;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int t = 32 * j + l32;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int f = 64 * wn + 32 * i + 8 * g + 4 * hh;   // 4 consecutive features
            g_floatx4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
            g_lds_st<g_floatx4>(s0 + (uint32_t)(t * 512 + 16 * ((f >> 2) ^ (t & 15))), v);
          }
        }
    }
    __syncthreads();
    // 64 rows x 16 chunks of 8 outputs; thread handles chunk (tid & 15) of
    // rows (tid >> 4) + 16 p
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int t = (tid >> 4) + 16 * p;
      const int tt = 64 * half + t;   // token within the block
      if (m0 + tt > M - 1) continue;
      const int f = 8 * oc;   // features f .. f+7 of the block
      const g_floatx4 lo =
          g_lds_ld<g_floatx4>(s0 + (uint32_t)(t * 512 + 16 * ((f >> 2) ^ (t & 15))));
      const g_floatx4 hi =
          g_lds_ld<g_floatx4>(s0 + (uint32_t)(t * 512 + 16 * (((f >> 2) + 1) ^ (t & 15))));
      float y[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      if (a.bias) {
        const g_bf16x8 b = *reinterpret_cast<const g_bf16x8*>(a.bias + n0 + f);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] += (float)b[e];
      }
      if (a.act_silu) {
#pragma unroll
        for (int e = 0; e < 8; ++e)   // y * sigmoid(y) = y / (1 + 2^(-y log2 e))
          y[e] = y[e] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * y[e]));
      }
      const int64_t row = m0 + tt;
      if (a.residual) {
        const g_bf16x8 rsd =
            *reinterpret_cast<const g_bf16x8*>(a.residual + row * a.ldr + n0 + f);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] += (float)rsd[e];
      }
      g_bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (__bf16)y[e];
      *reinterpret_cast<g_bf16x8*>(a.C + row * a.ldc + n0 + f) = o;
    }
    if (half == 0) __syncthreads();   // the first half is read before the second lands
  }
}

bool gemm_shape_ok(int M, int N, int K) { return M >= 0 && N % kGB == 0 && K % kGK == 0 && K > 0; }

hipError_t launch_gemm_bt(const GemmArgs& a, hipStream_t stream) {
  if (a.M <= 0) return hipSuccess;
  const int nT = (a.N / kGB) * ((a.M + kGB - 1) / kGB);
  const dim3 grid((unsigned)(kGXcds * ((nT + kGXcds - 1) / kGXcds))), block(kGThreads);
  hipLaunchKernelGGL(hstu_gemm_bt_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace hstu
