// attn_fwd.hip -- gfx950 (CDNA4) jagged HSTU attention forward.
//
// One workgroup (4 waves) computes one (sequence, head, 128-row query tile)
// item of the work list.  Wave w owns query rows i0+32w .. i0+32w+31; lane
// (l % 32) owns one query row and the lane half (l / 32) splits the
// contraction dimension, which is the operand layout of the 32x32 MFMA.
//
// For each 32-key tile of the item's key range (staged in LDS, double
// buffered through registers):
//   S^T = K Q^T              32x32 block, bf16 MFMA (fp32 accumulate)
//   x   = alpha*S + pos[|i-j|] + time[bucket(|t_i - t_j|)]
//   a   = allowed(i,j) ? SiLU(x) : 0      select, never a multiply by a mask
//   O^T += V^T A^T           the SiLU values go straight from the first MFMA's
//                            accumulators into the second MFMA's B operand
// and after the last tile the epilogue scales by 1/n_scale, takes LayerNorm
// over d_v per (token, head) with the two lane halves combined by one
// cross-lane exchange, multiplies by U and stores the rows of the sequence.
//
// Computing S^T (keys along the MFMA's M dimension, queries along N) places
// every query row's scores in one lane, so the accumulator registers are
// already the B operand of the aggregation MFMA (the order of the contraction
// index inside one MFMA is free as long as both operands agree), and the
// LayerNorm reduction stays inside a lane pair.
//
// Method: pointwise SiLU aggregation with position/time bias, zeroing after
// the nonlinearity, Norm then U gating ("HSTU tensor by tensor: SiLU
// aggregation, temporal bias and gating", sections "SiLU aggregation
// coefficients are not probabilities", "Do not copy softmax masking
// mechanically", "Relative time adds information content similarity lacks",
// "Similar shape, different aggregation").
#include <type_traits>

#include "hstu_device.hpp"

namespace hstu {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int64_t kT32Range = int64_t(1) << 30;  // |t - base| below this -> 32-bit path

template <typename T>
struct TileCfg {
  static constexpr bool kBf16 = std::is_same<T, __bf16>::value;
  static constexpr int kEpc = 16 / sizeof(T);      // elements per 16-byte chunk
  static constexpr int kStep = kBf16 ? 16 : 2;     // MFMA contraction depth
};

template <typename T, int DQK, int DV>
struct Smem {
  static constexpr bool kBf16 = TileCfg<T>::kBf16;
  static constexpr int kKPitch = DQK + (kBf16 ? 8 : 4);     // elements per K row
  static constexpr int kVRows = kBf16 ? DV : kBN;           // bf16: V stored transposed
  static constexpr int kVPitch = kBf16 ? (kBN + 8) : (DV + 4);
  T k[2][kBN][kKPitch];
  T v[2][kVRows][kVPitch];
  int64_t tj64[2][kBN];
  uint32_t tj32[2][kBN];
  int tbad[2];
  float trev[32];   // trev[z] = time[min(31 - z, Tt - 1)], z = leading zeros of 1+|dt|
  float tful[64];   // tful[b] = time[min(b, Tt - 1)]
};

__device__ inline uint32_t abs_diff_u32(uint32_t a, uint32_t b) { return a > b ? a - b : b - a; }

template <typename T, int DQK, int DV>
__global__ __launch_bounds__(kThreads) void hstu_attn_fwd_kernel(AttnArgs a) {
  using Cfg = TileCfg<T>;
  using SM = Smem<T, DQK, DV>;
  constexpr bool BF = Cfg::kBf16;
  constexpr int EPC = Cfg::kEpc;
  constexpr int NKC = DQK / Cfg::kStep;           // MFMA steps of S^T
  constexpr int NDB = (DV + 31) / 32;             // 32-wide d_v blocks of O^T
  constexpr int KCH = kBN * DQK / EPC;            // 16-byte chunks per K tile
  constexpr int VCH = kBN * DV / EPC;
  constexpr int KPT = (KCH + kThreads - 1) / kThreads;
  constexpr int VPT = (VCH + kThreads - 1) / kThreads;
  static_assert(DQK % Cfg::kStep == 0 && DQK % EPC == 0 && DV % EPC == 0, "shape");
  static_assert(!BF || DV % 32 == 0, "bf16 needs d_v multiple of 32");

  __shared__ __align__(16) SM sm;
  extern __shared__ float pos_s[];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int H = a.num_heads;
  const int item = blockIdx.x / H;
  const int h = blockIdx.x - item * H;
  if (item >= *a.count) return;

  const int2 pr = a.pairs[item];
  const int b = pr.x, qt = pr.y;
  const int seq0 = a.offsets[b];
  const int L = a.offsets[b + 1] - seq0;
  const SeqGeom g = seq_geom(L, a.num_targets ? a.num_targets[b] : 0, a.contextual_len,
                             a.max_attn_len);
  const int i0 = qt * kBM;
  const int i1 = min(i0 + kBM, L);
  int jlo, jhi;
  tile_key_range(g, i0, i1, jlo, jhi);
  const int kt_lo = jlo / kBN, kt_hi = jhi / kBN;

  const bool has_pos = a.pos_len > 0;
  const bool has_time = a.time_len > 0;
  const int P = a.pos_len;

  // ---- per-lane query row ------------------------------------------------
  const int i = i0 + wave * 32 + l32;
  const bool row_valid = i < i1;
  const RowBounds rb = row_valid ? row_bounds(g, i) : RowBounds{kEmptyLo, 0, -1};

  int64_t tbase = 0, ti64 = 0;
  uint32_t ti32 = uint32_t(kT32Range);
  bool row_t_ok = true;
  if (has_time) {
    tbase = a.timestamps[seq0 + i0];
    ti64 = row_valid ? a.timestamps[seq0 + i] : tbase;
    const int64_t rel = ti64 - tbase;
    row_t_ok = rel > -kT32Range && rel < kT32Range;
    ti32 = row_t_ok ? uint32_t(rel + kT32Range) : 0u;
  }

  // ---- bias tables into LDS ----------------------------------------------
  if (has_pos) {
    const int maxrel = max(i0 + kBM - 1 - kt_lo * kBN, kt_hi * kBN + kBN - 1 - i0);
    const int n_pos = min(P, maxrel + 1);
    for (int x = tid; x < n_pos; x += kThreads) pos_s[x] = a.pos_table[x];
  }
  if (has_time) {
    const int Tt = a.time_len;
    if (tid < 32) sm.trev[tid] = a.time_table[min(31 - tid, Tt - 1)];
    if (tid < 64) sm.tful[tid] = a.time_table[min(tid, Tt - 1)];
  }

  // ---- Q operand (B operand of S^T = K Q^T), kept in registers ----------
  const T* qrow = reinterpret_cast<const T*>(a.q) + (int64_t)(seq0 + (row_valid ? i : i0)) * a.ld_q +
                  (int64_t)h * DQK;
  typename std::conditional<BF, bf16x8, float>::type qf[NKC];
#pragma unroll
  for (int c = 0; c < NKC; ++c) {
    if constexpr (BF) {
      bf16x8 z = {};
      qf[c] = row_valid ? *reinterpret_cast<const bf16x8*>(qrow + c * 16 + hh * 8) : z;
    } else {
      qf[c] = row_valid ? qrow[c * 2 + hh] : 0.0f;
    }
  }

  // ---- K/V tile staging: global -> registers -> LDS ----------------------
  const T* kbase = reinterpret_cast<const T*>(a.k) + (int64_t)h * DQK;
  const T* vbase = reinterpret_cast<const T*>(a.v) + (int64_t)h * DV;
  uint4 kreg[KPT], vreg[VPT];
  int64_t treg = 0;

  auto load_tile = [&](int kt) {
    const int j0 = kt * kBN;
#pragma unroll
    for (int s = 0; s < KPT; ++s) {
      const int c = tid + s * kThreads;
      const int row = c / (DQK / EPC), col = (c % (DQK / EPC)) * EPC;
      const int j = j0 + row;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (c < KCH && j < L)
        val = *reinterpret_cast<const uint4*>(kbase + (int64_t)(seq0 + j) * a.ld_k + col);
      kreg[s] = val;
    }
#pragma unroll
    for (int s = 0; s < VPT; ++s) {
      const int c = tid + s * kThreads;
      const int row = c / (DV / EPC), col = (c % (DV / EPC)) * EPC;
      const int j = j0 + row;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (c < VCH && j < L)
        val = *reinterpret_cast<const uint4*>(vbase + (int64_t)(seq0 + j) * a.ld_v + col);
      vreg[s] = val;
    }
    if (has_time && tid < kBN) {
      const int j = j0 + tid;
      treg = j < L ? a.timestamps[seq0 + j] : tbase;
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int s = 0; s < KPT; ++s) {
      const int c = tid + s * kThreads;
      const int row = c / (DQK / EPC), col = (c % (DQK / EPC)) * EPC;
      if (c < KCH) *reinterpret_cast<uint4*>(&sm.k[buf][row][col]) = kreg[s];
    }
#pragma unroll
    for (int s = 0; s < VPT; ++s) {
      const int c = tid + s * kThreads;
      const int row = c / (DV / EPC), col = (c % (DV / EPC)) * EPC;
      if (c < VCH) {
        if constexpr (BF) {
          const __bf16* e = reinterpret_cast<const __bf16*>(&vreg[s]);
#pragma unroll
          for (int x = 0; x < 8; ++x) sm.v[buf][col + x][row] = e[x];
        } else {
          *reinterpret_cast<uint4*>(&sm.v[buf][row][col]) = vreg[s];
        }
      }
    }
    if (has_time && tid < kBN) {
      const int64_t rel = treg - tbase;
      const bool ok = rel > -kT32Range && rel < kT32Range;
      sm.tj64[buf][tid] = treg;
      sm.tj32[buf][tid] = ok ? uint32_t(rel + kT32Range) : 0u;
      const uint64_t bad = __ballot(!ok);
      if (tid == 0) sm.tbad[buf] = bad != 0;
    }
  };

  floatx16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

  load_tile(kt_lo);
  store_tile(0);
  __syncthreads();

  const float alpha = a.alpha;
  const bool wave_rows = i0 + wave * 32 < i1;

  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int buf = (kt - kt_lo) & 1;
    if (kt < kt_hi) load_tile(kt + 1);

    const int jb = kt * kBN;
    const bool lane_any = row_valid && ((rb.lo <= jb + 31 && rb.lo + rb.span >= jb) ||
                                        (rb.self_j >= jb && rb.self_j <= jb + 31));
    const bool lane_full = !row_valid || (rb.lo <= jb && rb.lo + rb.span >= jb + 31);
    if (wave_rows && __any(lane_any)) {
      const bool full = __all(lane_full);
      const bool t_fast = !has_time || (!sm.tbad[buf] && __all(row_t_ok));

      // S^T[j][i] for the 32 keys of this tile and the wave's 32 rows.
      floatx16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.0f;
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
        if constexpr (BF) {
          const bf16x8 kop = *reinterpret_cast<const bf16x8*>(&sm.k[buf][l32][c * 16 + hh * 8]);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qf[c], s, 0, 0, 0);
        } else {
          const float kop = sm.k[buf][l32][c * 2 + hh];
          s = __builtin_amdgcn_mfma_f32_32x32x2f32(kop, qf[c], s, 0, 0, 0);
        }
      }

      // bias, SiLU, mask.  Register r holds key jb + 8(r/4) + 4hh + r%4.
      float av[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jj = 8 * (r >> 2) + 4 * hh + (r & 3);
        const int j = jb + jj;
        float x = alpha * s[r];
        if (has_pos) {
          const int d = min(abs(i - j), P - 1);
          x += pos_s[d];
        }
        if (has_time) {
          if (t_fast) {
            const uint32_t dt1 = abs_diff_u32(ti32, sm.tj32[buf][jj]) + 1u;
            x += sm.trev[__builtin_clz(dt1)];
          } else {
            const int64_t tj = sm.tj64[buf][jj];
            const uint64_t dt = ti64 >= tj ? uint64_t(ti64) - uint64_t(tj) : uint64_t(tj) - uint64_t(ti64);
            x += sm.tful[63 - __builtin_clzll(dt + 1u)];
          }
        }
        const float e = __builtin_amdgcn_exp2f(-x * kLog2e);
        float y = x * __builtin_amdgcn_rcpf(1.0f + e);
        if (!full) {
          const bool ok = (uint32_t)(j - rb.lo) <= (uint32_t)rb.span || j == rb.self_j;
          y = ok ? y : 0.0f;
        }
        av[r] = y;
      }

      // O^T[d][i] += sum_j V[j][d] * A[i][j]
      if constexpr (BF) {
        bf16x8 pa[2];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          pa[0][x] = (__bf16)av[x];
          pa[1][x] = (__bf16)av[8 + x];
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const __bf16* vp = &sm.v[buf][32 * db + l32][0];
#pragma unroll
          for (int ins = 0; ins < 2; ++ins) {
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vp + 16 * ins + 4 * hh);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vp + 16 * ins + 8 + 4 * hh);
            const bf16x8 vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pa[ins], acc[db], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = 32 * db + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int jj = 8 * (r >> 2) + 4 * hh + (r & 3);
            const float vop = d < DV ? sm.v[buf][jj][d] : 0.0f;
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vop, av[r], acc[db], 0, 0, 0);
          }
        }
      }
    }

    if (kt < kt_hi) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: 1/n_scale, LayerNorm over d_v, * U, store -----------------
  // acc[db][r] holds d = 32db + 8(r/4) + 4hh + r%4 of row i.
  const float inv_n = a.inv_n_scale;
  float mean = 0.0f, rstd = 1.0f;
  const bool ln = a.epilogue == 0;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] *= inv_n;
  if (ln) {
    float sum = 0.0f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * db + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (d < DV) sum += acc[db][r];
      }
    sum += __shfl_xor(sum, 32, 64);
    mean = sum * (1.0f / DV);
    float sq = 0.0f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * db + 8 * (r >> 2) + 4 * hh + (r & 3);
        const float c = acc[db][r] - mean;
        if (d < DV) sq += c * c;
      }
    sq += __shfl_xor(sq, 32, 64);
    rstd = rsqrtf(sq * (1.0f / DV) + a.ln_eps);
  }
  if (row_valid) {
    const int64_t tok = seq0 + i;
    T* orow = reinterpret_cast<T*>(a.out) + tok * a.ld_out + (int64_t)h * DV;
    const T* urow = reinterpret_cast<const T*>(a.u) + tok * a.ld_u + (int64_t)h * DV;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * db + 8 * gq + 4 * hh;
        if (d0 < DV) {
          float y[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) y[x] = acc[db][4 * gq + x];
          if (ln) {
            if constexpr (BF) {
              const bf16x4 uu = *reinterpret_cast<const bf16x4*>(urow + d0);
#pragma unroll
              for (int x = 0; x < 4; ++x) y[x] = (y[x] - mean) * rstd * (float)uu[x];
            } else {
              const floatx4 uu = *reinterpret_cast<const floatx4*>(urow + d0);
#pragma unroll
              for (int x = 0; x < 4; ++x) y[x] = (y[x] - mean) * rstd * uu[x];
            }
          }
          if constexpr (BF) {
            bf16x4 o;
#pragma unroll
            for (int x = 0; x < 4; ++x) o[x] = (__bf16)y[x];
            *reinterpret_cast<bf16x4*>(orow + d0) = o;
          } else {
            floatx4 o;
#pragma unroll
            for (int x = 0; x < 4; ++x) o[x] = y[x];
            *reinterpret_cast<floatx4*>(orow + d0) = o;
          }
        }
      }
  }
}

template <typename T, int DQK, int DV>
static hipError_t launch_one(const AttnArgs& a, int64_t grid, hipStream_t stream) {
  auto kern = hstu_attn_fwd_kernel<T, DQK, DV>;
  const size_t dyn = (size_t)(a.pos_len > 0 ? a.pos_len : 1) * sizeof(float);
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       kPosMax * (int)sizeof(float));
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), dyn, stream, a);
  return hipGetLastError();
}

bool attn_supported(int dtype, int d_qk, int d_v) {
  if (dtype == 1) return (d_qk == 128 && d_v == 128) || (d_qk == 64 && d_v == 64);
  if (dtype == 0) return (d_qk == 128 && d_v == 128) || (d_qk == 64 && d_v == 64) ||
                         (d_qk == 8 && d_v == 8);
  return false;
}

hipError_t launch_attn(const AttnArgs& a, int dtype, int d_qk, int d_v, int64_t grid,
                       hipStream_t stream) {
  if (dtype == 1) {
    if (d_qk == 128 && d_v == 128) return launch_one<__bf16, 128, 128>(a, grid, stream);
    if (d_qk == 64 && d_v == 64) return launch_one<__bf16, 64, 64>(a, grid, stream);
  } else if (dtype == 0) {
    if (d_qk == 128 && d_v == 128) return launch_one<float, 128, 128>(a, grid, stream);
    if (d_qk == 64 && d_v == 64) return launch_one<float, 64, 64>(a, grid, stream);
    if (d_qk == 8 && d_v == 8) return launch_one<float, 8, 8>(a, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace hstu
