// attn_fwd.hip -- gfx950 (CDNA4) jagged HSTU attention forward.
//
// One workgroup (4 waves) computes one (sequence, head, 128-row query tile)
// item of the work list.  Wave w owns query rows i0+32w .. i0+32w+31; lane
// (l % 32) owns one query row and the lane half (l / 32) splits the
// contraction dimension, which is the operand layout of the 32x32 MFMA.
//
// Keys are staged 64 at a time in LDS (global -> registers -> LDS, the next
// tile's loads in flight while the current one is computed).  Each 32-key
// block of a tile:
//   S^T = K Q^T                 32x32, bf16 MFMA with fp32 accumulation
//   x   = alpha*S + pos[|i-j|] + time[floor(log2(1+|t_i-t_j|))]
//   a   = allowed(i,j) ? SiLU(x) : 0     a select, never a multiply by a mask
//   O^T += V^T A^T              the SiLU values go from the first MFMA's
//                               accumulator registers straight into the
//                               second MFMA's B operand
// and the epilogue scales by 1/n_scale, takes LayerNorm over d_v per (token,
// head) (the two lane halves of a row combine with one cross-lane exchange),
// multiplies by U and stores the rows that belong to the sequence.
//
// Computing S^T (keys on the MFMA's M side, queries on N) puts every query
// row's scores in one lane, so the accumulators already have the B-operand
// layout of the aggregation MFMA (the order of the contraction index inside
// one MFMA is free as long as both operands agree).  V stays row-major in LDS
// and its transposed operand comes from ds_read_b64_tr_b16.
//
// Scores are kept in log2 units: the bias tables are staged pre-multiplied by
// log2(e), x2 = alpha*log2(e)*S + bias2, and SiLU(x)*log2(e) = x2 / (1 +
// 2^-x2); the factor ln(2) is folded into the epilogue's 1/n_scale.
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
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int64_t kT32Range = int64_t(1) << 30;  // |t - base| below this: 32-bit path

template <typename T, int DQK, int DV>
struct Tile {
  static constexpr bool kBf16 = std::is_same<T, __bf16>::value;
  static constexpr int kEpc = 16 / (int)sizeof(T);             // elements per 16 B
  static constexpr int kStep = kBf16 ? 16 : 2;                  // MFMA contraction depth
  static constexpr int kKPitch = DQK + (kBf16 ? 8 : 4);         // padded K rows
  static constexpr int kVPitch = kBf16 ? DV : DV + 4;           // bf16 V rows: XOR-swizzled
  static constexpr int kVChunks = DV * (int)sizeof(T) / 16;     // 16-byte chunks per V row
  // Swizzle of 16-byte chunks in a bf16 V row, chosen so that the transposed
  // reads of one lane half (4 rows x 4 chunks) hit every LDS bank once.
  __device__ static int vswz(int row) {
    return kVChunks >= 16 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
  }
};

template <typename T, int DQK, int DV>
struct Smem {
  using TL = Tile<T, DQK, DV>;
  T k[kBN][TL::kKPitch];
  T v[kBN][TL::kVPitch];
  int64_t tj64[kBN];
  uint32_t tj32[kBN];
  int tbad;
  float trev[32];   // trev[z] = log2e * time[min(31 - z, Tt - 1)], z = clz(1 + |dt|)
  float tful[64];   // tful[b] = log2e * time[min(b, Tt - 1)]
};

__device__ inline uint32_t abs_diff_u32(uint32_t a, uint32_t b) { return a > b ? a - b : b - a; }

// Register r of a 32x32 accumulator (lane half hh) holds row 8(r/4) + 4hh + r%4.
__device__ constexpr int acc_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

template <typename T, int DQK, int DV, bool POS, bool TIME>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void
hstu_attn_fwd_kernel(AttnArgs a) {
  using TL = Tile<T, DQK, DV>;
  using SM = Smem<T, DQK, DV>;
  constexpr bool BF = TL::kBf16;
  constexpr int EPC = TL::kEpc;
  constexpr int NKC = DQK / TL::kStep;             // MFMA steps of S^T
  constexpr int NDB = (DV + 31) / 32;              // 32-wide d_v blocks of O^T
  constexpr int KCH = kBN * DQK / EPC;             // 16-byte chunks per K tile
  constexpr int VCH = kBN * DV / EPC;
  constexpr int KPT = (KCH + kThreads - 1) / kThreads;
  constexpr int VPT = (VCH + kThreads - 1) / kThreads;
  static_assert(DQK % TL::kStep == 0 && DQK % EPC == 0 && DV % EPC == 0, "shape");
  static_assert(!BF || DV % 32 == 0, "bf16 needs d_v multiple of 32");

  __shared__ __align__(16) SM sm;
  extern __shared__ float pos_s[];   // log2e * pos_table[0 .. n_pos)

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
  const int P = a.pos_len;

  // ---- per-lane query row ------------------------------------------------
  const int wr0 = i0 + wave * 32;
  const int i = wr0 + l32;
  const bool row_valid = i < i1;
  const bool wave_rows = wr0 < i1;
  const RowBounds rb = row_valid ? row_bounds(g, i) : RowBounds{kEmptyLo, 0, -1};

  int64_t tbase = 0, ti64 = 0;
  uint32_t ti32 = uint32_t(kT32Range);
  bool row_t_ok = true;
  if constexpr (TIME) {
    tbase = a.timestamps[seq0 + i0];
    ti64 = row_valid ? a.timestamps[seq0 + i] : tbase;
    const int64_t rel = ti64 - tbase;
    row_t_ok = rel > -kT32Range && rel < kT32Range;
    ti32 = row_t_ok ? uint32_t(rel + kT32Range) : 0u;
  }

  // ---- bias tables into LDS (in log2 units) ------------------------------
  if constexpr (POS) {
    const int maxrel = max(i0 + kBM - 1 - kt_lo * kBN, kt_hi * kBN + kBN - 1 - i0);
    const int n_pos = min(P, maxrel + 1);
    for (int x = tid; x < n_pos; x += kThreads) pos_s[x] = kLog2e * a.pos_table[x];
  }
  if constexpr (TIME) {
    const int Tt = a.time_len;
    if (tid < 32) sm.trev[tid] = kLog2e * a.time_table[min(31 - tid, Tt - 1)];
    if (tid < 64) sm.tful[tid] = kLog2e * a.time_table[min(tid, Tt - 1)];
  }

  // ---- Q operand (B operand of S^T = K Q^T), kept in registers ----------
  const T* qrow = reinterpret_cast<const T*>(a.q) +
                  (int64_t)(seq0 + (row_valid ? i : i0)) * a.ld_q + (int64_t)h * DQK;
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
    if constexpr (TIME) {
      if (tid < kBN) {
        const int j = j0 + tid;
        treg = j < L ? a.timestamps[seq0 + j] : tbase;
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int s = 0; s < KPT; ++s) {
      const int c = tid + s * kThreads;
      const int row = c / (DQK / EPC), col = (c % (DQK / EPC)) * EPC;
      if (c < KCH) *reinterpret_cast<uint4*>(&sm.k[row][col]) = kreg[s];
    }
#pragma unroll
    for (int s = 0; s < VPT; ++s) {
      const int c = tid + s * kThreads;
      const int row = c / (DV / EPC), chunk = c % (DV / EPC);
      if (c < VCH) {
        if constexpr (BF) {
          const int pch = chunk ^ TL::vswz(row);
          *reinterpret_cast<uint4*>(&sm.v[row][pch * EPC]) = vreg[s];
        } else {
          *reinterpret_cast<uint4*>(&sm.v[row][chunk * EPC]) = vreg[s];
        }
      }
    }
    if constexpr (TIME) {
      if (tid < kBN) {
        const int64_t rel = treg - tbase;
        const bool ok = rel > -kT32Range && rel < kT32Range;
        sm.tj64[tid] = treg;
        sm.tj32[tid] = ok ? uint32_t(rel + kT32Range) : 0u;
        const uint64_t bad = __ballot(!ok);   // the 64 staging lanes are wave 0
        if (tid == 0) sm.tbad = bad != 0;
      }
    }
  };

  floatx16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

  load_tile(kt_lo);
  store_tile();
  __syncthreads();

  const float alpha2 = a.alpha * kLog2e;

  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    if (kt < kt_hi) load_tile(kt + 1);

#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int jb = kt * kBN + sb * 32;
      const bool lane_any = row_valid && ((rb.lo <= jb + 31 && rb.lo + rb.span >= jb) ||
                                          (rb.self_j >= jb && rb.self_j <= jb + 31));
      const bool lane_full = !row_valid || (rb.lo <= jb && rb.lo + rb.span >= jb + 31);
      if (!(wave_rows && __any(lane_any))) continue;
      const bool full = __all(lane_full);

      // S^T[j][i] for the 32 keys of this block and the wave's 32 rows.
      floatx16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.0f;
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
        if constexpr (BF) {
          const bf16x8 kop =
              *reinterpret_cast<const bf16x8*>(&sm.k[sb * 32 + l32][c * 16 + hh * 8]);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qf[c], s, 0, 0, 0);
        } else {
          const float kop = sm.k[sb * 32 + l32][c * 2 + hh];
          s = __builtin_amdgcn_mfma_f32_32x32x2f32(kop, qf[c], s, 0, 0, 0);
        }
      }

      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = alpha2 * s[r];

      if constexpr (POS) {
        // Direct addressing when every (i, j) of the block has 0 <= i-j < P-1.
        const bool direct = (wr0 - (jb + 31) >= 0) && (wr0 + 31 - jb < P - 1);
        if (direct) {
          const float* pb = pos_s + (i - jb - 4 * hh - 27);   // >= 0 since wr0 >= jb + 31
#pragma unroll
          for (int r = 0; r < 16; ++r) x[r] += pb[27 - (8 * (r >> 2) + (r & 3))];
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = jb + acc_row(r, hh);
            x[r] += pos_s[min(max(i - j, j - i), P - 1)];
          }
        }
      }
      if constexpr (TIME) {
        const bool t_fast = !sm.tbad && __all(row_t_ok);
        if (t_fast) {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const uint4 t4 = *reinterpret_cast<const uint4*>(&sm.tj32[sb * 32 + 8 * gq + 4 * hh]);
            const uint32_t tv[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              x[4 * gq + e] += sm.trev[__builtin_clz(abs_diff_u32(ti32, tv[e]) + 1u)];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t tj = sm.tj64[sb * 32 + acc_row(r, hh)];
            const uint64_t dt = ti64 >= tj ? uint64_t(ti64) - uint64_t(tj)
                                           : uint64_t(tj) - uint64_t(ti64);
            x[r] += sm.tful[63 - __builtin_clzll(dt + 1u)];
          }
        }
      }

      // SiLU(x) * log2(e) = x2 / (1 + 2^-x2)
      float av[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        av[r] = x[r] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x[r]));
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = jb + acc_row(r, hh);
          const bool ok = (uint32_t)(j - rb.lo) <= (uint32_t)rb.span || j == rb.self_j;
          av[r] = ok ? av[r] : 0.0f;
        }
      }

      // O^T[d][i] += sum_j V[j][d] * A[i][j]
      if constexpr (BF) {
        bf16x8 pa[2];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pa[0][e] = (__bf16)av[e];
          pa[1][e] = (__bf16)av[8 + e];
        }
        // ds_read_b64_tr_b16: in each 16-lane group, lane 4e+q loads 4 values of
        // key row e at columns 4q..4q+3 of the group's 16 columns; lane c of the
        // group receives column c of the 4 rows.
        const int gl = lane & 15, grp = lane >> 4;
        const int er = gl >> 2, q4 = gl & 3;
        const char* vb = reinterpret_cast<const char*>(&sm.v[0][0]);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int col = 32 * db + 16 * (grp & 1) + 4 * q4;   // element column
#pragma unroll
          for (int ins = 0; ins < 2; ++ins) {
            shortx4 part[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const int row = sb * 32 + 16 * ins + 8 * half + 4 * hh + er;
              const int pch = (col >> 3) ^ TL::vswz(row);
              const int off = row * (DV * 2) + pch * 16 + (col & 7) * 2;
              part[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_shortx4*)(vb + off));
            }
            const shortx4 lo = part[0], hi = part[1];
            const bf16x8 vop = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pa[ins], acc[db], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = 32 * db + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float vop = d < DV ? sm.v[sb * 32 + acc_row(r, hh)][d] : 0.0f;
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vop, av[r], acc[db], 0, 0, 0);
          }
        }
      }
    }

    if (kt < kt_hi) {
      __syncthreads();   // every wave is done with the tile in LDS
      store_tile();
      __syncthreads();
    }
  }

  // ---- epilogue: ln(2)/n_scale, LayerNorm over d_v, * U, store ------------
  // acc[db][r] holds d = 32db + 8(r/4) + 4hh + r%4 of row i.
  const float osc = a.out_scale;
  float mean = 0.0f, rstd = 1.0f;
  const bool ln = a.epilogue == 0;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] *= osc;
  if (ln) {
    float sum = 0.0f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * db + acc_row(r, hh) < DV) sum += acc[db][r];
    sum += __shfl_xor(sum, 32, 64);
    mean = sum * (1.0f / DV);
    float sq = 0.0f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float c = acc[db][r] - mean;
        if (32 * db + acc_row(r, hh) < DV) sq += c * c;
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
          for (int e = 0; e < 4; ++e) y[e] = acc[db][4 * gq + e];
          if (ln) {
            if constexpr (BF) {
              const bf16x4 uu = *reinterpret_cast<const bf16x4*>(urow + d0);
#pragma unroll
              for (int e = 0; e < 4; ++e) y[e] = (y[e] - mean) * rstd * (float)uu[e];
            } else {
              const floatx4 uu = *reinterpret_cast<const floatx4*>(urow + d0);
#pragma unroll
              for (int e = 0; e < 4; ++e) y[e] = (y[e] - mean) * rstd * uu[e];
            }
          }
          if constexpr (BF) {
            bf16x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (__bf16)y[e];
            *reinterpret_cast<bf16x4*>(orow + d0) = o;
          } else {
            floatx4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = y[e];
            *reinterpret_cast<floatx4*>(orow + d0) = o;
          }
        }
      }
  }
}

template <typename T, int DQK, int DV, bool POS, bool TIME>
static hipError_t launch_one(const AttnArgs& a, int64_t grid, hipStream_t stream) {
  auto kern = hstu_attn_fwd_kernel<T, DQK, DV, POS, TIME>;
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

template <typename T, int DQK, int DV>
static hipError_t launch_bias(const AttnArgs& a, int64_t grid, hipStream_t stream) {
  const bool pos = a.pos_len > 0, tim = a.time_len > 0;
  if (pos && tim) return launch_one<T, DQK, DV, true, true>(a, grid, stream);
  if (pos) return launch_one<T, DQK, DV, true, false>(a, grid, stream);
  if (tim) return launch_one<T, DQK, DV, false, true>(a, grid, stream);
  return launch_one<T, DQK, DV, false, false>(a, grid, stream);
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
    if (d_qk == 128 && d_v == 128) return launch_bias<__bf16, 128, 128>(a, grid, stream);
    if (d_qk == 64 && d_v == 64) return launch_bias<__bf16, 64, 64>(a, grid, stream);
  } else if (dtype == 0) {
    if (d_qk == 128 && d_v == 128) return launch_bias<float, 128, 128>(a, grid, stream);
    if (d_qk == 64 && d_v == 64) return launch_bias<float, 64, 64>(a, grid, stream);
    if (d_qk == 8 && d_v == 8) return launch_bias<float, 8, 8>(a, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace hstu
