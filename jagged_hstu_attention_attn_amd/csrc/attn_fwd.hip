// attn_fwd.hip -- gfx950 (CDNA4) jagged HSTU attention forward.
//
// A persistent launch: every workgroup (4 waves) repeatedly takes a
// (sequence, head, 128-row query tile) item from its XCD's queue (see
// plan.hip); the workgroups of one queue share it cyclically.  Wave w owns
// query rows i0+32w .. i0+32w+31 of an item; lane (l % 32) owns one query row
// and the lane half (l / 32) splits the contraction dimension, which is the
// operand layout of the 32x32 MFMA.
//
// Keys are staged 32 at a time in three LDS buffers: the stage two ahead is
// copied from HBM straight into LDS (global_load_lds_dwordx4, no registers)
// while the current one is computed, one barrier per stage.  Each stage:
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
// Work per 32x32 block is decided per wave from uniform bounds: blocks no
// row of the wave may see are skipped, blocks every row sees fully skip the
// mask, blocks wholly below the diagonal read the position bias at constant
// offsets, and blocks whose (row, key) time gaps all fall in one bucket add
// one constant instead of looking the time bias up per element.
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
  static constexpr int kKChunks = DQK / kEpc;                   // 16-byte chunks per K row
  static constexpr int kVChunks = DV / kEpc;                    // 16-byte chunks per V row
  // XOR swizzles of the 16-byte chunks of a bf16 row (fp32 rows are plain).
  // K: the 16 lanes of a ds_read_b128 read one logical chunk of 16 consecutive
  // rows; the swizzle spreads them over all banks.  V: the transposed reads of
  // one lane half (4 rows x 4 chunks) hit every bank once.
  __device__ static int kswz(int row) {
    if constexpr (!kBf16) return 0;
    return kKChunks >= 16 ? (row & 15) : ((row >> 1) & (kKChunks - 1));
  }
  __device__ static int vswz(int row) {
    if constexpr (!kBf16) return 0;
    return kVChunks >= 16 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
  }
};

constexpr int kStages = 3;   // LDS buffers of the key/value pipeline

// One stage of the pipeline.  Each stage buffer is its own __shared__ object,
// so the compiler can tell that an LDS copy into one stage does not alias
// reads of another (and does not make those reads wait for the copy).
template <typename T, int DQK, int DV>
struct StageBuf {
  T k[kBN][DQK];
  T v[kBN][DV];
  int64_t tj64[kBN];
  uint32_t tj32[kBN];
  uint32_t tjmin, tjmax;   // 32-bit key times of the stage (valid keys)
  int tbad;                // some key needs the 64-bit time path
};

struct TimeTables {
  float trev[32];   // trev[z] = log2e * time[min(31 - z, Tt - 1)], z = clz(1 + |dt|)
  float tful[64];   // tful[b] = log2e * time[min(b, Tt - 1)]
};

typedef __attribute__((address_space(3))) void lds_void;

// LDS byte offset of a __shared__ address.
__device__ inline uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}

// HBM -> LDS copies (global_load_lds): lane l's bytes land at LDS offset
// `lds` + size*l.  Issued from inline assembly on purpose: the compiler then
// neither waits for them before unrelated LDS reads nor folds them into its
// own vmcnt accounting; every wait on them is an explicit wait_vmem below.
// They write no registers.  M0 is a reserved register, so clobbering it is
// harmless; the warning about it is silenced here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// `lds` must be the same for every lane of the wave.
__device__ inline void lds_copy16(const void* g, uint32_t lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m), "v"(g) : "memory", "m0");
}
__device__ inline void lds_copy4(const void* g, uint32_t lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(m), "v"(g) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N): all but the N most recent global loads / LDS copies of
// this wave are done (they complete in order).
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the pipeline.  __syncthreads() carries a release
// fence that waits for every outstanding LDS copy, which would drain the
// copies of the stage two ahead; here the caller has already waited for the
// copies that must have landed (vmcnt) and this waits for its own LDS writes
// (lgkmcnt), and the empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ inline void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt untouched
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS copies wave w issues per stage when `count` copies are spread over the
// waves round-robin.
__host__ __device__ constexpr int copies_of_wave(int count, int w) {
  return count > w ? (count - w + kWaves - 1) / kWaves : 0;
}

__device__ inline uint32_t abs_diff_u32(uint32_t a, uint32_t b) { return a > b ? a - b : b - a; }

// Register r of a 32x32 accumulator (lane half hh) holds row 8(r/4) + 4hh + r%4.
__device__ constexpr int acc_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

template <typename V>
__device__ inline V wave_min(V v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) { const V w = __shfl_xor(v, o, 64); v = w < v ? w : v; }
  return v;
}
template <typename V>
__device__ inline V wave_max(V v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) { const V w = __shfl_xor(v, o, 64); v = w > v ? w : v; }
  return v;
}
__device__ inline int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <typename T, int DQK, int DV, bool POS, bool TIME>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void
hstu_attn_fwd_kernel(AttnArgs a) {
  using TL = Tile<T, DQK, DV>;
  using SB = StageBuf<T, DQK, DV>;
  constexpr bool BF = TL::kBf16;
  constexpr int EPC = TL::kEpc;
  constexpr int NKC = DQK / TL::kStep;             // MFMA steps of S^T
  constexpr int NDB = (DV + 31) / 32;              // 32-wide d_v blocks of O^T
  constexpr int KCPR = TL::kKChunks;               // 16-byte chunks per K row
  constexpr int VCPR = TL::kVChunks;
  constexpr int KRPI = 64 / KCPR;                  // K rows per wave-wide LDS copy
  constexpr int VRPI = 64 / VCPR;
  constexpr int KNI = kBN / KRPI;                  // LDS copies per K stage
  constexpr int VNI = kBN / VRPI;
  static_assert(DQK % TL::kStep == 0 && DQK % EPC == 0 && DV % EPC == 0, "shape");
  static_assert(KCPR <= 64 && VCPR <= 64 && KRPI <= kBN && VRPI <= kBN, "stage shape");
  static_assert(!BF || DV % 32 == 0, "bf16 needs d_v multiple of 32");

  __shared__ __align__(16) SB st0, st1, st2;
  __shared__ TimeTables tt;
  extern __shared__ float pos_s[];   // log2e * pos_table[0 .. n_pos)
  auto stage = [&](auto bufc) -> SB& {
    constexpr int b = decltype(bufc)::value;
    if constexpr (b == 0) return st0;
    else if constexpr (b == 1) return st1;
    else return st2;
  };

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int P = a.pos_len;
  const int H = a.num_heads;

  if constexpr (TIME) {
    // log2(e) * time table, indexed two ways (see TimeTables)
    const int Tt = a.time_len;
    if (tid < 32) tt.trev[tid] = kLog2e * a.time_table[min(31 - tid, Tt - 1)];
    if (tid < 64) tt.tful[tid] = kLog2e * a.time_table[min(tid, Tt - 1)];
  }
  int pos_staged = 0;   // entries of pos_s already staged (uniform)

  // Queue walk: workgroup k serves queue k%8 and takes its entries k/8,
  // k/8 + W, k/8 + 2W, ... where W is the number of workgroups serving that
  // queue (at least 8 workgroups are launched, so every queue is served).
  const int qx = blockIdx.x & (kQueues - 1);
  const int qstride = ((int)gridDim.x + kQueues - 1 - qx) / kQueues;
  const int qcount = a.queue_count[qx];
  const int4* qitems = a.items + a.queue_start[qx];
  for (int idx = blockIdx.x >> 3; idx < qcount; idx += qstride) {
  const int4 it = qitems[idx];
  const int seq0 = it.x, L = it.y;
  const int qt = it.w / H, h = it.w - qt * H;
  SeqGeom g;
  g.L = L;
  g.n_h = it.z;
  g.c = clampi(a.contextual_len, 0, g.n_h);
  g.W = a.max_attn_len;
  const int i0 = qt * kBM;
  const int i1 = min(i0 + kBM, L);
  int jlo, jhi;
  tile_key_range(g, i0, i1, jlo, jhi);
  const int kt_lo = jlo / kBN, kt_hi = jhi / kBN;

  // ---- per-lane query row and the wave's uniform key bounds --------------
  const int wr0 = i0 + wave * 32;
  const int i = wr0 + l32;
  const bool row_valid = i < i1;
  const bool wave_rows = wr0 < i1;
  const RowBounds rb = row_valid ? row_bounds(g, i) : RowBounds{kEmptyLo, 0, -1};
  // some row may see a key of [w_jmin, w_jmax]; every row sees every key of
  // [w_lomax, w_himin].
  int w_jmin, w_jmax, w_lomax, w_himin;
  {
    const bool nonempty = rb.lo != kEmptyLo;
    const int hi = rb.lo + rb.span;
    int jmin = nonempty ? rb.lo : (rb.self_j >= 0 ? rb.self_j : 0x7fffffff);
    int jmax = nonempty ? max(hi, rb.self_j) : rb.self_j;
    if (!row_valid) { jmin = 0x7fffffff; jmax = -1; }
    w_jmin = uni(wave_min(jmin));
    w_jmax = uni(wave_max(jmax));
    w_lomax = uni(wave_max(row_valid ? rb.lo : -1));
    w_himin = uni(wave_min(row_valid ? (nonempty ? hi : -1) : 0x7fffffff));
  }

  // row times (set after the first stage copies are issued)
  int64_t tbase = 0, ti64 = 0;
  uint32_t ti32 = uint32_t(kT32Range);
  bool w_t_ok = true;
  uint32_t w_tmin = 0, w_tmax = 0;
  // Q operand (B operand of S^T = K Q^T), kept in registers
  typename std::conditional<BF, bf16x8, float>::type qf[NKC];

  // ---- K/V stages: HBM -> LDS copies, 32 keys per stage --------------------
  const char* kseq = reinterpret_cast<const char*>(a.k) +
                     ((int64_t)seq0 * a.ld_k + (int64_t)h * DQK) * (int64_t)sizeof(T);
  const char* vseq = reinterpret_cast<const char*>(a.v) +
                     ((int64_t)seq0 * a.ld_v + (int64_t)h * DV) * (int64_t)sizeof(T);

  // Copy key tile kt (keys, values and, with a time bias, the raw int64
  // timestamps) into stage buffer `bufc`.  A wave-wide copy writes 64
  // consecutive 16-byte chunks of LDS (KRPI whole rows); each lane picks the
  // global chunk that belongs at its LDS position under the swizzle.  Rows
  // past the end of the sequence repeat its last row (finite values whose
  // scores are always masked and whose coefficients are therefore 0).
  auto issue_stage = [&](auto bufc, int kt) {
    SB& sb = stage(bufc);
    const int j0 = kt * kBN;
    const bool whole = j0 + kBN <= L;
#pragma unroll
    for (int s2 = 0; s2 < (KNI + kWaves - 1) / kWaves; ++s2) {
      const int n = wave + s2 * kWaves;
      if (n < KNI) {
        const int row = n * KRPI + lane / KCPR;
        const int c = (lane % KCPR) ^ TL::kswz(row);
        const int j = whole ? j0 + row : min(j0 + row, L - 1);
        lds_copy16(kseq + ((int64_t)j * a.ld_k + c * EPC) * (int64_t)sizeof(T),
                   lds_off(&sb.k[n * KRPI][0]));
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < (VNI + kWaves - 1) / kWaves; ++s2) {
      const int n = wave + s2 * kWaves;
      if (n < VNI) {
        const int row = n * VRPI + lane / VCPR;
        const int c = (lane % VCPR) ^ TL::vswz(row);
        const int j = whole ? j0 + row : min(j0 + row, L - 1);
        lds_copy16(vseq + ((int64_t)j * a.ld_v + c * EPC) * (int64_t)sizeof(T),
                   lds_off(&sb.v[n * VRPI][0]));
      }
    }
    if constexpr (TIME) {
      if (wave == 0) {   // 64 lanes x 4 bytes = the 32 int64 timestamps
        const int j = min(j0 + (lane >> 1), L - 1);
        lds_copy4(reinterpret_cast<const int32_t*>(a.timestamps + seq0 + j) + (lane & 1),
                  lds_off(&sb.tj64[0]));
      }
    }
  };

  // Key times of a landed stage (wave 0, lanes 0..31): 32-bit offsets, their
  // range over the valid keys, and whether any key needs the 64-bit path.
  auto finish_stage = [&](auto bufc, int kt) {
    SB& sb = stage(bufc);
    if constexpr (TIME) {
      if (tid < kBN) {
        const int64_t tj = sb.tj64[tid];
        const int64_t rel = tj - tbase;
        const bool ok = rel > -kT32Range && rel < kT32Range;
        const uint32_t t32 = ok ? uint32_t(rel + kT32Range) : 0u;
        const bool key_valid = kt * kBN + tid < L;
        sb.tj32[tid] = t32;
        const uint64_t bad = __ballot(!ok);
        uint32_t mn = key_valid ? t32 : 0xffffffffu, mx = key_valid ? t32 : 0u;
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) {
          const uint32_t a2 = __shfl_xor(mn, o, 64), b2 = __shfl_xor(mx, o, 64);
          mn = a2 < mn ? a2 : mn;
          mx = b2 > mx ? b2 : mx;
        }
        if (tid == 0) {
          sb.tjmin = mn;
          sb.tjmax = mx;
          sb.tbad = bad != 0;
        }
      }
    }
  };

  floatx16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

  const float alpha2 = a.alpha * kLog2e;

  // One 32-key stage from LDS buffer `buf` (compile-time) for this wave's rows.
  auto compute_stage = [&](auto bufc, int kt) {
    SB& sb = stage(bufc);
    const int jb = kt * kBN;
    // uniform block class for this wave
    if (!wave_rows || jb > w_jmax || jb + 31 < w_jmin) return;
    const bool full = w_lomax <= jb && w_himin >= jb + 31;

    // S^T[j][i] for the 32 keys of this block and the wave's 32 rows.
    floatx16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.0f;
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      if constexpr (BF) {
        const bf16x8 kop =
            *reinterpret_cast<const bf16x8*>(&sb.k[l32][((2 * c + hh) ^ TL::kswz(l32)) * 8]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qf[c], s, 0, 0, 0);
      } else {
        const float kop = sb.k[l32][c * 2 + hh];
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kop, qf[c], s, 0, 0, 0);
      }
    }

    // x2 = alpha*log2e*S + log2e*pos
    float x[16];
    if constexpr (POS) {
      // constant offsets when every (i, j) of the block has 0 <= i-j < P-1
      if (wr0 - (jb + 31) >= 0 && wr0 + 31 - jb < P - 1) {
        const float* pb = pos_s + (i - jb - 4 * hh - 27);   // >= 0 since wr0 >= jb + 31
#pragma unroll
        for (int r = 0; r < 16; ++r)
          x[r] = fmaf(s[r], alpha2, pb[27 - (8 * (r >> 2) + (r & 3))]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = jb + acc_row(r, hh);
          x[r] = fmaf(s[r], alpha2, pos_s[min(max(i - j, j - i), P - 1)]);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = s[r] * alpha2;
    }

    // + log2e*time bias
    if constexpr (TIME) {
      if (!sb.tbad && w_t_ok) {
        const uint32_t kmin = sb.tjmin, kmax = sb.tjmax;
        // range of |t_i - t_j| over the block's valid rows and keys
        uint32_t dmin = 0;
        if (w_tmin > kmax) dmin = w_tmin - kmax;
        if (kmin > w_tmax) dmin = kmin - w_tmax;
        const uint32_t dmax = max(w_tmax > kmin ? w_tmax - kmin : 0u,
                                  kmax > w_tmin ? kmax - w_tmin : 0u);
        const int z0 = __builtin_clz(dmin + 1u), z1 = __builtin_clz(dmax + 1u);
        if (z0 == z1) {
          const float tb = tt.trev[z0];
#pragma unroll
          for (int r = 0; r < 16; ++r) x[r] += tb;
        } else {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const uint4 t4 =
                *reinterpret_cast<const uint4*>(&sb.tj32[8 * gq + 4 * hh]);
            const uint32_t tv[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              x[4 * gq + e] += tt.trev[__builtin_clz(abs_diff_u32(ti32, tv[e]) + 1u)];
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t tj = sb.tj64[acc_row(r, hh)];
          const uint64_t dt = ti64 >= tj ? uint64_t(ti64) - uint64_t(tj)
                                         : uint64_t(tj) - uint64_t(ti64);
          x[r] += tt.tful[63 - __builtin_clzll(dt + 1u)];
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
      const char* vb = reinterpret_cast<const char*>(&sb.v[0][0]);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int col = 32 * db + 16 * (grp & 1) + 4 * q4;   // element column
#pragma unroll
        for (int ins = 0; ins < 2; ++ins) {
          shortx4 part[2];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int row = 16 * ins + 8 * half + 4 * hh + er;
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
          const float vop = d < DV ? sb.v[acc_row(r, hh)][d] : 0.0f;
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vop, av[r], acc[db], 0, 0, 0);
        }
      }
    }
  };

  // Three-buffer pipeline, unrolled by three so that buffer indices are
  // compile-time constants: stage kt is computed from buffer B while stage
  // kt+1 (already copied) lands in buffer B+1 and stage kt+2 is copied into
  // buffer B+2.  Before the barrier each wave waits for its own copies of
  // stage kt+1 only -- its copies of stage kt+2 (the most recent) stay in flight.
  auto wait_next = [&](bool ahead) {
    constexpr int c0 = copies_of_wave(KNI, 0) + copies_of_wave(VNI, 0) + (TIME ? 1 : 0);
    constexpr int c1 = copies_of_wave(KNI, 1) + copies_of_wave(VNI, 1);
    constexpr int c2 = copies_of_wave(KNI, 2) + copies_of_wave(VNI, 2);
    constexpr int c3 = copies_of_wave(KNI, 3) + copies_of_wave(VNI, 3);
    if (!ahead) { wait_vmem<0>(); return; }
    if (wave == 0) wait_vmem<c0>();
    else if (wave == 1) wait_vmem<c1>();
    else if (wave == 2) wait_vmem<c2>();
    else wait_vmem<c3>();
  };
  auto step = [&](auto bufc, int kt) {
    constexpr int buf = decltype(bufc)::value;
    using NB1 = std::integral_constant<int, (buf + 1) % kStages>;
    using NB2 = std::integral_constant<int, (buf + 2) % kStages>;
    const bool more1 = kt + 1 <= kt_hi, more2 = kt + 2 <= kt_hi;
    if (more2) issue_stage(NB2{}, kt + 2);
    compute_stage(bufc, kt);
    if (more1) {
      wait_next(more2);
      finish_stage(NB1{}, kt + 1);
      stage_barrier();
    }
  };

  // Item prologue.  The first two stage copies go out first; the loads the
  // compiler tracks itself (row times, position table, Q) come after them, so
  // its own waits for those never hold back copies issued later.
  if constexpr (TIME) tbase = a.timestamps[seq0 + i0];   // finish_stage needs it
  issue_stage(std::integral_constant<int, 0>{}, kt_lo);
  if (kt_lo + 1 <= kt_hi) issue_stage(std::integral_constant<int, 1>{}, kt_lo + 1);

  if constexpr (TIME) {
    ti64 = row_valid ? a.timestamps[seq0 + i] : tbase;
    const int64_t rel = ti64 - tbase;
    const bool ok = rel > -kT32Range && rel < kT32Range;
    ti32 = ok ? uint32_t(rel + kT32Range) : 0u;
    w_t_ok = __all(ok);
    w_tmin = (uint32_t)uni((int)wave_min(row_valid ? ti32 : 0xffffffffu));
    w_tmax = (uint32_t)uni((int)wave_max(row_valid ? ti32 : 0u));
  }
  // position table into LDS (log2 units), grown as items need it
  if constexpr (POS) {
    const int maxrel = max(i0 + kBM - 1 - kt_lo * kBN, kt_hi * kBN + kBN - 1 - i0);
    const int n_pos = min(P, maxrel + 1);
    for (int x = pos_staged + tid; x < n_pos; x += kThreads) pos_s[x] = kLog2e * a.pos_table[x];
    pos_staged = max(pos_staged, n_pos);
  }
  {
    const T* qrow = reinterpret_cast<const T*>(a.q) +
                    (int64_t)(seq0 + (row_valid ? i : i0)) * a.ld_q + (int64_t)h * DQK;
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      if constexpr (BF) {
        bf16x8 z = {};
        qf[c] = row_valid ? *reinterpret_cast<const bf16x8*>(qrow + c * 16 + hh * 8) : z;
      } else {
        qf[c] = row_valid ? qrow[c * 2 + hh] : 0.0f;
      }
    }
  }
  // The compiler waits for the Q loads here (in the prologue, where every
  // copy is in flight anyway); afterwards the empty asm makes the registers
  // plain values, so no wait on them is placed inside the stage loop, where it
  // would also drain the copies of the stage two ahead.
#pragma unroll
  for (int c = 0; c < NKC; ++c) asm volatile("" : "+v"(qf[c]));
  wait_next(kt_lo + 1 <= kt_hi);
  finish_stage(std::integral_constant<int, 0>{}, kt_lo);
  stage_barrier();   // also publishes the bias tables
  for (int kt = kt_lo;; kt += kStages) {
    step(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 > kt_hi) break;
    step(std::integral_constant<int, 1>{}, kt + 1);
    if (kt + 2 > kt_hi) break;
    step(std::integral_constant<int, 2>{}, kt + 2);
    if (kt + 3 > kt_hi) break;
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

  __syncthreads();   // the LDS of this item is free again
  }  // queue walk
}

template <typename T, int DQK, int DV, bool POS, bool TIME>
static hipError_t launch_one(const AttnArgs& a, int n_wg, hipStream_t stream) {
  auto kern = hstu_attn_fwd_kernel<T, DQK, DV, POS, TIME>;
  const size_t dyn = (size_t)(a.pos_len > 0 ? a.pos_len : 1) * sizeof(float);
  hipLaunchKernelGGL(kern, dim3((unsigned)n_wg), dim3(kThreads), dyn, stream, a);
  return hipGetLastError();
}

// Resident workgroups per CU for one instantiation and dynamic LDS size.
template <typename T, int DQK, int DV, bool POS, bool TIME>
static int blocks_per_cu(int pos_len) {
  auto kern = hstu_attn_fwd_kernel<T, DQK, DV, POS, TIME>;
  static bool attr_done = false;
  if (!attr_done) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            kPosMax * (int)sizeof(float)) != hipSuccess)
      return -1;
    attr_done = true;
  }
  const size_t dyn = (size_t)(pos_len > 0 ? pos_len : 1) * sizeof(float);
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, kThreads, dyn) != hipSuccess)
    return -1;
  return nb;
}

template <typename T, int DQK, int DV>
static hipError_t launch_bias(const AttnArgs& a, int n_wg, hipStream_t stream) {
  const bool pos = a.pos_len > 0, tim = a.time_len > 0;
  if (pos && tim) return launch_one<T, DQK, DV, true, true>(a, n_wg, stream);
  if (pos) return launch_one<T, DQK, DV, true, false>(a, n_wg, stream);
  if (tim) return launch_one<T, DQK, DV, false, true>(a, n_wg, stream);
  return launch_one<T, DQK, DV, false, false>(a, n_wg, stream);
}

template <typename T, int DQK, int DV>
static int bpc_bias(int pos_len, int time_len) {
  const bool pos = pos_len > 0, tim = time_len > 0;
  if (pos && tim) return blocks_per_cu<T, DQK, DV, true, true>(pos_len);
  if (pos) return blocks_per_cu<T, DQK, DV, true, false>(pos_len);
  if (tim) return blocks_per_cu<T, DQK, DV, false, true>(pos_len);
  return blocks_per_cu<T, DQK, DV, false, false>(pos_len);
}

int attn_grid(int dtype, int d_qk, int d_v, int pos_len, int time_len) {
  int bpc = -1;
  if (dtype == 1) {
    if (d_qk == 128 && d_v == 128) bpc = bpc_bias<__bf16, 128, 128>(pos_len, time_len);
    if (d_qk == 64 && d_v == 64) bpc = bpc_bias<__bf16, 64, 64>(pos_len, time_len);
  } else if (dtype == 0) {
    if (d_qk == 128 && d_v == 128) bpc = bpc_bias<float, 128, 128>(pos_len, time_len);
    if (d_qk == 64 && d_v == 64) bpc = bpc_bias<float, 64, 64>(pos_len, time_len);
    if (d_qk == 8 && d_v == 8) bpc = bpc_bias<float, 8, 8>(pos_len, time_len);
  }
  if (bpc <= 0) return -1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  return cus * bpc;
}

bool attn_supported(int dtype, int d_qk, int d_v) {
  if (dtype == 1) return (d_qk == 128 && d_v == 128) || (d_qk == 64 && d_v == 64);
  if (dtype == 0) return (d_qk == 128 && d_v == 128) || (d_qk == 64 && d_v == 64) ||
                         (d_qk == 8 && d_v == 8);
  return false;
}

hipError_t launch_attn(const AttnArgs& a, int dtype, int d_qk, int d_v, int n_wg,
                       hipStream_t stream) {
  if (dtype == 1) {
    if (d_qk == 128 && d_v == 128) return launch_bias<__bf16, 128, 128>(a, n_wg, stream);
    if (d_qk == 64 && d_v == 64) return launch_bias<__bf16, 64, 64>(a, n_wg, stream);
  } else if (dtype == 0) {
    if (d_qk == 128 && d_v == 128) return launch_bias<float, 128, 128>(a, n_wg, stream);
    if (d_qk == 64 && d_v == 64) return launch_bias<float, 64, 64>(a, n_wg, stream);
    if (d_qk == 8 && d_v == 8) return launch_bias<float, 8, 8>(a, n_wg, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace hstu
