// attn_fwd.hip -- gfx950 (CDNA4) jagged HSTU attention forward.
//
// A persistent launch: every workgroup (4 waves) repeatedly takes a
// (sequence, head, 128-row query tile) unit from the scheduler's plan (see
// plan.hip): its own list of units, or a work queue it shares.  Wave w owns
// query rows i0+32w .. i0+32w+31 of an item; lane (l % 32) owns one query row
// and the lane half (l / 32) splits the contraction dimension, which is the
// operand layout of the 32x32 MFMA (v_mfma_f32_32x32x16_bf16; 32x32x2 for
// fp32).  Two workgroups share a CU, so each SIMD runs two waves of different
// workgroups whose matrix-core and vector-ALU phases overlap.
//
// Keys are staged 32 at a time in four LDS buffers, copied from HBM straight
// into LDS (global_load_lds, no registers) three stages ahead, one barrier per
// stage.  Per 32-key block and wave:
//   S^T = K Q^T + C              32x32, bf16 MFMA with fp32 accumulation; the
//                                accumulator starts at the position bias
//   x   = alpha*S + time[bucket(|t_i - t_j|)]     (one FMA per score)
//   a   = allowed(i,j) ? SiLU(x) : 0     a select, never a multiply by a mask
//   O^T += V^T A^T               the SiLU values go from the first MFMA's
//                                accumulator registers straight into the
//                                second MFMA's B operand
// and the epilogue scales by 1/n_scale, takes LayerNorm over d_v per (token,
// head) (the two lane halves of a row combine with one cross-lane exchange),
// multiplies by U and stores the rows that belong to the sequence.  All LDS
// reads of a block are issued before its arithmetic, so their latency hides
// behind the score MFMAs and the SiLU.
//
// Computing S^T (keys on the MFMA's M side, queries on N) puts every query
// row's scores in one lane, so the accumulators already have the B-operand
// layout of the aggregation MFMA (the order of the contraction index inside
// one MFMA is free as long as both operands agree).  V stays row-major in LDS
// and its transposed operand comes from ds_read_b64_tr_b16.  The 16-byte
// chunks of each staged K and V row are XOR-swizzled so that the rows one LDS
// cycle reads fall on distinct banks.
//
// Scores are kept in log2 units.  The position bias of a 128 x 32 block takes
// only 159 distinct values, one per i - j.  Each stage gathers them from the
// table into LDS (every lane of the copy reads the entry of its own clamped
// |i - j|), rescales them once, and every score's accumulator starts from its
// value: C = log2(e) pos / am and x2 = am S + log2(e) time = log2(e) x, with
// am = alpha log2(e) (am = 1 and Q = 0 when alpha is 0).  SiLU(x) log2(e) =
// x2 / (1 + 2^-x2); the factor ln(2) is folded into the epilogue's 1/n_scale.
//
// Work per block is decided per wave from uniform bounds: blocks no row of
// the wave may see are skipped, blocks every row sees fully skip the mask, and
// blocks whose (row, key) time gaps all fall in one bucket add one constant
// instead of looking the time bias up per score.
//
// Method: pointwise SiLU aggregation with position/time bias, zeroing after
// the nonlinearity, Norm then U gating ("HSTU tensor by tensor: SiLU
// aggregation, temporal bias and gating", sections "SiLU aggregation
// coefficients are not probabilities", "Do not copy softmax masking
// mechanically", "Relative time adds information content similarity lacks",
// "Similar shape, different aggregation").
#include <type_traits>

#include <hip/hip_ext.h>

#include "attn_common.hpp"

namespace hstu {

constexpr int kStages = 4;                       // LDS buffers of the key/value pipeline
constexpr int kRows = kBM / kWaves;              // query rows per wave
static_assert(kRows == 32, "one 32x32 MFMA tile of query rows per wave");
static_assert(kBN == 32, "a key block is one 32-key score tile");

// One stage of the pipeline.  Each stage buffer is its own __shared__ object,
// so the compiler can tell that the accesses of different stages never alias.
template <typename T, int DQK, int DV, bool CLAMP>
struct StageBuf {
  using C = Cfg<T, DQK, DV>;
  char k[kBN * C::kKRow];        // keys: row j at byte j * kKRow, chunks swizzled
  char v[kBN * C::kVRow];        // values
  float diag[kDiagCopies * 64];  // position bias of i - j = i0 - j0 + 127 - f, at f
  int64_t ts64[kBN];             // raw key timestamps
  uint32_t ts32[kBN];            // key timestamps relative to the item's base
  uint32_t tmin, tmax;           // range of ts32 over the valid keys
  int tbad;                      // some key needs the 64-bit time path
  int pad_;
  float cpos[CLAMP ? 64 : 1];    // clamped-position bias of key (lane % 32): n_h - j
};

// Copies wave w issues per stage when copy n goes to wave n % kWaves.
__host__ __device__ constexpr int copies_of_wave(int count, int w) {
  return count > w ? (count - w + kWaves - 1) / kWaves : 0;
}
// Position-bias copy p goes to wave kWaves-1-p, the timestamp copy to the
// wave below those.
constexpr int kTsWave = kWaves - 1 - kDiagCopies;
static_assert(kTsWave >= 0, "enough waves for the bias copies");
// All LDS copies wave w issues per stage.
template <int NK, int NV, bool POS, bool TIME>
__host__ __device__ constexpr int stage_copies(int w) {
  return copies_of_wave(NK, w) + copies_of_wave(NV, w) +
         ((POS && w > kTsWave) ? 1 : 0) + ((TIME && w == kTsWave) ? 1 : 0);
}

// Waves per SIMD the kernel is built for: two workgroups per CU (a wave has
// 256 registers) up to d = 128; with d = 256 the 32 x 256 fp32 output tile
// alone takes 128 registers and the Q operands 64, so one workgroup per CU
// (512 registers a wave, four 33 KB stage buffers of LDS).
template <int DQK, int DV>
constexpr int kWavesPerSimd = (DQK > 128 || DV > 128) ? 1 : 2;

// POSM: 0 = no position bias, 1 = position bias of |i - j|, 2 = of the
// clamped positions |p_i - p_j| (candidate rows take it from cpos).
template <typename T, int DQK, int DV, int POSM, bool TIME>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<DQK, DV>))) void
hstu_attn_fwd_kernel(AttnArgs a) {
  constexpr bool POS = POSM != 0;
  constexpr bool clamp = POSM == 2;
  using C = Cfg<T, DQK, DV>;
  using SB = StageBuf<T, DQK, DV, clamp>;
  constexpr bool BF = C::kBf16;
  constexpr int ES = C::kEs;
  constexpr int NKC = C::kNKC;
  constexpr int NDB = C::kNDB;
  constexpr int KROW = C::kKRow, VROW = C::kVRow;
  constexpr int KCH = C::kKCh, VCH = C::kVCh;
  constexpr int NK = C::kNK, NV = C::kNV;
  constexpr int SK = (NK + kWaves - 1) / kWaves;   // K copies per wave (at most)
  constexpr int SV = (NV + kWaves - 1) / kWaves;
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  using B3 = std::integral_constant<int, 3>;

  __shared__ __align__(16) SB st0, st1, st2, st3;
  __shared__ TimeTables tt;
  __shared__ int s_ticket;   // arrival order of a split item's chunk
  auto stage = [&](auto bufc) __attribute__((always_inline)) -> SB& {
    constexpr int b = decltype(bufc)::value % kStages;
    if constexpr (b == 0) return st0;
    else if constexpr (b == 1) return st1;
    else if constexpr (b == 2) return st2;
    else return st3;
  };

  const int tid = threadIdx.x;
  // the wave index is the same in every lane: keep it in a scalar register so
  // that everything derived from it (rows, copy schedule, bounds) is uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int P = a.pos_len;
  const int H = a.num_heads;
  const float alpha2 = a.alpha * kLog2e;
  const bool alpha_zero = alpha2 == 0.0f;
  const float am = alpha_zero ? 1.0f : alpha2;   // x2 = am * S + time
  const float pscale = kLog2e / am;              // position bias in accumulator units
  const uint32_t ldk_b = (uint32_t)(a.ld_k * ES), ldv_b = (uint32_t)(a.ld_v * ES);
  const int my_copies = stage_copies<NK, NV, POS, TIME>(wave) + ((clamp && wave == kTsWave) ? 1 : 0);

  if constexpr (TIME) {
    // log2(e) * time table, indexed two ways (see TimeTables)
    const int Tt = a.time_len;
    if (tid < 32) tt.trev[tid] = kLog2e * a.time_table[min(31 - tid, Tt - 1)];
    if (tid < 64) tt.tful[tid] = kLog2e * a.time_table[min(tid, Tt - 1)];
  }

  // Lane l of K copy n fills LDS chunk m = 64n + l: row m / KCH, physical
  // chunk m % KCH, which holds the row's logical chunk (m % KCH) ^ kswz(row).
  // Byte offsets of those chunks from the stage's first row:
  uint32_t k_off[SK], v_off[SV];
#pragma unroll
  for (int s = 0; s < SK; ++s) {
    const int m = 64 * (s * kWaves + wave) + lane, row = m / KCH;
    k_off[s] = (uint32_t)row * ldk_b + 16u * (uint32_t)((m % KCH) ^ C::kswz(row));
  }
#pragma unroll
  for (int s = 0; s < SV; ++s) {
    const int m = 64 * (s * kWaves + wave) + lane, row = m / VCH;
    v_off[s] = (uint32_t)row * ldv_b + 16u * (uint32_t)((m % VCH) ^ C::vswz(row));
  }

  // Work walk.  Static plan: planned workgroup v processes units [wg[2v],
  // wg[2v] + wg[2v+1]) in order; a launch of another size than the plan's
  // maps the planned workgroups onto its own cyclically.  Queue modes (hdr[2]
  // set; one queue, or one per XCD): the workgroup starts with unit
  // first + w of its queue (work_queue), and during every item it fetches
  // its next unit, first + n plus the queue counter's previous value,
  // through s_qnext (two slots by item parity, so a slot is rewritten only
  // after every wave has passed the barriers of the item that read it).
  // Indices only grow, so every workgroup stops once its next unit is past
  // its queue's last.
  __shared__ int s_qnext[2];
  const bool queue = a.hdr[2] != kPlanStatic;
  const WorkQueue wkq = work_queue(a.hdr);
  const int n_plan = queue ? (int)gridDim.x : a.hdr[0];
  int q_item = 0;   // items this workgroup has started (queue slot parity)
  for (int v = blockIdx.x; v < n_plan; v += gridDim.x) {
  const int u_begin = queue ? wkq.first + wkq.w : a.wg[2 * v];
  const int u_end = queue ? wkq.end : u_begin + a.wg[2 * v + 1];
  for (int u = u_begin; u < u_end; u = queue ? s_qnext[(q_item++) & 1] : u + 1) {
  const int4 it = a.units[2 * u];
  const int4 ch = a.units[2 * u + 1];   // key tiles [ch.x, ch.y]; split slot, chunk
  const int seq0 = it.x, L = it.y;
  const int qt = it.w / H, h = it.w - qt * H;
  SeqGeom geo;
  geo.L = L;
  geo.n_h = it.z;
  geo.c = clampi(a.contextual_len, 0, geo.n_h);
  geo.W = a.max_attn_len;
  const int i0 = ((ch.w & kUnitCandRows) ? geo.n_h : 0) + qt * kBM;
  const int i1 = min(i0 + kBM, L);
  int jlo, jhi;
  tile_key_range(geo, i0, i1, jlo, jhi);
  const int kt_lo = max(jlo / kBN, ch.x), kt_hi = min(jhi / kBN, ch.y);

  // ---- per-lane query row and the wave's uniform key bounds --------------
  const int wr0 = i0 + wave * kRows;
  const int i = wr0 + l32;
  const bool row_valid = i < i1;
  const bool wave_rows = wr0 < i1;
  // some row may see a key of [w_jmin, w_jmax]; every row sees every key of
  // [w_lomax, w_himin].
  int w_jmin, w_jmax, w_lomax, w_himin;
  {
    const RowBounds rb = row_valid ? row_bounds(geo, i) : RowBounds{kEmptyLo, 0, -1};
    const bool nonempty = rb.lo != kEmptyLo;
    const int hi = rb.lo + rb.span;
    int jmin = nonempty ? rb.lo : (rb.self_j >= 0 ? rb.self_j : 0x7fffffff);
    int jmax = nonempty ? max(hi, rb.self_j) : rb.self_j;
    if (!row_valid) { jmin = 0x7fffffff; jmax = -1; }
    w_jmin = wave_min(jmin);
    w_jmax = wave_max(jmax);
    w_lomax = wave_max(row_valid ? rb.lo : -1);
    w_himin = wave_min(row_valid ? (nonempty ? hi : -1) : 0x7fffffff);
  }
  // some row of this wave is a candidate whose bias uses clamped positions
  const bool w_cand = clamp && wave_rows && wr0 + kRows - 1 >= geo.n_h;
  (void)w_cand;
  auto needs = [&](int kt) __attribute__((always_inline)) {
    const int jb = kt * kBN;
    return wave_rows && jb <= w_jmax && jb + kBN - 1 >= w_jmin;
  };
  auto is_full = [&](int kt) __attribute__((always_inline)) {
    const int jb = kt * kBN;
    return w_lomax <= jb && w_himin >= jb + kBN - 1;
  };

  const uint64_t kseq = uni_ptr(reinterpret_cast<const char*>(a.k) +
                                ((int64_t)seq0 * a.ld_k + (int64_t)h * DQK) * ES);
  const uint64_t vseq = uni_ptr(reinterpret_cast<const char*>(a.v) +
                                ((int64_t)seq0 * a.ld_v + (int64_t)h * DV) * ES);
  const uint64_t pos_base = POS ? uni_ptr(a.pos_table) : 0;
  const uint64_t ts_base = TIME ? uni_ptr(a.timestamps + seq0) : 0;

  // Copy key tile kt (keys, values, the block's position-bias values and the
  // raw timestamps) into stage buffer `bufc`.  Rows past the end of the
  // sequence repeat its last row (finite values whose scores are always masked
  // and whose coefficients are therefore 0).
  // A key tile is read once by every query tile that reaches it; in a
  // sequence of at most two query tiles that is at most twice, and such
  // tiles are copied non-temporally (measured on the ranking batch: 50 -> 44
  // us, with the long batches unchanged).
  const bool kv_nt = L <= 2 * kBM;
  auto issue_stage = [&](auto bufc, int kt) __attribute__((always_inline)) {
    SB& sb = stage(bufc);
    const int j0 = kt * kBN;
    const bool whole = j0 + kBN <= L;
    const uint64_t kb = kseq + (uint64_t)j0 * ldk_b, vb = vseq + (uint64_t)j0 * ldv_b;
#pragma unroll
    for (int s = 0; s < SK; ++s) {
      const int n = s * kWaves + wave;   // uniform
      if (n < NK) {
        uint32_t off = k_off[s];
        if (!whole) {
          const int m = 64 * n + lane, row = m / KCH;
          off = (uint32_t)min(row, L - 1 - j0) * ldk_b +
                16u * (uint32_t)((m % KCH) ^ C::kswz(row));
        }
        if (kv_nt) lds_copy16_nt(kb, off, lds_off(sb.k) + 1024u * (uint32_t)n);
        else lds_copy16(kb, off, lds_off(sb.k) + 1024u * (uint32_t)n);
      }
    }
#pragma unroll
    for (int s = 0; s < SV; ++s) {
      const int n = s * kWaves + wave;
      if (n < NV) {
        uint32_t off = v_off[s];
        if (!whole) {
          const int m = 64 * n + lane, row = m / VCH;
          off = (uint32_t)min(row, L - 1 - j0) * ldv_b +
                16u * (uint32_t)((m % VCH) ^ C::vswz(row));
        }
        if (kv_nt) lds_copy16_nt(vb, off, lds_off(sb.v) + 1024u * (uint32_t)n);
        else lds_copy16(vb, off, lds_off(sb.v) + 1024u * (uint32_t)n);
      }
    }
    if constexpr (POS) {
      if (wave > kTsWave) {
        const int p = kWaves - 1 - wave;
        const int d = i0 - j0 + (kBM - 1) - (64 * p + lane);
        const int ix = min(d < 0 ? -d : d, P - 1);
        lds_copy4(pos_base, 4u * (uint32_t)ix, lds_off(sb.diag) + 256u * (uint32_t)p);
      }
    }
    if constexpr (TIME) {
      if (wave == kTsWave) {
        const int j = min(j0 + (lane >> 1), L - 1);
        lds_copy4(ts_base, 8u * (uint32_t)j + 4u * (uint32_t)(lane & 1), lds_off(sb.ts64));
      }
    }
    if constexpr (POS) {
      if (clamp && wave == kTsWave) {   // bias of n_h - j (0 for candidate keys)
        const int d = geo.n_h - (j0 + (lane & (kBN - 1)));
        const int ix = min(d > 0 ? d : 0, P - 1);
        lds_copy4(pos_base, 4u * (uint32_t)ix, lds_off(sb.cpos));
      }
    }
  };

  // row times (loaded in the prologue)
  int64_t tbase = 0;
  uint32_t ti32 = uint32_t(kT32Range);
  bool w_t_ok = true;
  uint32_t w_tmin = 0, w_tmax = 0;

  // Once this wave's own copies of stage kt have landed: rescale the
  // position-bias values it gathered and, in the wave that copied the
  // timestamps, form the 32-bit key times, their range over the valid keys
  // and whether any key needs the 64-bit path.
  auto finish_stage = [&](auto bufc, int kt) __attribute__((always_inline)) {
    SB& sb = stage(bufc);
    if constexpr (POS) {
      if (wave > kTsWave) {
        const int e = 64 * (kWaves - 1 - wave) + lane;
        if (e < kDiag) sb.diag[e] *= pscale;
      }
      if (clamp && wave == kTsWave) sb.cpos[lane] *= pscale;
    }
    if constexpr (TIME) {
      if (wave == kTsWave) {   // lanes 0..31: one key each
        int kl = lane & (kBN - 1);
        asm volatile("" : "+v"(kl));   // addresses from here, not kept live across the loop
        const int64_t tj = sb.ts64[kl];
        const int64_t rel = tj - tbase;
        const bool ok = rel > -kT32Range && rel < kT32Range;
        const uint32_t t32 = ok ? uint32_t(rel + kT32Range) : 0u;
        const int nvalid = min(kBN, L - kt * kBN);   // valid keys of the block (>= 1)
        if (lane < kBN) sb.ts32[kl] = t32;
        const bool bad = __ballot(!ok) != 0;
        // Range of the valid keys' times.  Keys are normally in time order:
        // then it is (first, last), checked with one lane shift; otherwise
        // the block is marked as spanning every bucket (exact per-score path).
        const uint32_t nxt = (uint32_t)__builtin_amdgcn_update_dpp(
            (int)t32, (int)t32, 0x130, 0xf, 0xf, false);   // lane l gets lane l+1
        const bool desc = lane + 1 < nvalid && nxt < t32;
        const bool sorted = __ballot(desc) == 0;
        const uint32_t first = (uint32_t)__builtin_amdgcn_readlane((int)t32, 0);
        const uint32_t last = (uint32_t)__builtin_amdgcn_readlane((int)t32, nvalid - 1);
        if (lane == 0) {
          sb.tmin = sorted ? first : 0u;
          sb.tmax = sorted ? last : 0xffffffffu;
          sb.tbad = bad;
        }
      }
    }
  };

  // Q operand (B operand of S^T = K Q^T), kept in registers
  typename std::conditional<BF, bf16x8, float>::type qf[NKC];
  floatx16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

  // lane -> index into a stage's diag: f = i0 - j0 + 127 - (i - j)
  //   = 127 - 32 wave - l32 + 4hh + 8(r/4) + r%4   (ascending in r%4)
  const int dbase = (kBM - 1) - kRows * wave - l32 + 4 * hh;

  // Whether every (row, key) time gap of block kt for this wave falls in one
  // bucket; then `tb` is that bucket's (log2e-scaled) bias.
  auto time_const = [&](SB& sb, float& tb) __attribute__((always_inline)) -> bool {
    if (!w_t_ok || uni(sb.tbad) != 0) return false;
    const uint32_t kmin = (uint32_t)uni((int)sb.tmin), kmax = (uint32_t)uni((int)sb.tmax);
    uint32_t dmin = 0;
    if (w_tmin > kmax) dmin = w_tmin - kmax;
    if (kmin > w_tmax) dmin = kmin - w_tmax;
    const uint32_t dmax = max(w_tmax > kmin ? w_tmax - kmin : 0u,
                              kmax > w_tmin ? kmax - w_tmin : 0u);
    const int z0 = uni(__builtin_clz(dmin + 1u)), z1 = uni(__builtin_clz(dmax + 1u));
    if (z0 != z1) return false;
    tb = __builtin_bit_cast(float, uni(__builtin_bit_cast(int, tt.trev[z0])));   // scalar
    return true;
  };

  // One 32-key block from stage buffer `sb`: scores, bias, SiLU, mask,
  // aggregation.  Every LDS read of the block is issued first.
  auto block = [&](SB& sb, int kt) __attribute__((always_inline)) {
    const int jb = kt * kBN;
    // ---- LDS reads: score start (position bias) and K operands ----
    floatx16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (POS) s[r] = sb.diag[dbase + 8 * (r >> 2) + (r & 3)];
      else s[r] = 0.0f;
    }
    if constexpr (clamp) {
      if (w_cand) {   // candidate rows: bias of the clamped positions
        const bool cr = i >= geo.n_h;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float cv = sb.cpos[acc_row(r, hh)];
          s[r] = cr ? cv : s[r];
        }
      }
    }
    // K operand of MFMA step c (logical chunk 2c + hh of key row l32)
    auto kread = [&](int c) __attribute__((always_inline)) {
      if constexpr (BF) {
        return *reinterpret_cast<const bf16x8*>(sb.k + l32 * KROW +
                                                16 * ((2 * c + hh) ^ C::kswz(l32)));
      } else {
        const int d = 2 * c + hh;
        return *reinterpret_cast<const float*>(sb.k + l32 * KROW +
                                               16 * ((d >> 2) ^ C::kswz(l32)) + 4 * (d & 3));
      }
    };
    // two halves of the contraction: the second half's reads are issued once
    // the first half's MFMAs have taken their operands
    constexpr int NH = (NKC + 1) / 2;
    typename std::conditional<BF, bf16x8, float>::type kop[NH];
#pragma unroll
    for (int c = 0; c < NH; ++c) kop[c] = kread(c);
    __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the arithmetic
#pragma unroll
    for (int c = 0; c < NH; ++c) {
      if constexpr (BF) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[c], qf[c], s, 0, 0, 0);
      else s = __builtin_amdgcn_mfma_f32_32x32x2f32(kop[c], qf[c], s, 0, 0, 0);
    }
#pragma unroll
    for (int c = NH; c < NKC; ++c) kop[c - NH] = kread(c);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = NH; c < NKC; ++c) {
      if constexpr (BF)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[c - NH], qf[c], s, 0, 0, 0);
      else s = __builtin_amdgcn_mfma_f32_32x32x2f32(kop[c - NH], qf[c], s, 0, 0, 0);
    }

    // V^T operands (bf16): ds_read_b64_tr_b16 -- in each 16-lane group, lane
    // 4e+q loads 4 values of key row e at columns 4q..4q+3 of the group's 16
    // columns; lane c of the group receives column c of the 4 rows.  MFMA ins
    // (keys 16 ins ..) takes rows 16ins + 4hh + {0..3} and 16ins + 8 + 4hh +
    // {0..3}, matching the accumulator rows of the SiLU values it multiplies.
    bf16x8 vop[BF ? 2 * NDB : 1];
    if constexpr (BF) {
      const int gl = lane & 15, grp = lane >> 4;
      const int er = gl >> 2;
      const int rlane = 4 * hh + er;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int col = 32 * db + 16 * (grp & 1) + 4 * (gl & 3);
        const uint32_t base = lds_off(sb.v) + (uint32_t)(rlane * VROW) +
                              16u * (uint32_t)((col >> 3) ^ C::vswz(rlane)) + 2u * (col & 7);
#pragma unroll
        for (int ins = 0; ins < 2; ++ins) {
          const shortx4 lo =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr4(base + (16 * ins) * VROW));
          const shortx4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr4(base + (16 * ins + 8) * VROW));
          vop[2 * db + ins] = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // V reads land during the SiLU


    // ---- x2 = am * S + log2e * time ----
    float x[16];
    if constexpr (TIME) {
      float tb = 0.0f;
      if (time_const(sb, tb)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = fmaf(s[r], am, tb);
      } else if (w_t_ok && uni(sb.tbad) == 0) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const uint4 t4 = *reinterpret_cast<const uint4*>(&sb.ts32[8 * gq + 4 * hh]);
          const uint32_t tv[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t d1 = (ti32 > tv[e] ? ti32 - tv[e] : tv[e] - ti32) + 1u;
            x[4 * gq + e] = fmaf(s[4 * gq + e], am, tt.trev[__builtin_clz(d1)]);
          }
        }
      } else {
        // times too far apart for 32 bits (rare): full 64-bit differences,
        // with the row time read again
        const int64_t t_i = row_valid ? a.timestamps[seq0 + i] : tbase;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t tj = sb.ts64[acc_row(r, hh)];
          const uint64_t dt = t_i >= tj ? uint64_t(t_i) - uint64_t(tj)
                                        : uint64_t(tj) - uint64_t(t_i);
          x[r] = fmaf(s[r], am, tt.tful[63 - __builtin_clzll(dt + 1u)]);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = s[r] * am;
    }

    // ---- illegal pairs: an argument whose SiLU is exactly -0 (2^1e30 is
    // +inf, its reciprocal 0); selecting before the SiLU keeps the SiLU and
    // the aggregation MFMAs in one straight-line stretch ----
    if (!is_full(kt)) {
      const RowBounds rb = row_valid ? row_bounds(geo, i) : RowBounds{kEmptyLo, 0, -1};
      const int jl = jb + 4 * hh - rb.lo, js = jb + 4 * hh - rb.self_j;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 8 * (r >> 2) + (r & 3);
        const bool ok = (uint32_t)(jl + kk) <= (uint32_t)rb.span || js + kk == 0;
        x[r] = ok ? x[r] : kMaskedX;
      }
    }
    float av[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) av[r] = silu2(x[r]);

    // ---- O^T[d][i] += sum_j V[j][d] * A[i][j] ----
    if constexpr (BF) {
      bf16x8 pa[2];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pa[0][e] = (__bf16)av[e];
        pa[1][e] = (__bf16)av[8 + e];
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int ins = 0; ins < 2; ++ins)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[2 * db + ins], pa[ins], acc[db],
                                                           0, 0, 0);
    } else {
      // 32x32x2: contraction slot hh <-> key acc_row(r, hh) for step r
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = 32 * db + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = acc_row(r, hh);
          const float vv = d < DV ? *reinterpret_cast<const float*>(
                                        sb.v + row * VROW + 16 * ((d >> 2) ^ C::vswz(row)) +
                                        4 * (d & 3))
                                  : 0.0f;
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv, av[r], acc[db], 0, 0, 0);
        }
      }
    }
  };

  // ---- item prologue -------------------------------------------------------
  // The first two stages go out first; then the loads the compiler tracks
  // itself (row times, Q), whose completion it waits for right here (the
  // empty asm statements make the registers plain values afterwards, so no
  // wait on them is placed in the stage loop, where it would also drain the
  // copies ahead); then the third stage.
  issue_stage(B0{}, kt_lo);
  if (kt_lo + 1 <= kt_hi) issue_stage(B1{}, kt_lo + 1);
  // Queue: the counter's previous value, fetched by wave 0's lane 0 and read
  // by it only, after the wait below.  Left unset in the other lanes: a
  // default value there would make the compiler merge the two right here,
  // which waits for the atomic and for every copy issued before it.
  int q_fetch;
  if (queue && tid == 0) q_fetch = atomicAdd(const_cast<int32_t*>(a.hdr) + wkq.ctr, 1);
  int64_t ti64 = 0;   // this lane's row time (prologue only)
  if constexpr (TIME) {
    // Neither value is used before the wait below: a use here (a select
    // between them, say) would make the compiler wait for every copy issued
    // so far, the stages above included.  Rows past the tile take the last
    // row's time; their scores are never used.
    tbase = a.timestamps[seq0 + i0];
    ti64 = a.timestamps[seq0 + min(i, i1 - 1)];
  }
  // Q tile: every wave copies its 32 rows into LDS with whole-row copies (1 KB
  // per copy; stage buffers 2 and 3 are not in use yet), then reads its MFMA
  // operands from there.  Rows past the tile repeat its last row.
  const uint32_t q_lds = lds_off(wave < 2 ? st2.k : st3.k) + (uint32_t)((wave & 1) * kRows * KROW);
  if (C::kQLds && wave_rows && !alpha_zero) {
    int ql = lane;   // recomputed per item: kept out of the registers live across items
    asm volatile("" : "+v"(ql));
    const uint64_t qb = uni_ptr(reinterpret_cast<const char*>(a.q) +
                                ((int64_t)(seq0 + i0) * a.ld_q + (int64_t)h * DQK) * ES);
    const uint32_t ldq_b = (uint32_t)(a.ld_q * ES);
#pragma unroll
    for (int n = 0; n < kRows * KCH / 64; ++n) {
      const int m = 64 * n + ql, r = m / KCH;
      const int row = min(wr0 + r, i1 - 1) - i0;
      lds_copy16_nt(qb, (uint32_t)row * ldq_b + 16u * (uint32_t)((m % KCH) ^ C::kswz(r)),
                 q_lds + 1024u * (uint32_t)n);
    }
  }
  if constexpr (!C::kQLds) {
    // Q operands straight from HBM: lane (row i, half hh) takes 16 bytes of
    // its row per MFMA step
    const char* qrow = reinterpret_cast<const char*>(a.q) +
                       ((int64_t)(seq0 + min(i, i1 - 1)) * a.ld_q + (int64_t)h * DQK) * ES;
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      if constexpr (BF) {
        const bf16x8 z = {};
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 16 * (2 * c + hh));
        qf[c] = (row_valid && !alpha_zero) ? v : z;
      } else {
        const float v = *reinterpret_cast<const float*>(qrow + 4 * (2 * c + hh));
        qf[c] = (row_valid && !alpha_zero) ? v : 0.0f;
      }
    }
  }
  wait_vmem<0>();
  asm volatile("" : "+v"(q_fetch));   // a plain value from here: no wait of its own
  if (queue && tid == 0) {
    s_qnext[q_item & 1] = wkq.first + wkq.n + q_fetch;   // published by the barrier below
    // Every processed unit makes one fetch, so the counter ends at the
    // number of units: the fetch that returned the last value was the run's
    // last, and its workgroup rewinds the counter for the next run of the
    // same plan.
    if (q_fetch == wkq.end - wkq.first - 1) const_cast<int32_t*>(a.hdr)[wkq.ctr] = 0;
  }
#pragma unroll
  for (int c = 0; C::kQLds && c < NKC; ++c) {
    if constexpr (BF) {
      const bf16x8 z = {};
      qf[c] = (row_valid && !alpha_zero)
                  ? lds_ld<bf16x8>(q_lds + l32 * KROW + 16 * ((2 * c + hh) ^ C::kswz(l32)))
                  : z;
    } else {
      const int d = 2 * c + hh;
      qf[c] = (row_valid && !alpha_zero)
                  ? lds_ld<float>(q_lds + l32 * KROW + 16 * ((d >> 2) ^ C::kswz(l32)) +
                                  4 * (d & 3))
                  : 0.0f;
    }
  }
  if constexpr (TIME) {
    asm volatile("" : "+v"(ti64));
    const int64_t rel = ti64 - tbase;
    const bool ok = rel > -kT32Range && rel < kT32Range;
    ti32 = ok ? uint32_t(rel + kT32Range) : 0u;
    w_t_ok = __all(ok);
    w_tmin = wave_min(row_valid ? ti32 : 0xffffffffu);
    w_tmax = wave_max(row_valid ? ti32 : 0u);
  }
  finish_stage(B0{}, kt_lo);   // stage kt_lo+1 is finished by the first step
  stage_barrier();             // also publishes the time tables; Q reads are done
  if (kt_lo + 2 <= kt_hi) issue_stage(B2{}, kt_lo + 2);

  // Epilogue staging: each wave uses 32 rows of a stage buffer that neither
  // the last block nor any copy still in flight touches (the buffers after
  // the last block's, last read two or more barriers before the last step).
  const bool ln = a.epilogue == 0;
  auto ep_lds = [&]() __attribute__((always_inline)) -> uint32_t {
    const int b_ep = ((kt_hi - kt_lo) + 1 + (wave >> 1)) & (kStages - 1);
    return (b_ep == 0 ? lds_off(st0.k) : b_ep == 1 ? lds_off(st1.k) : b_ep == 2 ? lds_off(st2.k)
                                                                               : lds_off(st3.k)) +
           (uint32_t)((wave & 1) * kRows * VROW);
  };
  // U rows of this wave into the epilogue buffer; issued at the start of the
  // last step so that their latency hides behind the last block.
  auto issue_u = [&]() __attribute__((always_inline)) {
    if (!C::kEpLds || !(ln && wave_rows)) return;
    int ul = lane;
    asm volatile("" : "+v"(ul));
    const uint32_t e_lds = ep_lds();
    const uint64_t ub = uni_ptr(reinterpret_cast<const char*>(a.u) +
                                ((int64_t)(seq0 + i0) * a.ld_u + (int64_t)h * DV) * ES);
    const uint32_t ldu_b = (uint32_t)(a.ld_u * ES);
#pragma unroll
    for (int n = 0; n < kRows * VCH / 64; ++n) {
      const int m = 64 * n + ul, r = m / VCH;
      const int row = min(wr0 + r, i1 - 1) - i0;
      lds_copy16_nt(ub, (uint32_t)row * ldu_b + 16u * (uint32_t)((m % VCH) ^ row_swz<VCH>(r)),
                 e_lds + 1024u * (uint32_t)n);
    }
  };

  // One pipeline step on key block kt held in buffer `bufc`: copy block kt+3
  // into the buffer freed by the previous barrier, compute block kt, then
  // (own copies of block kt+1 landed) finish block kt+1 and synchronise.
  auto step = [&](auto bufc, int kt) __attribute__((always_inline)) {
    constexpr int b = decltype(bufc)::value;
    using N1 = std::integral_constant<int, (b + 1) % kStages>;
    using N3 = std::integral_constant<int, (b + 3) % kStages>;
    const bool more3 = kt + 3 <= kt_hi, more2 = kt + 2 <= kt_hi;
    if (more3) issue_stage(N3{}, kt + 3);
    if (kt + 1 <= kt_hi) {
      wait_vmem_n(more3 ? 2 * my_copies : (more2 ? my_copies : 0));
      finish_stage(N1{}, kt + 1);   // its LDS traffic overlaps block kt
    } else {
      issue_u();
    }
    if (needs(kt)) block(stage(bufc), kt);
    if (kt + 1 <= kt_hi) stage_barrier();
  };
  for (int kt = kt_lo;; kt += kStages) {
    step(B0{}, kt);
    if (kt + 1 > kt_hi) break;
    step(B1{}, kt + 1);
    if (kt + 2 > kt_hi) break;
    step(B2{}, kt + 2);
    if (kt + 3 > kt_hi) break;
    step(B3{}, kt + 3);
    if (kt + 4 > kt_hi) break;
  }

  // ---- chunk of a split item: publish the partial output; the chunk that
  // arrives last adds all partials in chunk order and runs the epilogue ----
  // The partials are written and read only with device-scope (agent) atomic
  // stores and loads, which go to and come from the device's coherence point
  // (global_store/global_load with sc1) on whatever XCD the chunks run: a
  // chunk's stores have completed (vmcnt 0) before its workgroup bumps the
  // item's arrival counter, and the last chunk issues its loads only after
  // its own bump has returned the count of the others.  No cache-wide
  // write-back or invalidation is needed.
  const int n_chunks = ch.w & 0x7fff;
  if (n_chunks > 1) {
    // slot layout: [wave][db][r/4][lane] x 4 floats (two 8-byte words)
    auto slot = [&](int c) __attribute__((always_inline)) {
      return reinterpret_cast<uint64_t*>(a.partials + (int64_t)(ch.z + c) * a.slot_floats) +
             2 * (wave * NDB * 4 * 64 + lane);
    };
    uint64_t* own = slot((ch.w >> 16) & 0x7fff);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int hw = 0; hw < 2; ++hw) {
          // (__float_as_uint, not __builtin_bit_cast: this compiler turns a
          // bit cast of a vector element into a cast of element 0)
          const uint64_t w2 = (uint64_t)__float_as_uint(acc[db][4 * q4 + 2 * hw]) |
                              ((uint64_t)__float_as_uint(acc[db][4 * q4 + 2 * hw + 1]) << 32);
          __hip_atomic_store(own + 2 * (db * 4 + q4) * 64 + hw, w2, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
    wait_vmem<0>();    // this wave's partial has reached the coherence point
    __syncthreads();
    if (tid == 0)
      s_ticket = __hip_atomic_fetch_add(a.counters + ch.z, 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_ticket != n_chunks - 1) continue;   // another chunk finishes the item
    if (tid == 0) a.counters[ch.z] = 0;       // ready for the next run of this plan
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
    for (int c = 0; c < n_chunks; ++c) {
      const uint64_t* src = slot(c);
      uint64_t p[NDB][4][2];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
          for (int hw = 0; hw < 2; ++hw)
            p[db][q4][hw] = __hip_atomic_load(src + 2 * (db * 4 + q4) * 64 + hw,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
          for (int hw = 0; hw < 2; ++hw) {
            acc[db][4 * q4 + 2 * hw] += __uint_as_float((uint32_t)p[db][q4][hw]);
            acc[db][4 * q4 + 2 * hw + 1] += __uint_as_float((uint32_t)(p[db][q4][hw] >> 32));
          }
    }
  }

  // ---- epilogue: ln(2)/n_scale, LayerNorm over d_v, * U, store ------------
  // acc[db][r] holds d = 32db + 8(r/4) + 4hh + r%4 of row i.  U comes in and
  // the output goes out through LDS with whole-row copies and stores (8 full
  // 128-byte lines per instruction); each wave uses 32 rows of a stage buffer
  // that the last block does not read (the other waves may still be in it).
  const float osc = a.out_scale;
  float mean = 0.0f, rstd = 1.0f;
  int el = lane;   // recomputed per item: kept out of the registers live across items
  asm volatile("" : "+v"(el));
  const uint32_t e_lds = ep_lds();
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] *= osc;
  // the aggregation before the gate, kept for the backward (training)
  if (a.out_raw != nullptr && row_valid) {
    char* rrow = reinterpret_cast<char*>(a.out_raw) +
                 ((int64_t)(seq0 + i) * a.ld_raw + (int64_t)h * DV) * ES;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * db + 8 * gq + 4 * hh;
        if (d0 < DV) {
          if constexpr (BF) {
            bf16x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (__bf16)acc[db][4 * gq + e];
            *reinterpret_cast<bf16x4*>(rrow + 2 * d0) = o;
          } else {
            floatx4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = acc[db][4 * gq + e];
            *reinterpret_cast<floatx4*>(rrow + 4 * d0) = o;
          }
        }
      }
  }
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
  if (!C::kEpLds && row_valid) {
    // y = (O - mean) * rstd * U straight between registers and HBM
    const char* urow = reinterpret_cast<const char*>(a.u) +
                       ((int64_t)(seq0 + i) * a.ld_u + (int64_t)h * DV) * ES;
    char* orow = reinterpret_cast<char*>(a.out) +
                 ((int64_t)(seq0 + i) * a.ld_out + (int64_t)h * DV) * ES;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * db + 8 * gq + 4 * hh;
        if (d0 < DV) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = acc[db][4 * gq + e];
          if constexpr (BF) {
            if (ln) {
              const bf16x4 uu = *reinterpret_cast<const bf16x4*>(urow + 2 * d0);
#pragma unroll
              for (int e = 0; e < 4; ++e) y[e] = (y[e] - mean) * rstd * (float)uu[e];
            }
            bf16x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (__bf16)y[e];
            __builtin_nontemporal_store(o, reinterpret_cast<bf16x4*>(orow + 2 * d0));
          } else {
            if (ln) {
              const floatx4 uu = *reinterpret_cast<const floatx4*>(urow + 4 * d0);
#pragma unroll
              for (int e = 0; e < 4; ++e) y[e] = (y[e] - mean) * rstd * uu[e];
            }
            floatx4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = y[e];
            __builtin_nontemporal_store(o, reinterpret_cast<floatx4*>(orow + 4 * d0));
          }
        }
      }
  }
  if (C::kEpLds && wave_rows) {
    wait_vmem<0>();   // this wave's U rows have landed
    // y = (O - mean) * rstd * U in place of U, as the output's element type
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * db + 8 * gq + 4 * hh;
        if (d0 < DV) {
          const int byte = d0 * ES;
          const uint32_t off = e_lds + (uint32_t)(l32 * VROW) +
                               16u * (uint32_t)((byte >> 4) ^ row_swz<VCH>(l32)) +
                               (uint32_t)(byte & 15);
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = acc[db][4 * gq + e];
          if constexpr (BF) {
            if (ln) {
              const bf16x4 uu = lds_ld<bf16x4>(off);
#pragma unroll
              for (int e = 0; e < 4; ++e) y[e] = (y[e] - mean) * rstd * (float)uu[e];
            }
            bf16x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (__bf16)y[e];
            lds_st<bf16x4>(off, o);
          } else {
            if (ln) {
              const floatx4 uu = lds_ld<floatx4>(off);
#pragma unroll
              for (int e = 0; e < 4; ++e) y[e] = (y[e] - mean) * rstd * uu[e];
            }
            floatx4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = y[e];
            lds_st<floatx4>(off, o);
          }
        }
      }
    // whole rows out: lane l of store n writes physical chunk (64n + l) % VCH
    // of row (64n + l) / VCH, i.e. logical chunk ^ swizzle, rows of the tile only
    char* obase = reinterpret_cast<char*>(uni_ptr(
        reinterpret_cast<char*>(a.out) + ((int64_t)(seq0 + wr0) * a.ld_out + (int64_t)h * DV) * ES));
    const uint32_t ldo_b = (uint32_t)(a.ld_out * ES);
#pragma unroll
    for (int n = 0; n < kRows * VCH / 64; ++n) {
      const int m = 64 * n + el, r = m / VCH;
      const uintx4 w4 = lds_ld<uintx4>(e_lds + 16u * (uint32_t)m);
      if (wr0 + r < i1)
        __builtin_nontemporal_store(w4, reinterpret_cast<uintx4*>(obase + ((uint32_t)r * ldo_b +
                                           16u * (uint32_t)((m % VCH) ^ row_swz<VCH>(r)))));
    }
  }

  // The LDS of this item is free again once every wave is here; the output
  // stores need not have completed (the next item's first wait covers them).
  stage_barrier();
  }  // units
  }  // planned workgroups
}

template <typename T, int DQK, int DV, int POSM, bool TIME>
static hipError_t launch_one(const AttnArgs& a, int n_wg, hipStream_t stream, hipEvent_t start,
                             hipEvent_t stop) {
  auto kern = hstu_attn_fwd_kernel<T, DQK, DV, POSM, TIME>;
  if (start || stop)
    hipExtLaunchKernelGGL(kern, dim3((unsigned)n_wg), dim3(kThreads), 0, stream, start, stop, 0,
                          a);
  else
    hipLaunchKernelGGL(kern, dim3((unsigned)n_wg), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// Resident workgroups per CU for one instantiation.
template <typename T, int DQK, int DV, int POSM, bool TIME>
static int blocks_per_cu() {
  auto kern = hstu_attn_fwd_kernel<T, DQK, DV, POSM, TIME>;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, kThreads, 0) != hipSuccess)
    return -1;
  return nb;
}

template <typename T, int DQK, int DV>
static hipError_t launch_bias(const AttnArgs& a, int n_wg, hipStream_t stream, hipEvent_t t0,
                              hipEvent_t t1) {
  const bool pos = a.pos_len > 0, tim = a.time_len > 0, cl = a.pos_clamp != 0;
  if (pos && cl && tim) return launch_one<T, DQK, DV, 2, true>(a, n_wg, stream, t0, t1);
  if (pos && cl) return launch_one<T, DQK, DV, 2, false>(a, n_wg, stream, t0, t1);
  if (pos && tim) return launch_one<T, DQK, DV, 1, true>(a, n_wg, stream, t0, t1);
  if (pos) return launch_one<T, DQK, DV, 1, false>(a, n_wg, stream, t0, t1);
  if (tim) return launch_one<T, DQK, DV, 0, true>(a, n_wg, stream, t0, t1);
  return launch_one<T, DQK, DV, 0, false>(a, n_wg, stream, t0, t1);
}

template <typename T, int DQK, int DV>
static int bpc_bias(int pos_len, int time_len, bool cl) {
  const bool pos = pos_len > 0, tim = time_len > 0;
  if (pos && cl && tim) return blocks_per_cu<T, DQK, DV, 2, true>();
  if (pos && cl) return blocks_per_cu<T, DQK, DV, 2, false>();
  if (pos && tim) return blocks_per_cu<T, DQK, DV, 1, true>();
  if (pos) return blocks_per_cu<T, DQK, DV, 1, false>();
  if (tim) return blocks_per_cu<T, DQK, DV, 0, true>();
  return blocks_per_cu<T, DQK, DV, 0, false>();
}

int attn_grid(int dtype, int d_qk, int d_v, int pos_len, int time_len, bool clamp) {
  int bpc = -1;
  if (dtype == 1) {
    if (d_qk == 128 && d_v == 128) bpc = bpc_bias<__bf16, 128, 128>(pos_len, time_len, clamp);
    if (d_qk == 64 && d_v == 64) bpc = bpc_bias<__bf16, 64, 64>(pos_len, time_len, clamp);
    if (d_qk == 64 && d_v == 128) bpc = bpc_bias<__bf16, 64, 128>(pos_len, time_len, clamp);
    if (d_qk == 128 && d_v == 64) bpc = bpc_bias<__bf16, 128, 64>(pos_len, time_len, clamp);
    if (d_qk == 256 && d_v == 256) bpc = bpc_bias<__bf16, 256, 256>(pos_len, time_len, clamp);
  } else if (dtype == 0) {
    if (d_qk == 128 && d_v == 128) bpc = bpc_bias<float, 128, 128>(pos_len, time_len, clamp);
    if (d_qk == 64 && d_v == 64) bpc = bpc_bias<float, 64, 64>(pos_len, time_len, clamp);
    if (d_qk == 8 && d_v == 8) bpc = bpc_bias<float, 8, 8>(pos_len, time_len, clamp);
  }
  if (bpc <= 0) return -1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  return cus * bpc;
}

bool attn_supported(int dtype, int d_qk, int d_v) {
  if (dtype == 1)
    return (d_qk == 128 && d_v == 128) || (d_qk == 64 && d_v == 64) ||
           (d_qk == 64 && d_v == 128) || (d_qk == 128 && d_v == 64) ||
           (d_qk == 256 && d_v == 256);
  if (dtype == 0) return (d_qk == 128 && d_v == 128) || (d_qk == 64 && d_v == 64) ||
                         (d_qk == 8 && d_v == 8);
  return false;
}

hipError_t launch_attn(const AttnArgs& a, int dtype, int d_qk, int d_v, int n_wg,
                       hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  if (dtype == 1) {
    if (d_qk == 128 && d_v == 128) return launch_bias<__bf16, 128, 128>(a, n_wg, stream, t0, t1);
    if (d_qk == 64 && d_v == 64) return launch_bias<__bf16, 64, 64>(a, n_wg, stream, t0, t1);
    if (d_qk == 64 && d_v == 128) return launch_bias<__bf16, 64, 128>(a, n_wg, stream, t0, t1);
    if (d_qk == 128 && d_v == 64) return launch_bias<__bf16, 128, 64>(a, n_wg, stream, t0, t1);
    if (d_qk == 256 && d_v == 256) return launch_bias<__bf16, 256, 256>(a, n_wg, stream, t0, t1);
  } else if (dtype == 0) {
    if (d_qk == 128 && d_v == 128) return launch_bias<float, 128, 128>(a, n_wg, stream, t0, t1);
    if (d_qk == 64 && d_v == 64) return launch_bias<float, 64, 64>(a, n_wg, stream, t0, t1);
    if (d_qk == 8 && d_v == 8) return launch_bias<float, 8, 8>(a, n_wg, stream, t0, t1);
  }
  return hipErrorInvalidValue;
}

}  // namespace hstu
