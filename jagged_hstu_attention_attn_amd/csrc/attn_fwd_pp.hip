// attn_fwd_pp.hip -- gfx950 jagged HSTU attention forward for long sequences:
// eight waves per workgroup, one workgroup per CU, and the two waves that
// share a SIMD alternate between matrix-core work and vector work.
//
// Work items are the scheduler's units (sequence, head, 128-row query tile,
// key-tile range), as for the four-wave kernel.  Wave w and wave w + 4 own the
// same 32 query rows and run on the same SIMD (waves of a workgroup are
// placed on SIMD w % 4).  The item's key tiles are dealt between the two
// groups of four waves (group 0: tiles kt_lo, kt_lo + 2, ...; group 1: kt_lo +
// 1, kt_lo + 3, ...), so each group accumulates a partial O over half of the
// keys; the aggregation is a plain sum over keys (no softmax), so the halves
// simply add at the end.
//
// Per 32-key block a wave runs
//   matrix phase:  O^T += V^T A^T for its previous block, then
//                  S^T  = K Q^T + C for its current block   (16 bf16 MFMAs)
//   vector phase:  x = am S + time bias, mask select, SiLU -> A (bf16)
// and the two groups are kept half a step apart by the workgroup barrier:
//   phase X: group 0 matrix phase   | group 1 vector phase
//   phase Y: group 0 vector phase   | group 1 matrix phase
// so on every SIMD one wave keeps the matrix core busy while its partner
// issues the exponentials and reciprocals of the SiLU -- the two wave kinds
// overlap in hardware instead of relying on the compiler to interleave them.
//
// Keys are staged 32 per block in a ring of 8 LDS slots (keys, values,
// position-bias diagonal, timestamps), copied from HBM straight into LDS
// (global_load_lds) two steps (four blocks) ahead.  The epilogue splits the
// columns: wave w finishes d_v columns 0-63 of its rows and wave w + 4
// columns 64-127, after the partner waves exchange the other half of their
// partial O through LDS; LayerNorm statistics combine across the pair.
//
// Method: pointwise SiLU aggregation with position/time bias, zeroing after
// the nonlinearity, Norm then U gating ("HSTU tensor by tensor: SiLU
// aggregation, temporal bias and gating", sections "SiLU aggregation
// coefficients are not probabilities", "Do not copy softmax masking
// mechanically", "Relative time adds information content similarity lacks",
// "Similar shape, different aggregation").
#include <hip/hip_ext.h>

#include "attn_common.hpp"

namespace hstu {

constexpr int kPPWaves = 8;
constexpr int kPPThreads = kPPWaves * 64;
constexpr int kRing = 8;          // LDS slots of the key/value ring
constexpr int kPPRows = 32;       // query rows per wave
constexpr int kPPAhead = 2;       // steps (two blocks each) copied ahead
static_assert(kBM == 4 * kPPRows, "four row groups of 32 per item");
static_assert(kBN == 32, "a key block is one 32-key score tile");

template <bool CLAMP>
struct PPSlot {
  char k[kBN * 256];            // keys: row j at byte 256 j, 16-byte chunks swizzled
  char v[kBN * 256];            // values
  float diag[kDiagCopies * 64]; // position bias of i - j = i0 - j0 + 127 - f, at f
  int64_t ts64[kBN];            // raw key timestamps
  uint32_t ts32[kBN];           // key timestamps relative to the item's base
  uint32_t tmin, tmax;          // range of ts32 over the valid keys
  int tbad;                     // some key needs the 64-bit time path
  int pad_;
  float cpos[CLAMP ? 64 : 4];   // clamped-position bias of key (lane % 32): n_h - j
};

// POSM: 0 = no position bias, 1 = position bias of |i - j|, 2 = of the
// clamped positions |p_i - p_j| (candidate rows take it from cpos).
template <int POSM, bool TIME>
__global__ __launch_bounds__(kPPThreads) __attribute__((amdgpu_waves_per_eu(2))) void
hstu_attn_fwd_pp_kernel(AttnArgs a) {
  constexpr bool POS = POSM != 0;
  constexpr bool clamp = POSM == 2;
  using C = Cfg<__bf16, 128, 128>;
  using SL = PPSlot<clamp>;
  constexpr int KROW = 256, VROW = 256, KCH = 16;
  constexpr int NKC = 8;     // MFMA steps of the scores (d_qk / 16)
  constexpr int NDB = 4;     // 32-wide d_v blocks of O^T
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  __shared__ __align__(16) SL ring[kRing];
  __shared__ TimeTables tt;
  __shared__ int s_ticket;
  __shared__ int s_qnext[2];
  __shared__ float s_red[2][kPPWaves][kPPRows];   // LayerNorm partial sums of the pairs

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 2;        // group: which half of the key blocks
  const int wq = wave & 3;        // row group: rows 32 wq .. 32 wq + 31 of the item
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int P = a.pos_len;
  const int H = a.num_heads;
  const float alpha2 = a.alpha * kLog2e;
  const bool alpha_zero = alpha2 == 0.0f;
  const float am = alpha_zero ? 1.0f : alpha2;   // x2 = am * S + time
  const float pscale = kLog2e / am;              // position bias in accumulator units
  const uint32_t ldk_b = (uint32_t)(a.ld_k * 2), ldv_b = (uint32_t)(a.ld_v * 2);

  if constexpr (TIME) {
    const int Tt = a.time_len;
    if (tid < 32) tt.trev[tid] = kLog2e * a.time_table[min(31 - tid, Tt - 1)];
    if (tid < 64) tt.tful[tid] = kLog2e * a.time_table[min(tid, Tt - 1)];
  }

  // Copies of one block: wave w copies 1 KB chunk w of its keys and of its
  // values (rows 4w .. 4w+3); waves 0-5 gather the position-bias diagonal
  // (block w / 3, part w % 3), waves 6-7 the raw timestamps (block w - 6),
  // waves 0-1 the clamped-position bias (block w).
  // Per-lane values are derived inside the loops from `opaque_lane()`, which
  // the compiler cannot hoist: computing them again costs a few vector
  // instructions, keeping them live across the loop costs registers the
  // accumulators need.
  auto opaque_lane = [&]() __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    return ln;
  };
  // copies this wave issues for block b (0 / 1) of a step
  auto block_copies = [&](int b) __attribute__((always_inline)) -> int {
    return 2 + ((POS && wave < 6 && wave / 3 == b) ? 1 : 0) +
           ((TIME && wave >= 6 && wave - 6 == b) ? 1 : 0) + ((clamp && wave == b) ? 1 : 0);
  };

  // Work walk (as the four-wave kernel): static plan or work queues.
  const bool queue = a.hdr[2] != kPlanStatic;
  const WorkQueue wkq = work_queue(a.hdr);
  const int n_plan = queue ? (int)gridDim.x : a.hdr[0];
  int q_item = 0;
  for (int v = blockIdx.x; v < n_plan; v += gridDim.x) {
  const int u_begin = queue ? wkq.first + wkq.w : a.wg[2 * v];
  const int u_end = queue ? wkq.end : u_begin + a.wg[2 * v + 1];
  for (int u = u_begin; u < u_end; u = queue ? s_qnext[(q_item++) & 1] : u + 1) {
  const int4 it = a.units[2 * u];
  const int4 ch = a.units[2 * u + 1];
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
  const int n = kt_hi - kt_lo + 1;           // blocks of this unit (>= 1)
  const int n0 = (n + 1) >> 1, n1 = n >> 1;  // blocks of group 0 / group 1
  const int ng = g ? n1 : n0;
  const int S = n0 + 1;                      // steps (the last one only aggregates)
  auto kt_of = [&](int t) __attribute__((always_inline)) { return kt_lo + 2 * t + g; };
  auto slot_of = [&](int kt) __attribute__((always_inline)) -> SL& {
    return ring[(kt - kt_lo) & (kRing - 1)];
  };

  // ---- per-lane query row and the wave's uniform key bounds --------------
  const int wr0 = i0 + wq * kPPRows;
  const int i = wr0 + l32;
  const bool row_valid = i < i1;
  const bool wave_rows = wr0 < i1;
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
  const bool w_cand = clamp && wave_rows && wr0 + kPPRows - 1 >= geo.n_h;
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
                                ((int64_t)seq0 * a.ld_k + (int64_t)h * 128) * 2);
  const uint64_t vseq = uni_ptr(reinterpret_cast<const char*>(a.v) +
                                ((int64_t)seq0 * a.ld_v + (int64_t)h * 128) * 2);
  const uint64_t pos_base = POS ? uni_ptr(a.pos_table) : 0;
  const uint64_t ts_base = TIME ? uni_ptr(a.timestamps + seq0) : 0;
  const bool kv_nt = L <= 2 * kBM;

  // Copy key block kt into its ring slot; b = its place (0 / 1) in its step.
  // Rows past the end of the sequence repeat its last row.
  auto issue_block = [&](int kt, int b) __attribute__((always_inline)) {
    SL& sl = slot_of(kt);
    const int j0 = kt * kBN;
    const int ln = opaque_lane();
    const int kv_row = 4 * wave + (ln >> 4);
    const uint32_t kv_chunk = 16u * (uint32_t)((ln & 15) ^ C::kswz(kv_row));
    const uint32_t v_chunk = 16u * (uint32_t)((ln & 15) ^ C::vswz(kv_row));
    const uint32_t r = (uint32_t)min(kv_row, L - 1 - j0);   // rows past L repeat row L - 1
    const uint32_t ko = r * ldk_b + kv_chunk, vo = r * ldv_b + v_chunk;
    const uint64_t kb = kseq + (uint64_t)j0 * ldk_b, vb = vseq + (uint64_t)j0 * ldv_b;
    if (kv_nt) {
      lds_copy16_nt(kb, ko, lds_off(sl.k) + 1024u * (uint32_t)wave);
      lds_copy16_nt(vb, vo, lds_off(sl.v) + 1024u * (uint32_t)wave);
    } else {
      lds_copy16(kb, ko, lds_off(sl.k) + 1024u * (uint32_t)wave);
      lds_copy16(vb, vo, lds_off(sl.v) + 1024u * (uint32_t)wave);
    }
    if constexpr (POS) {
      if (wave < 6 && wave / 3 == b) {
        const int p = wave - 3 * b;
        const int d = i0 - j0 + (kBM - 1) - (64 * p + ln);
        const int ix = min(d < 0 ? -d : d, P - 1);
        lds_copy4(pos_base, 4u * (uint32_t)ix, lds_off(sl.diag) + 256u * (uint32_t)p);
      }
      if (clamp && wave == b) {   // bias of n_h - j (0 for candidate keys)
        const int d = geo.n_h - (j0 + (ln & (kBN - 1)));
        const int ix = min(d > 0 ? d : 0, P - 1);
        lds_copy4(pos_base, 4u * (uint32_t)ix, lds_off(sl.cpos));
      }
    }
    if constexpr (TIME) {
      if (wave >= 6 && wave - 6 == b) {
        const int j = min(j0 + (ln >> 1), L - 1);
        lds_copy4(ts_base, 8u * (uint32_t)j + 4u * (uint32_t)(ln & 1), lds_off(sl.ts64));
      }
    }
  };
  // blocks of step s: 2s and 2s + 1 (item-relative), those that exist
  auto step_blocks = [&](int s) __attribute__((always_inline)) {
    return s < 0 ? 0 : min(2, max(0, n - 2 * s));
  };
  auto issue_step = [&](int s) __attribute__((always_inline)) {
    const int nb = step_blocks(s);
    if (nb > 0) issue_block(kt_lo + 2 * s, 0);
    if (nb > 1) issue_block(kt_lo + 2 * s + 1, 1);
  };
  auto step_copies = [&](int s) __attribute__((always_inline)) -> int {
    const int nb = step_blocks(s);
    return (nb > 0 ? block_copies(0) : 0) + (nb > 1 ? block_copies(1) : 0);
  };

  // row times (loaded in the prologue)
  int64_t tbase = 0;
  uint32_t ti32 = uint32_t(kT32Range);
  bool w_t_ok = true;
  uint32_t w_tmin = 0, w_tmax = 0;

  // Key times of block kt, once its copies have landed: 32-bit times relative
  // to the item's base, their range over the valid keys, and whether any key
  // needs the 64-bit path.  Run by one wave; read after the next barrier.
  auto finish_ts = [&](int kt) __attribute__((always_inline)) {
    SL& sl = slot_of(kt);
    const int kl = opaque_lane() & (kBN - 1);
    const int64_t tj = sl.ts64[kl];
    const int64_t rel = tj - tbase;
    const bool ok = rel > -kT32Range && rel < kT32Range;
    const uint32_t t32 = ok ? uint32_t(rel + kT32Range) : 0u;
    const int nvalid = min(kBN, L - kt * kBN);
    if (lane < kBN) sl.ts32[kl] = t32;
    const bool bad = __ballot(!ok) != 0;
    const uint32_t nxt = (uint32_t)__builtin_amdgcn_update_dpp(
        (int)t32, (int)t32, 0x130, 0xf, 0xf, false);   // lane l gets lane l+1
    const bool desc = lane + 1 < nvalid && nxt < t32;
    const bool sorted = __ballot(desc) == 0;
    const uint32_t first = (uint32_t)__builtin_amdgcn_readlane((int)t32, 0);
    const uint32_t last = (uint32_t)__builtin_amdgcn_readlane((int)t32, nvalid - 1);
    if (lane == 0) {
      sl.tmin = sorted ? first : 0u;
      sl.tmax = sorted ? last : 0xffffffffu;
      sl.tbad = bad;
    }
  };

  // Q operand (B operand of S^T = K Q^T) and the O^T accumulators
  bf16x8 qf[NKC];
  floatx16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
  floatx16 s;          // scores of the wave's current block (matrix -> vector phase)
  bf16x8 pa[2];        // its SiLU values (vector -> next matrix phase)
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.0f;
  pa[0] = bf16x8{};
  pa[1] = bf16x8{};

  // position-bias diagonal index of score r of lane (l32, hh):
  // f = i0 - j0 + 127 - (i - j) = 127 - 32 wq - l32 + 4hh + 8(r/4) + r%4

  auto time_const = [&](SL& sl, float& tb) __attribute__((always_inline)) -> bool {
    if (!w_t_ok || uni(sl.tbad) != 0) return false;
    const uint32_t kmin = (uint32_t)uni((int)sl.tmin), kmax = (uint32_t)uni((int)sl.tmax);
    uint32_t dmin = 0;
    if (w_tmin > kmax) dmin = w_tmin - kmax;
    if (kmin > w_tmax) dmin = kmin - w_tmax;
    const uint32_t dmax = max(w_tmax > kmin ? w_tmax - kmin : 0u,
                              kmax > w_tmin ? kmax - w_tmin : 0u);
    const int z0 = uni(__builtin_clz(dmin + 1u)), z1 = uni(__builtin_clz(dmax + 1u));
    if (z0 != z1) return false;
    tb = __builtin_bit_cast(float, uni(__builtin_bit_cast(int, tt.trev[z0])));
    return true;
  };

  // ---- matrix phase of group block t: aggregate block t-1, score block t --
  // Operands come from LDS in halves (V^T of d_v blocks 0-1, then 2-3; K of
  // contraction steps 0-3, then 4-7) and the two independent MFMA chains
  // alternate, so each half's reads land while the other chain runs.
  auto mfma_phase = [&](int t) __attribute__((always_inline)) {
    const bool agg = t >= 1 && t - 1 < ng && needs(kt_of(t - 1));
    const bool sc = t < ng && needs(kt_of(t));
    if (!agg && !sc) return;
    const int ln = opaque_lane();
    const int ml32 = ln & 31, mhh = ln >> 5;
    // V^T operands of block t-1 (ds_read_b64_tr_b16: in each 16-lane group
    // lane 4e+q loads 4 values of key row e at columns 4q..4q+3 of the
    // group's 16 columns; lane c receives column c of the 4 rows)
    SL& sv = slot_of(kt_of(t - 1));
    const int vgl = ln & 15, vgrp = ln >> 4;
    const int rlane = 4 * mhh + (vgl >> 2);
    auto vread = [&](bf16x8* vop, int db0) __attribute__((always_inline)) {
#pragma unroll
      for (int d2 = 0; d2 < 2; ++d2) {
        const int col = 32 * (db0 + d2) + 16 * (vgrp & 1) + 4 * (vgl & 3);
        const uint32_t base = lds_off(sv.v) + (uint32_t)(rlane * VROW) +
                              16u * (uint32_t)((col >> 3) ^ C::vswz(rlane)) + 2u * (col & 7);
#pragma unroll
        for (int ins = 0; ins < 2; ++ins) {
          const shortx4 lo =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr4(base + (16 * ins) * VROW));
          const shortx4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr4(base + (16 * ins + 8) * VROW));
          vop[2 * d2 + ins] = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
    };
    auto vmfma = [&](const bf16x8* vop, int db0) __attribute__((always_inline)) {
#pragma unroll
      for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
        for (int ins = 0; ins < 2; ++ins)
          acc[db0 + d2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[2 * d2 + ins], pa[ins],
                                                                  acc[db0 + d2], 0, 0, 0);
    };
    SL& sk = slot_of(kt_of(t));
    auto kread = [&](bf16x8* kop, int c0) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        kop[c] = *reinterpret_cast<const bf16x8*>(
            sk.k + ml32 * KROW + 16 * ((2 * (c0 + c) + mhh) ^ C::kswz(ml32)));
    };
    auto kmfma = [&](const bf16x8* kop, int c0) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[c], qf[c0 + c], s, 0, 0, 0);
    };
    // position-bias start of the scores
    auto sinit = [&]() __attribute__((always_inline)) {
      const int mdbase = (kBM - 1) - kPPRows * wq - ml32 + 4 * mhh;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (POS) s[r] = sk.diag[mdbase + 8 * (r >> 2) + (r & 3)];
        else s[r] = 0.0f;
      }
      if constexpr (clamp) {
        if (w_cand) {
          const bool cr = i >= geo.n_h;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float cv = sk.cpos[acc_row(r, mhh)];
            s[r] = cr ? cv : s[r];
          }
        }
      }
    };
    bf16x8 va[4], vb[4], ka[4], kb[4];
    if (agg && sc) {
      vread(va, 0);
      kread(ka, 0);
      sinit();
      __builtin_amdgcn_sched_barrier(0);
      vmfma(va, 0);
      vread(vb, 2);
      if constexpr (POS) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] *= pscale;
      }
      __builtin_amdgcn_sched_barrier(0);
      kmfma(ka, 0);
      kread(kb, 4);
      __builtin_amdgcn_sched_barrier(0);
      vmfma(vb, 2);
      kmfma(kb, 4);
    } else if (agg) {
      vread(va, 0);
      vread(vb, 2);
      __builtin_amdgcn_sched_barrier(0);
      vmfma(va, 0);
      vmfma(vb, 2);
    } else {
      kread(ka, 0);
      sinit();
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (POS) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] *= pscale;
      }
      kmfma(ka, 0);
      kread(kb, 4);
      __builtin_amdgcn_sched_barrier(0);
      kmfma(kb, 4);
    }
  };

  // ---- vector phase of group block t: bias, mask, SiLU -> bf16 ------------
  auto valu_phase = [&](int t) __attribute__((always_inline)) {
    if (t < 0 || t >= ng) return;
    const int kt = kt_of(t);
    if (!needs(kt)) return;
    SL& sl = slot_of(kt);
    const int jb = kt * kBN;
    const int vhh = opaque_lane() >> 5;
    float x[16];
    if constexpr (TIME) {
      float tb = 0.0f;
      if (time_const(sl, tb)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = fmaf(s[r], am, tb);
      } else if (w_t_ok && uni(sl.tbad) == 0) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const uint4 t4 = *reinterpret_cast<const uint4*>(&sl.ts32[8 * gq + 4 * vhh]);
          const uint32_t tv[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t d1 = (ti32 > tv[e] ? ti32 - tv[e] : tv[e] - ti32) + 1u;
            x[4 * gq + e] = fmaf(s[4 * gq + e], am, tt.trev[__builtin_clz(d1)]);
          }
        }
      } else {
        const int64_t t_i = row_valid ? a.timestamps[seq0 + i] : tbase;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t tj = sl.ts64[acc_row(r, vhh)];
          const uint64_t dt = t_i >= tj ? uint64_t(t_i) - uint64_t(tj)
                                        : uint64_t(tj) - uint64_t(t_i);
          x[r] = fmaf(s[r], am, tt.tful[63 - __builtin_clzll(dt + 1u)]);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = s[r] * am;
    }
    if (!is_full(kt)) {
      const RowBounds rb = row_valid ? row_bounds(geo, i) : RowBounds{kEmptyLo, 0, -1};
      int jl = jb + 4 * vhh - rb.lo, js = jb + 4 * vhh - rb.self_j;
      asm volatile("" : "+v"(jl), "+v"(js));   // per block: not 32 per-item offsets
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 8 * (r >> 2) + (r & 3);
        const bool ok = (uint32_t)(jl + kk) <= (uint32_t)rb.span || js + kk == 0;
        x[r] = ok ? x[r] : kMaskedX;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pa[0][e] = (__bf16)silu2(x[e]);
      pa[1][e] = (__bf16)silu2(x[8 + e]);
    }
  };

  // ---- item prologue -------------------------------------------------------
  // Steps 0 and 1 (blocks 0-3, ring slots 0-3) go out first, then the row
  // times and the query tile, staged into ring slots 6 and 7 (32 KB: rows of
  // row group wq at slot 6 + wq / 2, half wq % 2); wave w copies the first
  // and wave w + 4 the second half of its rows' 8 KB.
  issue_step(0);
  issue_step(1);
  int q_fetch;
  if (queue && tid == 0) q_fetch = atomicAdd(const_cast<int32_t*>(a.hdr) + wkq.ctr, 1);
  int64_t ti64 = 0;
  if constexpr (TIME) {
    tbase = a.timestamps[seq0 + i0];
    ti64 = a.timestamps[seq0 + min(i, i1 - 1)];
  }
  const uint32_t q_lds = lds_off(ring[6 + (wq >> 1)].k) + (uint32_t)((wq & 1) * kPPRows * KROW);
  if (wave_rows && !alpha_zero) {
    int ql = lane;
    asm volatile("" : "+v"(ql));
    const uint64_t qb = uni_ptr(reinterpret_cast<const char*>(a.q) +
                                ((int64_t)(seq0 + i0) * a.ld_q + (int64_t)h * 128) * 2);
    const uint32_t ldq_b = (uint32_t)(a.ld_q * 2);
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) {
      const int n8 = 4 * g + nn;
      const int m = 64 * n8 + ql, r = m / KCH;
      const int row = min(wr0 + r, i1 - 1) - i0;
      lds_copy16_nt(qb, (uint32_t)row * ldq_b + 16u * (uint32_t)((m % KCH) ^ C::kswz(r)),
                    q_lds + 1024u * (uint32_t)n8);
    }
  }
  wait_vmem<0>();
  asm volatile("" : "+v"(q_fetch));
  if (queue && tid == 0) {
    s_qnext[q_item & 1] = wkq.first + wkq.n + q_fetch;
    if (q_fetch == wkq.end - wkq.first - 1) const_cast<int32_t*>(a.hdr)[wkq.ctr] = 0;
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
  stage_barrier();   // query tile, steps 0-1 and the time tables are in LDS
  {
    const int ln = opaque_lane();
    const int ql32 = ln & 31, qhh = ln >> 5;
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      const bf16x8 z = {};
      qf[c] = (row_valid && !alpha_zero)
                  ? lds_ld<bf16x8>(q_lds + ql32 * KROW + 16 * ((2 * c + qhh) ^ C::kswz(ql32)))
                  : z;
    }
  }

  // Epilogue staging: U rows (and then the output) of wave w's column half
  // in slot (2S + g) & 7 at 4 KB * wq, row r at 128 r with its eight 16-byte
  // chunks XOR-swizzled by r & 7; slots (2S + 2 + wq) & 7 carry the pairs'
  // exchange of partial O.  None of these slots is read by the last two steps.
  const bool ln = a.epilogue == 0;
  const uint32_t e_lds = lds_off(ring[(2 * S + g) & (kRing - 1)].k) + 4096u * (uint32_t)wq;
  auto issue_u = [&]() __attribute__((always_inline)) -> int {
    if (!(ln && wave_rows)) return 0;
    int ul = lane;
    asm volatile("" : "+v"(ul));
    const uint64_t ub = uni_ptr(reinterpret_cast<const char*>(a.u) +
                                ((int64_t)(seq0 + i0) * a.ld_u + (int64_t)h * 128 + 64 * g) * 2);
    const uint32_t ldu_b = (uint32_t)(a.ld_u * 2);
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) {
      const int m = 64 * nn + ul, r = m >> 3;
      const int row = min(wr0 + r, i1 - 1) - i0;
      lds_copy16_nt(ub, (uint32_t)row * ldu_b + 16u * (uint32_t)((m & 7) ^ (r & 7)),
                    e_lds + 1024u * (uint32_t)nn);
    }
    return 4;
  };

  // ---- steps ---------------------------------------------------------------
  for (int st = 0; st < S; ++st) {
    issue_step(st + kPPAhead);
    const int ucnt = (st == S - 2) ? issue_u() : 0;
    // phase X
    if constexpr (TIME) {
      if (wave < 2 && 2 * st + wave < n) finish_ts(kt_lo + 2 * st + wave);
    }
    if (g == 0) mfma_phase(st);
    else valu_phase(st - 1);
    stage_barrier();
    // phase Y
    if (g == 0) valu_phase(st);
    else mfma_phase(st);
    // the next step's blocks have landed (this wave's copies; the barrier
    // makes everyone's visible)
    wait_vmem_n(step_copies(st + kPPAhead) + ucnt);
    stage_barrier();
  }

  // ---- partner exchange: wave w keeps columns 0-63, wave w + 4 64-127 -----
  // Afterwards o[j] holds column 64 g + 32 (j / 16) + 8 (r / 4) + 4 hh + r % 4
  // (r = j % 16) of row i.
  float o[32];
  {
    const uint32_t x_lds = lds_off(ring[(2 * S + 2 + wq) & (kRing - 1)].k);
    // outgoing half: group 0 sends blocks 2-3, group 1 sends blocks 0-1
    const uint32_t out_b = x_lds + (uint32_t)g * 8192u + 16u * (uint32_t)lane;
    const uint32_t in_b = x_lds + (uint32_t)(1 - g) * 8192u + 16u * (uint32_t)lane;
    auto xchg = [&](auto half) __attribute__((always_inline)) {
      constexpr int keep = decltype(half)::value;   // 0: keep blocks 0-1
      constexpr int send = 1 - keep;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        floatx4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = acc[2 * send + (j >> 2)][4 * (j & 3) + e];
        lds_st<floatx4>(out_b + 1024u * (uint32_t)j, o4);
      }
      stage_barrier();
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const floatx4 i4 = lds_ld<floatx4>(in_b + 1024u * (uint32_t)j);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[4 * j + e] = acc[2 * keep + (j >> 2)][4 * (j & 3) + e] + i4[e];
      }
    };
    if (g == 0) xchg(B0{});
    else xchg(B1{});
  }

  // ---- chunk of a split item: publish the partial output; the chunk that
  // arrives last adds all partials in chunk order and runs the epilogue ----
  const int n_chunks = ch.w & 0x7fff;
  bool finish = true;
  if (n_chunks > 1) {
    // slot layout: [wave][j / 2][lane] x (2 floats)
    auto slot = [&](int c) __attribute__((always_inline)) {
      return reinterpret_cast<uint64_t*>(a.partials + (int64_t)(ch.z + c) * a.slot_floats) +
             wave * 16 * 64 + lane;
    };
    uint64_t* own = slot((ch.w >> 16) & 0x7fff);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint64_t w2 = (uint64_t)__float_as_uint(o[2 * j]) |
                          ((uint64_t)__float_as_uint(o[2 * j + 1]) << 32);
      __hip_atomic_store(own + 64 * j, w2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_vmem<0>();
    __syncthreads();
    if (tid == 0)
      s_ticket = __hip_atomic_fetch_add(a.counters + ch.z, 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    finish = s_ticket == n_chunks - 1;
    if (finish) {
      if (tid == 0) a.counters[ch.z] = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) o[j] = 0.0f;
      for (int c = 0; c < n_chunks; ++c) {
        const uint64_t* src = slot(c);
        uint64_t p[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          p[j] = __hip_atomic_load(src + 64 * j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          o[2 * j] += __uint_as_float((uint32_t)p[j]);
          o[2 * j + 1] += __uint_as_float((uint32_t)(p[j] >> 32));
        }
      }
    }
  }

  if (finish) {
    // ---- epilogue: ln(2)/n_scale, LayerNorm over d_v, * U, store ---------
    const float osc = a.out_scale;
    int el = lane;
    asm volatile("" : "+v"(el));
    {
      const int gg = g;
#pragma unroll
      for (int j = 0; j < 32; ++j) o[j] *= osc;
      if (a.out_raw != nullptr && row_valid) {
        char* rrow = reinterpret_cast<char*>(a.out_raw) +
                     ((int64_t)(seq0 + i) * a.ld_raw + (int64_t)h * 128 + 64 * gg) * 2;
#pragma unroll
        for (int j4 = 0; j4 < 8; ++j4) {
          const int d0 = 32 * (j4 >> 2) + 8 * (j4 & 3) + 4 * hh;
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (__bf16)o[4 * j4 + e];
          *reinterpret_cast<bf16x4*>(rrow + 2 * d0) = o;
        }
      }
      float mean = 0.0f, rstd = 1.0f;
      if (ln) {
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) sum += o[j];
        sum += __shfl_xor(sum, 32, 64);
        if (hh == 0) s_red[0][wave][l32] = sum;
        stage_barrier();
        mean = (sum + s_red[0][wave ^ 4][l32]) * (1.0f / 128);
        float sq = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const float c = o[j] - mean;
          sq += c * c;
        }
        sq += __shfl_xor(sq, 32, 64);
        if (hh == 0) s_red[1][wave][l32] = sq;
        stage_barrier();
        rstd = rsqrtf((sq + s_red[1][wave ^ 4][l32]) * (1.0f / 128) + a.ln_eps);
      }
      if (wave_rows) {
        if (ln) wait_vmem<0>();   // this wave's U rows have landed
#pragma unroll
        for (int j4 = 0; j4 < 8; ++j4) {
          const int d0 = 32 * (j4 >> 2) + 8 * (j4 & 3) + 4 * hh;   // within the half
          const uint32_t off = e_lds + (uint32_t)(l32 * 128) +
                               16u * (uint32_t)((d0 >> 3) ^ (l32 & 7)) + 2u * (d0 & 7);
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = o[4 * j4 + e];
          if (ln) {
            const bf16x4 uu = lds_ld<bf16x4>(off);
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = (y[e] - mean) * rstd * (float)uu[e];
          }
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (__bf16)y[e];
          lds_st<bf16x4>(off, o);
        }
        // whole 128-byte row halves out: lane l of store nn writes physical
        // chunk (64 nn + l) % 8 of row (64 nn + l) / 8
        char* obase = reinterpret_cast<char*>(
            uni_ptr(reinterpret_cast<char*>(a.out) +
                    ((int64_t)(seq0 + wr0) * a.ld_out + (int64_t)h * 128 + 64 * gg) * 2));
        const uint32_t ldo_b = (uint32_t)(a.ld_out * 2);
#pragma unroll
        for (int nn = 0; nn < 4; ++nn) {
          const int m = 64 * nn + el, r = m >> 3;
          const uintx4 w4 = lds_ld<uintx4>(e_lds + 16u * (uint32_t)m);
          if (wr0 + r < i1)
            __builtin_nontemporal_store(
                w4, reinterpret_cast<uintx4*>(obase + ((uint32_t)r * ldo_b +
                                                       16u * (uint32_t)((m & 7) ^ (r & 7)))));
        }
      }
    }
  } else if (ln && wave_rows) {
    wait_vmem<0>();   // U rows in flight into LDS land before the slot is reused
  }
  // The LDS of this item is free again once every wave is here.
  stage_barrier();
  }  // units
  }  // planned workgroups
}

template <int POSM, bool TIME>
static hipError_t launch_pp_one(const AttnArgs& a, int n_wg, hipStream_t stream,
                                hipEvent_t start, hipEvent_t stop) {
  auto kern = hstu_attn_fwd_pp_kernel<POSM, TIME>;
  if (start || stop)
    hipExtLaunchKernelGGL(kern, dim3((unsigned)n_wg), dim3(kPPThreads), 0, stream, start, stop,
                          0, a);
  else
    hipLaunchKernelGGL(kern, dim3((unsigned)n_wg), dim3(kPPThreads), 0, stream, a);
  return hipGetLastError();
}

template <int POSM, bool TIME>
static int pp_blocks_per_cu() {
  auto kern = hstu_attn_fwd_pp_kernel<POSM, TIME>;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, kPPThreads, 0) != hipSuccess)
    return -1;
  return nb;
}

bool attn_pp_supported(int dtype, int d_qk, int d_v) {
  return dtype == 1 && d_qk == 128 && d_v == 128;
}

int attn_pp_grid(int pos_len, int time_len, bool clamp) {
  const bool pos = pos_len > 0, tim = time_len > 0;
  int bpc;
  if (pos && clamp && tim) bpc = pp_blocks_per_cu<2, true>();
  else if (pos && clamp) bpc = pp_blocks_per_cu<2, false>();
  else if (pos && tim) bpc = pp_blocks_per_cu<1, true>();
  else if (pos) bpc = pp_blocks_per_cu<1, false>();
  else if (tim) bpc = pp_blocks_per_cu<0, true>();
  else bpc = pp_blocks_per_cu<0, false>();
  if (bpc <= 0) return -1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  return cus * bpc;
}

hipError_t launch_attn_pp(const AttnArgs& a, int n_wg, hipStream_t stream, hipEvent_t t0,
                          hipEvent_t t1) {
  const bool pos = a.pos_len > 0, tim = a.time_len > 0, cl = a.pos_clamp != 0;
  if (pos && cl && tim) return launch_pp_one<2, true>(a, n_wg, stream, t0, t1);
  if (pos && cl) return launch_pp_one<2, false>(a, n_wg, stream, t0, t1);
  if (pos && tim) return launch_pp_one<1, true>(a, n_wg, stream, t0, t1);
  if (pos) return launch_pp_one<1, false>(a, n_wg, stream, t0, t1);
  if (tim) return launch_pp_one<0, true>(a, n_wg, stream, t0, t1);
  return launch_pp_one<0, false>(a, n_wg, stream, t0, t1);
}

}  // namespace hstu
