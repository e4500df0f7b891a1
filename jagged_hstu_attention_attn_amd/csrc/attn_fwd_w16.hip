// attn_fwd_w16.hip -- gfx950 jagged HSTU attention forward, bf16 with
// d_qk = d_v = 128: sixteen query rows per wave, four waves per SIMD.
//
// A wave of this GPU issues one vector instruction every ~8 cycles when it
// runs alone on its SIMD; the SIMD reaches its vector throughput only with
// several waves in flight.  Each 32-key block costs a wave ~60 vector
// instructions of bias, SiLU and packing, so the kernel keeps the per-wave
// register footprint under 128 (16 rows: O 32 registers, Q 16, scores 8) and
// runs 8 waves per workgroup and two workgroups per CU -- four waves per
// SIMD, whose dependent chains (LDS reads -> score MFMAs -> SiLU ->
// aggregation MFMAs) interleave.
//
// Work items are the scheduler's units (sequence, head, 128-row query tile,
// key-tile range), as for the other forward kernels; wave w owns rows
// i0 + 16w .. i0 + 16w + 15.  Keys are staged 32 at a time in four LDS
// buffers, copied from HBM straight into LDS (global_load_lds); a step
// computes two key blocks while the next two are copied, one barrier per
// step.  Per 32-key block and wave, with v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T + C       two 16-key x 16-row tiles; lane l holds keys
//                         16 t + 4 (l / 16) + i (t = 0, 1; i = 0..3) of row
//                         l % 16, the accumulator starting at the position bias
//   x   = am S + time bias, mask select, A = SiLU(x)     (8 values per lane)
//   O^T += V^T A^T        eight 16-column tiles of d_v; the 8 SiLU values of
//                         a lane are its B operand as they stand (contraction
//                         slot 8 (l / 16) + j is key 4 (l / 16) + j for j < 4
//                         and 16 + 4 (l / 16) + j - 4 otherwise), and V^T
//                         comes in the same key order from two transposed
//                         LDS reads (ds_read_b64_tr_b16) per tile.
// The epilogue scales by ln(2)/n_scale, takes LayerNorm over d_v per (token,
// head) -- a row's 128 columns sit in the four lanes l % 16 + 16 g -- gates
// by U and stores whole rows through LDS.
//
// Method: pointwise SiLU aggregation with position/time bias, zeroing after
// the nonlinearity, Norm then U gating ("HSTU tensor by tensor: SiLU
// aggregation, temporal bias and gating", sections "SiLU aggregation
// coefficients are not probabilities", "Do not copy softmax masking
// mechanically", "Relative time adds information content similarity lacks",
// "Similar shape, different aggregation").
#include <hip/hip_ext.h>

#include <cstddef>

#include "attn_common.hpp"

namespace hstu {

constexpr int kW16Waves = 8;
constexpr int kW16Threads = kW16Waves * 64;
constexpr int kW16Rows = 16;        // query rows per wave
constexpr int kW16Stages = 4;       // LDS buffers of the key/value pipeline
static_assert(kBM == kW16Waves * kW16Rows, "eight row groups of 16 per item");
static_assert(kBN == 32, "a key block is two 16-key score tiles");

typedef float floatx4v __attribute__((ext_vector_type(4)));

template <bool CLAMP>
struct W16Stage {
  char k[kBN * 256];            // keys: row j at 256 j, chunk c at (c ^ (j & 15))
  char v[kBN * 256];            // values: row j at 256 j, chunk c at (c ^ 2 (j & 7))
  float diag[kDiagCopies * 64]; // position bias of i - j = i0 - j0 + 127 - f, at f
  int64_t ts64[kBN];            // raw key timestamps
  uint32_t ts32[kBN];           // key timestamps relative to the item's base
  uint32_t tmin, tmax;          // range of ts32 over the valid keys
  int tbad;                     // some key needs the 64-bit time path
  int pad_;                     // (tmin .. pad_: one 16-byte read)
  float cpos[CLAMP ? 64 : 4];   // clamped-position bias of key (lane % 32): n_h - j
};

static_assert(offsetof(W16Stage<false>, tmin) % 16 == 0 && offsetof(W16Stage<true>, tmin) % 16 == 0,
              "the key-time range is one aligned 16-byte read");

// Physical 16-byte chunk of logical chunk c in staged row `row`.
__device__ inline int w16_kchunk(int c, int row) { return c ^ (row & 15); }
__device__ inline int w16_vchunk(int c, int row) { return c ^ (2 * (row & 7)); }

// POSM: 0 = no position bias, 1 = position bias of |i - j|, 2 = of the
// clamped positions |p_i - p_j| (candidate rows take it from cpos).
// TR: the transposed walk of the backward's value gradient, dV_j = sum_i
// a_ij dO_i: a tile's "rows" are keys j (their k rows in place of q), the
// streamed blocks are the query rows i that can see them (q rows as keys,
// dO rows as values), each lane's allowed partners are the key's column of
// the mask (col_bounds) and the epilogue is none; the position and time
// biases depend on |i - j| and |t_i - t_j| only, so they are unchanged.
template <int POSM, bool TIME, bool TR>
__global__ __launch_bounds__(kW16Threads) __attribute__((amdgpu_waves_per_eu(4))) void
hstu_attn_fwd_w16_kernel(AttnArgs a) {
  constexpr bool POS = POSM != 0;
  constexpr bool clamp = POSM == 2;
  static_assert(!(TR && clamp), "the transposed walk takes the plain position bias");
  // the allowed partners of this lane's row (of its key, transposed)
  auto bounds = [](const SeqGeom& g, int x) __attribute__((always_inline)) {
    return TR ? col_bounds(g, x) : row_bounds(g, x);
  };
  using SB = W16Stage<clamp>;
  constexpr int ROWB = 256;          // staged row bytes (128 bf16)
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  using B3 = std::integral_constant<int, 3>;

  // 256-byte aligned stage buffers: the K/V read offsets XOR into bits 5-7
  // of a lane's in-buffer offset, which the buffer base never touches
  __shared__ __align__(256) SB st0, st1, st2, st3;
  __shared__ TimeTables tt;
  __shared__ int s_ticket;
  __shared__ int s_qnext[2];
  auto stage = [&](auto bufc) __attribute__((always_inline)) -> SB& {
    constexpr int b = decltype(bufc)::value % kW16Stages;
    if constexpr (b == 0) return st0;
    else if constexpr (b == 1) return st1;
    else if constexpr (b == 2) return st2;
    else return st3;
  };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int P = a.pos_len;
  const int H = a.num_heads;
  const float alpha2 = a.alpha * kLog2e;
  const bool alpha_zero = alpha2 == 0.0f;
  const float am = alpha_zero ? 1.0f : alpha2;   // x2 = am * S + time
  const float pscale = kLog2e / am;              // position bias in accumulator units
  const uint32_t ldk_b = (uint32_t)(a.ld_k * 2), ldv_b = (uint32_t)(a.ld_v * 2);
  // copies of one stage: wave w copies 1 KB chunk w of the keys and of the
  // values (rows 4w .. 4w + 3); the bias inputs go to "role" waves among
  // waves 0-3, which a stage in an odd buffer maps to wave 3 - role (the two
  // stages of a step spread that work over the four): roles 1-3 gather the
  // position-bias diagonal (part role - 1), role 0 the raw timestamps and
  // the clamped-position bias.  Waves w and w + 4 share a SIMD, whose
  // arbiter favours the older wave, so waves 4-7 compute more slowly and
  // reach each barrier last; the extra copies go to the waves that wait.
  constexpr int kTsW = 0, kCposW = 0, kDiagW0 = 1;
  auto role_wave = [&](auto bufc) __attribute__((always_inline)) {
    return ((decltype(bufc)::value & 1) && wave < 4) ? 3 - wave : wave;
  };
  static_assert(kDiagW0 + kDiagCopies <= kW16Waves, "enough waves for the bias copies");

  // Per-lane values are derived from an opaque lane index inside the loops
  // (the compiler cannot hoist them): recomputing costs a few vector
  // instructions, keeping them live would cost the registers that let four
  // waves share a SIMD.
  auto opaque_lane = [&]() __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    return ln;
  };

  // This lane's K/V copy offsets within a stage of whole rows: row 4w + l/16
  // of the block, swizzled chunk of l % 16 (kernel constants; the last block
  // of a sequence clamps its rows instead).
  const int cp_row = 4 * wave + (lane >> 4);
  const uint32_t ko_full = (uint32_t)cp_row * ldk_b + 16u * (uint32_t)w16_kchunk(lane & 15, cp_row);
  const uint32_t vo_full = (uint32_t)cp_row * ldv_b + 16u * (uint32_t)w16_vchunk(lane & 15, cp_row);

  if constexpr (TIME) {
    const int Tt = a.time_len;
    if (tid < 32) tt.trev[tid] = kLog2e * a.time_table[min(31 - tid, Tt - 1)];
    if (tid < 64) tt.tful[tid] = kLog2e * a.time_table[min(tid, Tt - 1)];
  }

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
  tile_range(geo, i0, i1, TR, jlo, jhi);
  const int kt_lo = max(jlo / kBN, ch.x), kt_hi = min(jhi / kBN, ch.y);
  // Key blocks are walked from a rotation of [kt_lo, kt_hi]: no softmax, so
  // the order is free.  Under a window a tile's range starts four blocks
  // after its predecessor's, and walking in plain order would have the next
  // tile read a block four steps later, after the workgroups of an L2 have
  // read as much again as that L2 holds.  Walking so that step s takes the
  // block kt = s (mod nk) lets the neighbouring tiles of one L2, whose
  // ranges have the same length, read each block at about the same time.
  const int nk = kt_hi - kt_lo + 1;
  const int rot = (geo.W > 0 && nk > 1) ? (nk - kt_lo % nk) % nk : 0;
  auto blk = [&](int s) __attribute__((always_inline)) {
    const int t = s + rot;
    return kt_lo + (t >= nk ? t - nk : t);
  };

  // ---- per-lane query row and the wave's uniform key bounds --------------
  const int wr0 = i0 + wave * kW16Rows;
  const int i = wr0 + (lane & 15);
  const bool row_valid = i < i1;
  const bool wave_rows = wr0 < i1;
  int w_jmin, w_jmax, w_lomax, w_himin;
  {
    const RowBounds rb = row_valid ? bounds(geo, i) : RowBounds{kEmptyLo, 0, -1};
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
  const bool w_cand = clamp && wave_rows && wr0 + kW16Rows - 1 >= geo.n_h;
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

  // Copy key tile kt into stage buffer `bufc`.  Rows past the end of the
  // sequence repeat its last row (finite values whose scores are masked).
  auto issue_stage = [&](auto bufc, int kt) __attribute__((always_inline)) {
    SB& sb = stage(bufc);
    const int j0 = kt * kBN;
    const int ln = opaque_lane();
    uint32_t ko = ko_full, vo = vo_full;
    if (j0 + kBN > L) {   // the sequence's last block: rows past its end repeat row L - 1
      const int row = 4 * wave + (ln >> 4);
      const uint32_t r = (uint32_t)min(row, L - 1 - j0);
      ko = r * ldk_b + 16u * (uint32_t)w16_kchunk(ln & 15, row);
      vo = r * ldv_b + 16u * (uint32_t)w16_vchunk(ln & 15, row);
    }
    const uint64_t kb = kseq + (uint64_t)j0 * ldk_b, vb = vseq + (uint64_t)j0 * ldv_b;
    if (kv_nt) {
      lds_copy16_nt(kb, ko, lds_off(sb.k) + 1024u * (uint32_t)wave);
      lds_copy16_nt(vb, vo, lds_off(sb.v) + 1024u * (uint32_t)wave);
    } else {
      lds_copy16(kb, ko, lds_off(sb.k) + 1024u * (uint32_t)wave);
      lds_copy16(vb, vo, lds_off(sb.v) + 1024u * (uint32_t)wave);
    }
    const int rw = role_wave(bufc);
    if constexpr (POS) {
      if (rw >= kDiagW0 && rw < kDiagW0 + kDiagCopies) {   // part rw - kDiagW0 of the diagonal
        const int p = rw - kDiagW0;
        const int d = i0 - j0 + (kBM - 1) - (64 * p + ln);
        const int ix = min(d < 0 ? -d : d, P - 1);
        lds_copy4(pos_base, 4u * (uint32_t)ix, lds_off(sb.diag) + 256u * (uint32_t)p);
      }
      if (clamp && rw == kCposW) {   // bias of n_h - j (0 for candidate keys)
        const int d = geo.n_h - (j0 + (ln & (kBN - 1)));
        const int ix = min(d > 0 ? d : 0, P - 1);
        lds_copy4(pos_base, 4u * (uint32_t)ix, lds_off(sb.cpos));
      }
    }
    if constexpr (TIME) {
      if (rw == kTsW) {
        const int j = min(j0 + (ln >> 1), L - 1);
        lds_copy4(ts_base, 8u * (uint32_t)j + 4u * (uint32_t)(ln & 1), lds_off(sb.ts64));
      }
    }
  };

  // row times (loaded in the prologue)
  int64_t tbase = 0;
  uint32_t ti32 = uint32_t(kT32Range);
  bool w_t_ok = true;
  uint32_t w_tmin = 0, w_tmax = 0;

  // Once this wave's own copies of stage kt have landed: rescale the
  // position-bias values it gathered; in the timestamp wave, form the 32-bit
  // key times, their range and whether any key needs the 64-bit path.
  auto finish_stage = [&](auto bufc, int kt) __attribute__((always_inline)) {
    SB& sb = stage(bufc);
    const int ln = opaque_lane();
    const int rw = role_wave(bufc);
    if constexpr (POS) {
      if (rw >= kDiagW0 && rw < kDiagW0 + kDiagCopies) {
        const int e = 64 * (rw - kDiagW0) + ln;
        if (e < kDiag) sb.diag[e] *= pscale;
      }
      if (clamp && rw == kCposW) sb.cpos[ln] *= pscale;
    }
    if constexpr (TIME) {
      if (rw == kTsW) {
        const int kl = ln & (kBN - 1);
        const int64_t tj = sb.ts64[kl];
        const int64_t rel = tj - tbase;
        const bool ok = rel > -kT32Range && rel < kT32Range;
        const uint32_t t32 = ok ? uint32_t(rel + kT32Range) : 0u;
        const int nvalid = min(kBN, L - kt * kBN);
        if (ln < kBN) sb.ts32[kl] = t32;
        const bool bad = __ballot(!ok) != 0;
        const uint32_t nxt = (uint32_t)__builtin_amdgcn_update_dpp(
            (int)t32, (int)t32, 0x130, 0xf, 0xf, false);   // lane l gets lane l+1
        const bool desc = ln + 1 < nvalid && nxt < t32;
        const bool sorted = __ballot(desc) == 0;
        const uint32_t first = (uint32_t)__builtin_amdgcn_readlane((int)t32, 0);
        const uint32_t last = (uint32_t)__builtin_amdgcn_readlane((int)t32, nvalid - 1);
        if (ln == 0) {
          sb.tmin = sorted ? first : 0u;
          sb.tmax = sorted ? last : 0xffffffffu;
          sb.tbad = bad;
        }
      }
    }
  };

  // Q operands (B of S^T = K Q^T): qf[c] holds d = 32c + 8 (l / 16) .. + 7
  // of row l % 16; O^T accumulators: acc[t][i] is d = 16 t + 4 (l / 16) + i
  bf16x8 qf[4];
  floatx4v acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[t][e] = 0.0f;

  // The buckets the (row, key) time gaps of this wave and a block can fall
  // in, from the block's key-time range `kr` (tmin, tmax, tbad as the stage
  // holds them, loaded with the block's first LDS reads) and the wave's
  // row-time range: the gap of every valid pair lies between the two ranges'
  // smallest and largest distance, so its clz(1 + dt) lies in [z1, z0].
  // False when some time needs the 64-bit path.  Uniform values throughout:
  // the distances between the ranges are written as max - b (scalar ALU)
  // rather than saturating differences (vector ALU).
  auto time_span = [&](const uint4& kr, int& z0, int& z1) __attribute__((always_inline)) -> bool {
    if (!w_t_ok || uni((int)kr.z) != 0) return false;
    const uint32_t kmin = (uint32_t)uni((int)kr.x), kmax = (uint32_t)uni((int)kr.y);
    const uint32_t wmin = (uint32_t)uni((int)w_tmin), wmax = (uint32_t)uni((int)w_tmax);
    // ranges [wmin, wmax] and [kmin, kmax]: at most one of the two gaps is positive
    const uint32_t dmin = (max(wmin, kmax) - kmax) + (max(kmin, wmax) - wmax);
    const uint32_t dmax = max(max(wmax, kmin) - kmin, max(kmax, wmin) - wmin);
    z0 = __builtin_clz(dmin + 1u);
    z1 = __builtin_clz(dmax + 1u);
    return true;
  };
  auto trev_u = [&](int z) __attribute__((always_inline)) -> float {   // a uniform table entry
    return __builtin_bit_cast(float, uni(__builtin_bit_cast(int, tt.trev[z])));
  };

  // One 32-key block from stage buffer `sb`.  The lane parts of its LDS
  // addresses are loop invariants (the stage's base is a constant offset).
  auto block = [&](SB& sb, int kt) __attribute__((always_inline)) {
    const int jb = kt * kBN;
    const int l16 = lane & 15, g4 = lane >> 4;
    // ---- score start (position bias) and the first half of the K operands
    floatx4v s0, s1;
    uint4 kr = {0u, 0u, 0u, 0u};   // key-time range of the block (TIME)
    if constexpr (TIME) kr = *reinterpret_cast<const uint4*>(&sb.tmin);
    const int dbase = (kBM - 1) - kW16Rows * wave - l16 + 4 * g4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (POS) {
        s0[e] = sb.diag[dbase + e];
        s1[e] = sb.diag[dbase + 16 + e];
      } else {
        s0[e] = 0.0f;
        s1[e] = 0.0f;
      }
    }
    if constexpr (clamp) {
      if (w_cand) {   // candidate rows: bias of the clamped positions
        const bool cr = i >= geo.n_h;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float c0 = sb.cpos[4 * g4 + e], c1 = sb.cpos[16 + 4 * g4 + e];
          s0[e] = cr ? c0 : s0[e];
          s1[e] = cr ? c1 : s1[e];
        }
      }
    }
    // K operand of (tile tk, step c): key 16 tk + l16, logical chunk 4c + g4,
    // physical chunk (4c + g4) ^ l16 = 4 (c ^ (l16 >> 2)) + (g4 ^ (l16 & 3)):
    // byte offset ka ^ 64c with ka below (its bits 6-7 hold l16 >> 2; the
    // stage base is 256-byte aligned, so it adds as an immediate offset)
    const uint32_t ka = (uint32_t)(l16 * ROWB + 16 * (g4 ^ (l16 & 3)) + 64 * (l16 >> 2));
    auto kread = [&](int tk, int c) __attribute__((always_inline)) {
      return lds_ld<bf16x8>(lds_off(sb.k) + (uint32_t)(tk * 16 * ROWB) + (ka ^ (64u * c)));
    };
    bf16x8 k0[2], k1[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      k0[c] = kread(0, c);
      k1[c] = kread(1, c);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0[c], qf[c], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1[c], qf[c], s1, 0, 0, 0);
    }
#pragma unroll
    for (int c = 2; c < 4; ++c) {
      k0[c - 2] = kread(0, c);
      k1[c - 2] = kread(1, c);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 2; c < 4; ++c) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0[c - 2], qf[c], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1[c - 2], qf[c], s1, 0, 0, 0);
    }

    // V^T operands of d_v tile t: in each 16-lane group (g4) lane 4e + q
    // addresses key row 4 g4 + e (then 16 + 4 g4 + e), columns 16 t + 4q ..
    // + 3; lane l16 receives column 16 t + l16 of the four rows
    // physical chunk (2t + (q >> 1)) ^ 2 (vrow & 7) = 2 (t ^ (vrow & 7)) +
    // (q >> 1): byte offset va ^ 32t (bits 5-7 of va hold vrow & 7)
    const int er = l16 >> 2, q = l16 & 3;
    const int vrow = 4 * g4 + er;
    const uint32_t va = (uint32_t)(vrow * ROWB + 8 * (q & 1) + 16 * (q >> 1) + 32 * (vrow & 7));
    auto vread = [&](int t) __attribute__((always_inline)) {
      const uint32_t off = lds_off(sb.v) + (va ^ (32u * t));
      const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr4(off));
      const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr4(off + 16 * ROWB));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 vop[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) vop[t] = vread(t);
    __builtin_amdgcn_sched_barrier(0);

    // ---- x2 = am * S + log2e * time ----
    float x[8];
    if constexpr (TIME) {
      int z0 = 0, z1 = 0;
      const bool t32 = time_span(kr, z0, z1);
      if (t32 && z0 == z1) {   // one bucket for the whole block
        const float tb = trev_u(z0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = fmaf(s0[e], am, tb);
          x[4 + e] = fmaf(s1[e], am, tb);
        }
      } else if (t32 && z0 == z1 + 1) {
        // two adjacent buckets: a gap + 1 from 2^(31 - z1) on is in the upper one
        const float tlo = trev_u(z0), thi = trev_u(z1);
        const uint32_t thr = 1u << (31 - z1);
#pragma unroll
        for (int tk = 0; tk < 2; ++tk) {
          const uint4 t4 = *reinterpret_cast<const uint4*>(&sb.ts32[16 * tk + 4 * (opaque_lane() >> 4)]);
          const uint32_t tv[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t d1 = (ti32 > tv[e] ? ti32 - tv[e] : tv[e] - ti32) + 1u;
            x[4 * tk + e] = fmaf(tk ? s1[e] : s0[e], am, d1 >= thr ? thi : tlo);
          }
        }
      } else if (t32) {
#pragma unroll
        for (int tk = 0; tk < 2; ++tk) {
          const uint4 t4 = *reinterpret_cast<const uint4*>(&sb.ts32[16 * tk + 4 * (opaque_lane() >> 4)]);
          const uint32_t tv[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t d1 = (ti32 > tv[e] ? ti32 - tv[e] : tv[e] - ti32) + 1u;
            x[4 * tk + e] = fmaf(tk ? s1[e] : s0[e], am, tt.trev[__builtin_clz(d1)]);
          }
        }
      } else {
        // times too far apart for 32 bits (rare): 64-bit differences
        const int64_t t_i = row_valid ? a.timestamps[seq0 + i] : tbase;
#pragma unroll
        for (int tk = 0; tk < 2; ++tk)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t tj = sb.ts64[16 * tk + 4 * g4 + e];
            const uint64_t dt = t_i >= tj ? uint64_t(t_i) - uint64_t(tj)
                                          : uint64_t(tj) - uint64_t(t_i);
            x[4 * tk + e] = fmaf(tk ? s1[e] : s0[e], am,
                                 tt.tful[63 - __builtin_clzll(dt + 1u)]);
          }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = s0[e] * am;
        x[4 + e] = s1[e] * am;
      }
    }
    // ---- illegal pairs: an argument whose SiLU is exactly -0 ----
    if (!is_full(kt)) {
      const RowBounds rb = row_valid ? bounds(geo, i) : RowBounds{kEmptyLo, 0, -1};
      int jl = jb + 4 * g4 - rb.lo, js = jb + 4 * g4 - rb.self_j;
      asm volatile("" : "+v"(jl), "+v"(js));
#pragma unroll
      for (int tk = 0; tk < 2; ++tk)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kk = 16 * tk + e;
          const bool ok = (uint32_t)(jl + kk) <= (uint32_t)rb.span || js + kk == 0;
          x[4 * tk + e] = ok ? x[4 * tk + e] : kMaskedX;
        }
    }
    bf16x8 pa;
#pragma unroll
    for (int e = 0; e < 8; ++e) pa[e] = (__bf16)silu2(x[e]);

    // ---- O^T[d][i] += sum_j V[j][d] A[i][j] ----
#pragma unroll
    for (int t = 0; t < 4; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[t], pa, acc[t], 0, 0, 0);
#pragma unroll
    for (int t = 4; t < 8; ++t) vop[t - 4] = vread(t);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 4; t < 8; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[t - 4], pa, acc[t], 0, 0, 0);
  };

  // ---- item prologue -------------------------------------------------------
  issue_stage(B0{}, blk(0));
  if (nk > 1) issue_stage(B1{}, blk(1));
  int q_fetch;
  if (queue && tid == 0) q_fetch = atomicAdd(const_cast<int32_t*>(a.hdr) + wkq.ctr, 1);
  int64_t ti64 = 0;
  if constexpr (TIME) {
    tbase = a.timestamps[seq0 + i0];
    ti64 = a.timestamps[seq0 + min(i, i1 - 1)];
  }
  // Query tile: each wave copies its 16 rows (4 KB) into stage buffers 2 and
  // 3, which are idle in the prologue (rows of waves 0-3 in buffer 2, 4-7 in
  // buffer 3), then reads its MFMA operands from there.
  const uint32_t q_lds =
      lds_off(wave < 4 ? st2.k : st3.k) + (uint32_t)((wave & 3) * kW16Rows * ROWB);
  if (wave_rows && !alpha_zero) {
    const int ql = opaque_lane();
    const uint64_t qb = uni_ptr(reinterpret_cast<const char*>(a.q) +
                                ((int64_t)(seq0 + i0) * a.ld_q + (int64_t)h * 128) * 2);
    const uint32_t ldq_b = (uint32_t)(a.ld_q * 2);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int m = 64 * n + ql, r = m >> 4;
      const int row = min(wr0 + r, i1 - 1) - i0;
      lds_copy16_nt(qb, (uint32_t)row * ldq_b + 16u * (uint32_t)w16_kchunk(m & 15, r),
                    q_lds + 1024u * (uint32_t)n);
    }
  }
  wait_vmem<0>();
  asm volatile("" : "+v"(q_fetch));
  if (queue && tid == 0) {
    s_qnext[q_item & 1] = wkq.first + wkq.n + q_fetch;
    if (q_fetch == wkq.end - wkq.first - 1) const_cast<int32_t*>(a.hdr)[wkq.ctr] = 0;
  }
  {
    const int ln = opaque_lane();
    const int l16 = ln & 15, g4 = ln >> 4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 z = {};
      qf[c] = (row_valid && !alpha_zero)
                  ? lds_ld<bf16x8>(q_lds + (uint32_t)(l16 * ROWB) +
                                   16u * (uint32_t)w16_kchunk(4 * c + g4, l16))
                  : z;
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
  finish_stage(B0{}, blk(0));
  if (nk > 1) finish_stage(B1{}, blk(1));
  stage_barrier();             // also publishes the time tables; Q reads are done

  // Epilogue staging: the 16 rows of wave w in stage buffer
  // ((kt_hi - kt_lo) + 1 + w / 4) % 4 at 4 KB * (w % 4) -- a buffer that
  // neither the last block nor any copy in flight touches.
  const bool ln_ep = a.epilogue == 0;
  auto ep_lds = [&]() __attribute__((always_inline)) -> uint32_t {
    const int b_ep = (((kt_hi - kt_lo) & ~1) + 2 + (wave >> 2)) & (kW16Stages - 1);
    return (b_ep == 0 ? lds_off(st0.k) : b_ep == 1 ? lds_off(st1.k) : b_ep == 2 ? lds_off(st2.k)
                                                                               : lds_off(st3.k)) +
           (uint32_t)((wave & 3) * kW16Rows * ROWB);
  };
  // U rows of this wave into the epilogue buffer; issued at the start of the
  // last step so that their latency hides behind the last block.
  auto issue_u = [&]() __attribute__((always_inline)) {
    if (!(ln_ep && wave_rows)) return;
    const int ul = opaque_lane();
    const uint32_t e_lds = ep_lds();
    const uint64_t ub = uni_ptr(reinterpret_cast<const char*>(a.u) +
                                ((int64_t)(seq0 + i0) * a.ld_u + (int64_t)h * 128) * 2);
    const uint32_t ldu_b = (uint32_t)(a.ld_u * 2);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int m = 64 * n + ul, r = m >> 4;
      const int row = min(wr0 + r, i1 - 1) - i0;
      lds_copy16_nt(ub, (uint32_t)row * ldu_b + 16u * (uint32_t)w16_kchunk(m & 15, r),
                    e_lds + 1024u * (uint32_t)n);
    }
  };

  // One pipeline step on the walk's blocks s, s + 1 held in buffers `bufc`,
  // `bufc` + 1: copy blocks s + 2, s + 3 into the other two buffers (freed
  // by the previous barrier), compute both blocks, then (this wave's copies
  // landed) finish the next two and synchronise.  The second copy is issued
  // after the first block: every wave leaves the barrier together, and
  // issuing all copies at once queues them behind each other.
  auto step = [&](auto bufc, int s) __attribute__((always_inline)) {
    constexpr int b = decltype(bufc)::value;
    using N1 = std::integral_constant<int, (b + 1) % kW16Stages>;
    using N2 = std::integral_constant<int, (b + 2) % kW16Stages>;
    using N3 = std::integral_constant<int, (b + 3) % kW16Stages>;
    const bool has1 = s + 1 < nk, next0 = s + 2 < nk, next1 = s + 3 < nk;
    const int kt = blk(s), kt1 = blk(s + 1), kt2 = blk(s + 2), kt3 = blk(s + 3);
    if (next0) issue_stage(N2{}, kt2);
    else issue_u();
    if (needs(kt)) block(stage(bufc), kt);
    if (next1) issue_stage(N3{}, kt3);
    if (has1 && needs(kt1)) block(stage(N1{}), kt1);
    if (next0) {
      wait_vmem<0>();
      finish_stage(N2{}, kt2);
      if (next1) finish_stage(N3{}, kt3);
      stage_barrier();
    }
  };
  for (int s = 0;; s += kW16Stages) {
    step(B0{}, s);
    if (s + 2 >= nk) break;
    step(B2{}, s + 2);
    if (s + 4 >= nk) break;
  }

  // ---- chunk of a split item: publish the partial output; the chunk that
  // arrives last adds all partials in chunk order and runs the epilogue ----
  const int n_chunks = ch.w & 0x7fff;
  if (n_chunks > 1) {
    // slot layout: [wave][t][lane] x 4 floats (two 8-byte words)
    auto slot = [&](int c) __attribute__((always_inline)) {
      return reinterpret_cast<uint64_t*>(a.partials + (int64_t)(ch.z + c) * a.slot_floats) +
             2 * (wave * 8 * 64 + lane);
    };
    uint64_t* own = slot((ch.w >> 16) & 0x7fff);
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int hw = 0; hw < 2; ++hw) {
        const uint64_t w2 = (uint64_t)__float_as_uint(acc[t][2 * hw]) |
                            ((uint64_t)__float_as_uint(acc[t][2 * hw + 1]) << 32);
        __hip_atomic_store(own + 2 * t * 64 + hw, w2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    wait_vmem<0>();
    __syncthreads();
    if (tid == 0)
      s_ticket = __hip_atomic_fetch_add(a.counters + ch.z, 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_ticket != n_chunks - 1) continue;   // another chunk finishes the item
    if (tid == 0) a.counters[ch.z] = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][e] = 0.0f;
    for (int c = 0; c < n_chunks; ++c) {
      const uint64_t* src = slot(c);
      uint64_t p[8][2];
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int hw = 0; hw < 2; ++hw)
          p[t][hw] = __hip_atomic_load(src + 2 * t * 64 + hw, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int hw = 0; hw < 2; ++hw) {
          acc[t][2 * hw] += __uint_as_float((uint32_t)p[t][hw]);
          acc[t][2 * hw + 1] += __uint_as_float((uint32_t)(p[t][hw] >> 32));
        }
    }
  }

  // ---- epilogue: ln(2)/n_scale, LayerNorm over d_v, * U, store ------------
  {
    const float osc = a.out_scale;
    const int ln = opaque_lane();
    const int l16 = ln & 15, g4 = ln >> 4;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][e] *= osc;
    if (a.out_raw != nullptr && row_valid) {
      char* rrow = reinterpret_cast<char*>(a.out_raw) +
                   ((int64_t)(seq0 + i) * a.ld_raw + (int64_t)h * 128) * 2;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)acc[t][e];
        *reinterpret_cast<bf16x4*>(rrow + 2 * (16 * t + 4 * g4)) = o;
      }
    }
    float mean = 0.0f, rstd = 1.0f;
    if (ln_ep) {
      float sum = 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) sum += acc[t][e];
      sum += __shfl_xor(sum, 16, 64);
      sum += __shfl_xor(sum, 32, 64);
      mean = sum * (1.0f / 128);
      float sq = 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float c = acc[t][e] - mean;
          sq += c * c;
        }
      sq += __shfl_xor(sq, 16, 64);
      sq += __shfl_xor(sq, 32, 64);
      rstd = rsqrtf(sq * (1.0f / 128) + a.ln_eps);
    }
    if (wave_rows) {
      const uint32_t e_lds = ep_lds();
      if (ln_ep) wait_vmem<0>();   // this wave's U rows have landed
      // y = (O - mean) * rstd * U in place of U: row l16, columns 16t + 4 g4 ..
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t off = e_lds + (uint32_t)(l16 * ROWB) +
                             16u * (uint32_t)w16_kchunk(2 * t + (g4 >> 1), l16) +
                             8u * (uint32_t)(g4 & 1);
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = acc[t][e];
        if (ln_ep) {
          const bf16x4 uu = lds_ld<bf16x4>(off);
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = (y[e] - mean) * rstd * (float)uu[e];
        }
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)y[e];
        lds_st<bf16x4>(off, o);
      }
      // whole rows out: lane l of store n writes physical chunk (64n + l) % 16
      // of row (64n + l) / 16, i.e. logical chunk ^ swizzle, rows of the tile only
      char* obase = reinterpret_cast<char*>(uni_ptr(
          reinterpret_cast<char*>(a.out) + ((int64_t)(seq0 + wr0) * a.ld_out + (int64_t)h * 128) * 2));
      const uint32_t ldo_b = (uint32_t)(a.ld_out * 2);
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int m = 64 * n + ln, r = m >> 4;
        const uintx4 w4 = lds_ld<uintx4>(e_lds + 16u * (uint32_t)m);
        if (wr0 + r < i1)
          __builtin_nontemporal_store(
              w4, reinterpret_cast<uintx4*>(obase + ((uint32_t)r * ldo_b +
                                                     16u * (uint32_t)w16_kchunk(m & 15, r))));
      }
    }
  }

  // The LDS of this item is free again once every wave is here.
  stage_barrier();
  }  // units
  }  // planned workgroups
}

template <int POSM, bool TIME, bool TR>
static hipError_t launch_w16_one(const AttnArgs& a, int n_wg, hipStream_t stream,
                                 hipEvent_t start, hipEvent_t stop) {
  auto kern = hstu_attn_fwd_w16_kernel<POSM, TIME, TR>;
  if (start || stop)
    hipExtLaunchKernelGGL(kern, dim3((unsigned)n_wg), dim3(kW16Threads), 0, stream, start, stop,
                          0, a);
  else
    hipLaunchKernelGGL(kern, dim3((unsigned)n_wg), dim3(kW16Threads), 0, stream, a);
  return hipGetLastError();
}

template <int POSM, bool TIME, bool TR>
static int w16_blocks_per_cu() {
  auto kern = hstu_attn_fwd_w16_kernel<POSM, TIME, TR>;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, kW16Threads, 0) != hipSuccess)
    return -1;
  return nb;
}

bool attn_w16_supported(int dtype, int d_qk, int d_v) {
  return dtype == 1 && d_qk == 128 && d_v == 128;
}

int attn_w16_grid(int pos_len, int time_len, bool clamp, bool transposed) {
  const bool pos = pos_len > 0, tim = time_len > 0;
  int bpc;
  if (transposed) {
    if (clamp) return -1;
    if (pos && tim) bpc = w16_blocks_per_cu<1, true, true>();
    else if (pos) bpc = w16_blocks_per_cu<1, false, true>();
    else if (tim) bpc = w16_blocks_per_cu<0, true, true>();
    else bpc = w16_blocks_per_cu<0, false, true>();
  } else if (pos && clamp && tim) bpc = w16_blocks_per_cu<2, true, false>();
  else if (pos && clamp) bpc = w16_blocks_per_cu<2, false, false>();
  else if (pos && tim) bpc = w16_blocks_per_cu<1, true, false>();
  else if (pos) bpc = w16_blocks_per_cu<1, false, false>();
  else if (tim) bpc = w16_blocks_per_cu<0, true, false>();
  else bpc = w16_blocks_per_cu<0, false, false>();
  if (bpc <= 0) return -1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  return cus * bpc;
}

hipError_t launch_attn_w16(const AttnArgs& a, int n_wg, hipStream_t stream, hipEvent_t t0,
                           hipEvent_t t1, bool transposed) {
  const bool pos = a.pos_len > 0, tim = a.time_len > 0, cl = a.pos_clamp != 0;
  if (transposed) {
    if (cl) return hipErrorInvalidValue;
    if (pos && tim) return launch_w16_one<1, true, true>(a, n_wg, stream, t0, t1);
    if (pos) return launch_w16_one<1, false, true>(a, n_wg, stream, t0, t1);
    if (tim) return launch_w16_one<0, true, true>(a, n_wg, stream, t0, t1);
    return launch_w16_one<0, false, true>(a, n_wg, stream, t0, t1);
  }
  if (pos && cl && tim) return launch_w16_one<2, true, false>(a, n_wg, stream, t0, t1);
  if (pos && cl) return launch_w16_one<2, false, false>(a, n_wg, stream, t0, t1);
  if (pos && tim) return launch_w16_one<1, true, false>(a, n_wg, stream, t0, t1);
  if (pos) return launch_w16_one<1, false, false>(a, n_wg, stream, t0, t1);
  if (tim) return launch_w16_one<0, true, false>(a, n_wg, stream, t0, t1);
  return launch_w16_one<0, false, false>(a, n_wg, stream, t0, t1);
}

}  // namespace hstu
