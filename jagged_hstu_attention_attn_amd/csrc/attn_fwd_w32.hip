// attn_fwd_w32.hip -- gfx950 jagged HSTU attention forward, bf16 with
// d_qk = d_v = 128: thirty-two query rows per wave, as two 16-row groups that
// share every K and V operand read, four waves per workgroup and two
// workgroups per CU (two waves per SIMD, up to 256 registers each).
//
// Against the sixteen-row kernel (eight waves of 16 rows, four waves per
// SIMD) a wave reads each staged K and V block once for twice the rows, so
// the LDS operand reads per matrix-core instruction halve, and it holds two
// independent chains per block: the second group's score MFMAs run while the
// first group's bias and SiLU issue, and the first group's aggregation MFMAs
// while the second group's SiLU issues (scheduling-group hints interleave
// them on the common path).
//
// Work items, stage layout and per-block arithmetic are the sixteen-row
// kernel's: the scheduler's units (sequence, head, 128-row query tile,
// key-tile range); keys staged 32 at a time in four LDS buffers copied from
// HBM straight into LDS (global_load_lds), a step computing two key blocks
// while the next two are copied, one barrier per step.  Per 32-key block and
// group, with v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T + C       two 16-key x 16-row tiles, the accumulator starting
//                         at the position bias
//   x   = am S + time bias, mask select, A = SiLU(x)     (8 values per lane)
//   O^T += V^T A^T        eight 16-column tiles of d_v
// The epilogue scales by ln(2)/n_scale, takes LayerNorm over d_v per (token,
// head), gates by U and stores whole rows through LDS.
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

constexpr int kW32Waves = 4;
constexpr int kW32Threads = kW32Waves * 64;
constexpr int kW32Rows = 32;        // query rows per wave
constexpr int kW32Stages = 4;       // LDS buffers of the key/value pipeline
static_assert(kBM == kW32Waves * kW32Rows, "four row groups of 32 per item");
static_assert(kBN == 32, "a key block is two 16-key score tiles");

typedef float floatx4v32 __attribute__((ext_vector_type(4)));

template <bool CLAMP>
struct W32Stage {
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

static_assert(offsetof(W32Stage<false>, tmin) % 16 == 0 && offsetof(W32Stage<true>, tmin) % 16 == 0,
              "the key-time range is one aligned 16-byte read");
static_assert(offsetof(W32Stage<false>, v) == kBN * 256,
              "K and V of a stage are contiguous: a wave's 32 staged rows span both");

// Physical 16-byte chunk of logical chunk c in staged row `row`.
__device__ inline int w32_kchunk(int c, int row) { return c ^ (row & 15); }
__device__ inline int w32_vchunk(int c, int row) { return c ^ (2 * (row & 7)); }

// POSM: 0 = no position bias, 1 = position bias of |i - j|, 2 = of the
// clamped positions |p_i - p_j| (candidate rows take it from cpos).
template <int POSM, bool TIME>
__global__ __launch_bounds__(kW32Threads) __attribute__((amdgpu_waves_per_eu(2))) void
hstu_attn_fwd_w32_kernel(AttnArgs a) {
  constexpr bool POS = POSM != 0;
  constexpr bool clamp = POSM == 2;
  using SB = W32Stage<clamp>;
  constexpr int ROWB = 256;          // staged row bytes (128 bf16)
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;

  __shared__ __align__(256) SB st0, st1, st2, st3;
  __shared__ TimeTables tt;
  __shared__ int s_ticket;
  __shared__ int s_qnext[2];
  auto stage = [&](auto bufc) __attribute__((always_inline)) -> SB& {
    constexpr int b = decltype(bufc)::value % kW32Stages;
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
  // Copies of one stage: wave w copies rows 8w .. 8w + 7 of the keys and of
  // the values (two 1 KB copies each).  The bias inputs go to "role" waves,
  // which a stage in an odd buffer maps to wave role ^ 2 (the two stages of
  // a step split that work between the two halves of the workgroup): roles
  // 0-2 gather the position-bias diagonal (part = role), role 3 the raw
  // timestamps and the clamped-position bias.
  constexpr int kTsW = 3, kCposW = 3;
  auto role_wave = [&](auto bufc) __attribute__((always_inline)) {
    return (decltype(bufc)::value & 1) ? (wave ^ 2) : wave;
  };
  static_assert(kDiagCopies <= 3, "three waves gather the position-bias diagonal");

  auto opaque_lane = [&]() __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    return ln;
  };

  // This lane's K/V copy offsets within a stage of whole rows: copy n covers
  // rows 8w + 4n .. + 3, row 8w + 4n + l/16, swizzled chunk of l % 16.
  uint32_t ko_full[2], vo_full[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int row = 8 * wave + 4 * n + (lane >> 4);
    ko_full[n] = (uint32_t)row * ldk_b + 16u * (uint32_t)w32_kchunk(lane & 15, row);
    vo_full[n] = (uint32_t)row * ldv_b + 16u * (uint32_t)w32_vchunk(lane & 15, row);
  }

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
  tile_key_range(geo, i0, i1, jlo, jhi);
  const int kt_lo = max(jlo / kBN, ch.x), kt_hi = min(jhi / kBN, ch.y);
  // Key blocks are walked from a rotation of [kt_lo, kt_hi] under a window
  // (no softmax, so the order is free): step s takes the block kt = s (mod
  // nk), so the neighbouring tiles of one L2, whose ranges have the same
  // length and start four blocks apart, read each block at about the same
  // time.
  const int nk = kt_hi - kt_lo + 1;
  const int rot = (geo.W > 0 && nk > 1) ? (nk - kt_lo % nk) % nk : 0;
  auto blk = [&](int s) __attribute__((always_inline)) {
    const int t = s + rot;
    return kt_lo + (t >= nk ? t - nk : t);
  };

  // ---- per-lane query rows (one per group) and the uniform key bounds -----
  const int wr0 = i0 + wave * kW32Rows;
  int ig[2];
  bool rvalid[2];
  bool grows[2];   // the group has a row of the tile
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    ig[g] = wr0 + 16 * g + (lane & 15);
    rvalid[g] = ig[g] < i1;
    grows[g] = wr0 + 16 * g < i1;
  }
  const bool wave_rows = grows[0];
  int w_jmin, w_jmax, w_lomax[2], w_himin[2];
  {
    int jmin = 0x7fffffff, jmax = -1;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const RowBounds rb = rvalid[g] ? row_bounds(geo, ig[g]) : RowBounds{kEmptyLo, 0, -1};
      const bool nonempty = rb.lo != kEmptyLo;
      const int hi = rb.lo + rb.span;
      int jmn = nonempty ? rb.lo : (rb.self_j >= 0 ? rb.self_j : 0x7fffffff);
      int jmx = nonempty ? max(hi, rb.self_j) : rb.self_j;
      if (!rvalid[g]) { jmn = 0x7fffffff; jmx = -1; }
      jmin = min(jmin, jmn);
      jmax = max(jmax, jmx);
      w_lomax[g] = wave_max(rvalid[g] ? rb.lo : -1);
      w_himin[g] = wave_min(rvalid[g] ? (nonempty ? hi : -1) : 0x7fffffff);
    }
    w_jmin = wave_min(jmin);
    w_jmax = wave_max(jmax);
  }
  bool w_cand[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) w_cand[g] = clamp && grows[g] && wr0 + 16 * g + 15 >= geo.n_h;
  (void)w_cand;
  auto needs = [&](int kt) __attribute__((always_inline)) {
    const int jb = kt * kBN;
    return wave_rows && jb <= w_jmax && jb + kBN - 1 >= w_jmin;
  };
  auto is_full = [&](int g, int kt) __attribute__((always_inline)) {
    const int jb = kt * kBN;
    return w_lomax[g] <= jb && w_himin[g] >= jb + kBN - 1;
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
    const uint64_t kb = kseq + (uint64_t)j0 * ldk_b, vb = vseq + (uint64_t)j0 * ldv_b;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      uint32_t ko = ko_full[n], vo = vo_full[n];
      if (j0 + kBN > L) {   // the sequence's last block: rows past its end repeat row L - 1
        const int row = 8 * wave + 4 * n + (ln >> 4);
        const uint32_t r = (uint32_t)min(row, L - 1 - j0);
        ko = r * ldk_b + 16u * (uint32_t)w32_kchunk(ln & 15, row);
        vo = r * ldv_b + 16u * (uint32_t)w32_vchunk(ln & 15, row);
      }
      const uint32_t dst = 1024u * (uint32_t)(2 * wave + n);
      if (kv_nt) {
        lds_copy16_nt(kb, ko, lds_off(sb.k) + dst);
        lds_copy16_nt(vb, vo, lds_off(sb.v) + dst);
      } else {
        lds_copy16(kb, ko, lds_off(sb.k) + dst);
        lds_copy16(vb, vo, lds_off(sb.v) + dst);
      }
    }
    const int rw = role_wave(bufc);
    if constexpr (POS) {
      if (rw < kDiagCopies) {
        const int d = i0 - j0 + (kBM - 1) - (64 * rw + ln);
        const int ix = min(d < 0 ? -d : d, P - 1);
        lds_copy4(pos_base, 4u * (uint32_t)ix, lds_off(sb.diag) + 256u * (uint32_t)rw);
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
  uint32_t ti32[2] = {uint32_t(kT32Range), uint32_t(kT32Range)};
  bool w_t_ok = true;
  uint32_t w_tmin[2] = {0, 0}, w_tmax[2] = {0, 0};

  // Once this wave's own copies of stage kt have landed: rescale the
  // position-bias values it gathered; in the timestamp wave, form the 32-bit
  // key times, their range and whether any key needs the 64-bit path.
  auto finish_stage = [&](auto bufc, int kt) __attribute__((always_inline)) {
    SB& sb = stage(bufc);
    const int ln = opaque_lane();
    const int rw = role_wave(bufc);
    if constexpr (POS) {
      if (rw < kDiagCopies) {
        const int e = 64 * rw + ln;
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

  // Q operands (B of S^T = K Q^T) of group g: qf[g][c] holds d = 32c + 8 (l /
  // 16) .. + 7 of row 16 g + l % 16; O^T accumulators: acc[g][t][i] is
  // d = 16 t + 4 (l / 16) + i of that row
  bf16x8 qf[2][4];
  floatx4v32 acc[2][8];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[g][t][e] = 0.0f;

  // Whether every (row, key) time gap of group g and a block falls in one
  // bucket, from the block's key-time range `kr` (tmin, tmax, tbad); then
  // `tb` is that bucket's bias.  Uniform values throughout.
  auto time_const = [&](const uint4& kr, int g, float& tb) __attribute__((always_inline)) -> bool {
    if (!w_t_ok || uni((int)kr.z) != 0) return false;
    const uint32_t kmin = (uint32_t)uni((int)kr.x), kmax = (uint32_t)uni((int)kr.y);
    const uint32_t wmin = (uint32_t)uni((int)w_tmin[g]), wmax = (uint32_t)uni((int)w_tmax[g]);
    // ranges [wmin, wmax] and [kmin, kmax]: at most one of the two gaps is positive
    const uint32_t dmin = (max(wmin, kmax) - kmax) + (max(kmin, wmax) - wmax);
    const uint32_t dmax = max(max(wmax, kmin) - kmin, max(kmax, wmin) - wmin);
    const int z0 = __builtin_clz(dmin + 1u), z1 = __builtin_clz(dmax + 1u);
    if (z0 != z1) return false;
    tb = __builtin_bit_cast(float, uni(__builtin_bit_cast(int, tt.trev[z0])));
    return true;
  };

  // x2 = am * S + log2e * time of group g, any time path, then the mask.
  auto scores_general = [&](SB& sb, int kt, const uint4& kr, int g, const floatx4v32& sa,
                            const floatx4v32& sbk, float* x) __attribute__((always_inline)) {
    const int jb = kt * kBN;
    const int g4 = lane >> 4;
    if constexpr (TIME) {
      float tb = 0.0f;
      if (time_const(kr, g, tb)) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = fmaf(sa[e], am, tb);
          x[4 + e] = fmaf(sbk[e], am, tb);
        }
      } else if (w_t_ok && uni(sb.tbad) == 0) {
#pragma unroll
        for (int tk = 0; tk < 2; ++tk) {
          const uint4 t4 = *reinterpret_cast<const uint4*>(&sb.ts32[16 * tk + 4 * g4]);
          const uint32_t tv[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t d1 = (ti32[g] > tv[e] ? ti32[g] - tv[e] : tv[e] - ti32[g]) + 1u;
            x[4 * tk + e] = fmaf(tk ? sbk[e] : sa[e], am, tt.trev[__builtin_clz(d1)]);
          }
        }
      } else {
        // times too far apart for 32 bits (rare): 64-bit differences
        const int64_t t_i = rvalid[g] ? a.timestamps[seq0 + ig[g]] : tbase;
#pragma unroll
        for (int tk = 0; tk < 2; ++tk)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t tj = sb.ts64[16 * tk + 4 * g4 + e];
            const uint64_t dt = t_i >= tj ? uint64_t(t_i) - uint64_t(tj)
                                          : uint64_t(tj) - uint64_t(t_i);
            x[4 * tk + e] = fmaf(tk ? sbk[e] : sa[e], am,
                                 tt.tful[63 - __builtin_clzll(dt + 1u)]);
          }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = sa[e] * am;
        x[4 + e] = sbk[e] * am;
      }
    }
    // illegal pairs: an argument whose SiLU is exactly -0
    if (!is_full(g, kt)) {
      // recomputed here (an opaque row index) rather than kept live from the prologue
      int row = ig[g];
      asm volatile("" : "+v"(row));
      const RowBounds rb = rvalid[g] ? row_bounds(geo, row) : RowBounds{kEmptyLo, 0, -1};
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
  };

  // One 32-key block from stage buffer `sb` for both row groups.
  auto block = [&](SB& sb, int kt) __attribute__((always_inline)) {
    const int l16 = lane & 15, g4 = lane >> 4;
    // ---- score starts (position bias) and the K operands ----
    floatx4v32 s[2][2];   // [group][16-key tile]
    uint4 kr = {0u, 0u, 0u, 0u};   // key-time range of the block (TIME)
    if constexpr (TIME) kr = *reinterpret_cast<const uint4*>(&sb.tmin);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int dbase = (kBM - 1) - kW32Rows * wave - 16 * g - l16 + 4 * g4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (POS) {
          s[g][0][e] = sb.diag[dbase + e];
          s[g][1][e] = sb.diag[dbase + 16 + e];
        } else {
          s[g][0][e] = 0.0f;
          s[g][1][e] = 0.0f;
        }
      }
      if constexpr (clamp) {
        if (w_cand[g]) {   // candidate rows: bias of the clamped positions
          const bool cr = ig[g] >= geo.n_h;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float c0 = sb.cpos[4 * g4 + e], c1 = sb.cpos[16 + 4 * g4 + e];
            s[g][0][e] = cr ? c0 : s[g][0][e];
            s[g][1][e] = cr ? c1 : s[g][1][e];
          }
        }
      }
    }
    // K operand of (tile tk, step c): key 16 tk + l16, logical chunk 4c + g4,
    // physical chunk (4c + g4) ^ l16: byte offset ka ^ 64c.  Read in two
    // halves (c = 0, 1 then 2, 3) into the same registers.
    const uint32_t ka = (uint32_t)(l16 * ROWB + 16 * (g4 ^ (l16 & 3)) + 64 * (l16 >> 2));
    auto kread = [&](int tk, int c) __attribute__((always_inline)) {
      return lds_ld<bf16x8>(lds_off(sb.k) + (uint32_t)(tk * 16 * ROWB) + (ka ^ (64u * c)));
    };
    // V^T operands of d_v tile t (as the sixteen-row kernel reads them)
    const int er = l16 >> 2, q = l16 & 3;
    const int vrow = 4 * g4 + er;
    const uint32_t va = (uint32_t)(vrow * ROWB + 8 * (q & 1) + 16 * (q >> 1) + 32 * (vrow & 7));
    auto vread = [&](int t) __attribute__((always_inline)) {
      const uint32_t off = lds_off(sb.v) + (va ^ (32u * t));
      const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr4(off));
      const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr4(off + 16 * ROWB));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 k0[2], k1[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      k0[c] = kread(0, c);
      k1[c] = kread(1, c);
    }

    // The common path: one time bucket for both groups and no mask.
    float tb0 = 0.0f, tb1 = 0.0f;
    bool fast = is_full(0, kt) && is_full(1, kt);
    if constexpr (TIME) fast = fast && time_const(kr, 0, tb0) && time_const(kr, 1, tb1);
    __builtin_amdgcn_sched_barrier(0);

    // ---- scores: both groups on the first K half, group 0 on the second ----
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        s[g][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0[c], qf[g][c], s[g][0], 0, 0, 0);
        s[g][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1[c], qf[g][c], s[g][1], 0, 0, 0);
      }
#pragma unroll
    for (int c = 2; c < 4; ++c) {
      k0[c - 2] = kread(0, c);
      k1[c - 2] = kread(1, c);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 2; c < 4; ++c) {
      s[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0[c - 2], qf[0][c], s[0][0], 0, 0, 0);
      s[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1[c - 2], qf[0][c], s[0][1], 0, 0, 0);
    }
    bf16x8 vop[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) vop[t] = vread(t);
    __builtin_amdgcn_sched_barrier(0);

    bf16x8 pa0, pa1;
    if (fast) {
      // ---- group 1's last score MFMAs, group 0 bias + SiLU interleaved ----
#pragma unroll
      for (int c = 2; c < 4; ++c) {
        s[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0[c - 2], qf[1][c], s[1][0], 0, 0, 0);
        s[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1[c - 2], qf[1][c], s[1][1], 0, 0, 0);
      }
      {
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = TIME ? fmaf(s[0][0][e], am, tb0) : s[0][0][e] * am;
          x[4 + e] = TIME ? fmaf(s[0][1][e], am, tb0) : s[0][1][e] * am;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) pa0[e] = (__bf16)silu2(x[e]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x402, 8, 0);   // then vector / transcendental
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- group 0 aggregation, group 1 bias + SiLU interleaved ----
#pragma unroll
      for (int t = 0; t < 8; ++t)
        acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[t], pa0, acc[0][t], 0, 0, 0);
      {
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = TIME ? fmaf(s[1][0][e], am, tb1) : s[1][0][e] * am;
          x[4 + e] = TIME ? fmaf(s[1][1][e], am, tb1) : s[1][1][e] * am;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) pa1[e] = (__bf16)silu2(x[e]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, 5, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int c = 2; c < 4; ++c) {
        s[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0[c - 2], qf[1][c], s[1][0], 0, 0, 0);
        s[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1[c - 2], qf[1][c], s[1][1], 0, 0, 0);
      }
      {
        float x[8];
        scores_general(sb, kt, kr, 0, s[0][0], s[0][1], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) pa0[e] = (__bf16)silu2(x[e]);
      }
#pragma unroll
      for (int t = 0; t < 8; ++t)
        acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[t], pa0, acc[0][t], 0, 0, 0);
      {
        float x[8];
        scores_general(sb, kt, kr, 1, s[1][0], s[1][1], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) pa1[e] = (__bf16)silu2(x[e]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- group 1 aggregation ----
#pragma unroll
    for (int t = 0; t < 8; ++t)
      acc[1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[t], pa1, acc[1][t], 0, 0, 0);
  };

  // ---- item prologue -------------------------------------------------------
  issue_stage(B0{}, blk(0));
  if (nk > 1) issue_stage(B1{}, blk(1));
  int q_fetch;
  if (queue && tid == 0) q_fetch = atomicAdd(const_cast<int32_t*>(a.hdr) + wkq.ctr, 1);
  int64_t ti64[2] = {0, 0};
  if constexpr (TIME) {
    tbase = a.timestamps[seq0 + i0];
#pragma unroll
    for (int g = 0; g < 2; ++g) ti64[g] = a.timestamps[seq0 + min(ig[g], i1 - 1)];
  }
  // Query tile: each wave copies its 32 rows (8 KB) into stage buffers 2 and
  // 3, idle in the prologue (rows of waves 0-1 in buffer 2, 2-3 in buffer 3,
  // each wave's 8 KB spanning K and V of that stage), then reads its MFMA
  // operands from there.
  const uint32_t q_lds = lds_off(wave < 2 ? st2.k : st3.k) + (uint32_t)((wave & 1) * kW32Rows * ROWB);
  if (wave_rows && !alpha_zero) {
    const int ql = opaque_lane();
    const uint64_t qb = uni_ptr(reinterpret_cast<const char*>(a.q) +
                                ((int64_t)(seq0 + i0) * a.ld_q + (int64_t)h * 128) * 2);
    const uint32_t ldq_b = (uint32_t)(a.ld_q * 2);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int m = 64 * n + ql, r = m >> 4;
      const int row = min(wr0 + r, i1 - 1) - i0;
      lds_copy16_nt(qb, (uint32_t)row * ldq_b + 16u * (uint32_t)w32_kchunk(m & 15, r),
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
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 z = {};
        qf[g][c] = (rvalid[g] && !alpha_zero)
                       ? lds_ld<bf16x8>(q_lds + (uint32_t)((16 * g + l16) * ROWB) +
                                        16u * (uint32_t)w32_kchunk(4 * c + g4, l16))
                       : z;
      }
  }
  if constexpr (TIME) {
    asm volatile("" : "+v"(ti64[0]), "+v"(ti64[1]));
    bool ok_all = true;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int64_t rel = ti64[g] - tbase;
      const bool ok = rel > -kT32Range && rel < kT32Range;
      ti32[g] = ok ? uint32_t(rel + kT32Range) : 0u;
      ok_all = ok_all && ok;
      w_tmin[g] = wave_min(rvalid[g] ? ti32[g] : 0xffffffffu);
      w_tmax[g] = wave_max(rvalid[g] ? ti32[g] : 0u);
    }
    w_t_ok = __all(ok_all);
  }
  finish_stage(B0{}, blk(0));
  if (nk > 1) finish_stage(B1{}, blk(1));
  stage_barrier();             // also publishes the time tables; Q reads are done

  // Epilogue staging: the 32 rows of wave w in stage buffer
  // ((nk - 1) & ~1) + 2 + w / 2 (mod 4) at 8 KB * (w % 2) -- a buffer that
  // neither the last block nor any copy in flight touches.
  const bool ln_ep = a.epilogue == 0;
  auto ep_lds = [&]() __attribute__((always_inline)) -> uint32_t {
    const int b_ep = (((kt_hi - kt_lo) & ~1) + 2 + (wave >> 1)) & (kW32Stages - 1);
    return (b_ep == 0 ? lds_off(st0.k) : b_ep == 1 ? lds_off(st1.k) : b_ep == 2 ? lds_off(st2.k)
                                                                               : lds_off(st3.k)) +
           (uint32_t)((wave & 1) * kW32Rows * ROWB);
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
    for (int n = 0; n < 8; ++n) {
      const int m = 64 * n + ul, r = m >> 4;
      const int row = min(wr0 + r, i1 - 1) - i0;
      lds_copy16_nt(ub, (uint32_t)row * ldu_b + 16u * (uint32_t)w32_kchunk(m & 15, r),
                    e_lds + 1024u * (uint32_t)n);
    }
  };

  // One pipeline step on the walk's blocks s, s + 1 held in buffers `bufc`,
  // `bufc` + 1: copy blocks s + 2, s + 3 into the other two buffers (freed
  // by the previous barrier; the second after the first block), compute
  // both blocks, then (this wave's copies landed) finish the next two and
  // synchronise.
  auto step = [&](auto bufc, int s) __attribute__((always_inline)) {
    constexpr int b = decltype(bufc)::value;
    using N1 = std::integral_constant<int, (b + 1) % kW32Stages>;
    using N2 = std::integral_constant<int, (b + 2) % kW32Stages>;
    using N3 = std::integral_constant<int, (b + 3) % kW32Stages>;
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
  for (int s = 0;; s += kW32Stages) {
    step(B0{}, s);
    if (s + 2 >= nk) break;
    step(B2{}, s + 2);
    if (s + 4 >= nk) break;
  }

  // ---- chunk of a split item: publish the partial output; the chunk that
  // arrives last adds all partials in chunk order and runs the epilogue ----
  const int n_chunks = ch.w & 0x7fff;
  if (n_chunks > 1) {
    // slot layout: [wave][group][t][lane] x 4 floats (two 8-byte words)
    auto slot = [&](int c, int g) __attribute__((always_inline)) {
      return reinterpret_cast<uint64_t*>(a.partials + (int64_t)(ch.z + c) * a.slot_floats) +
             2 * ((wave * 2 + g) * 8 * 64 + lane);
    };
    const int own_c = (ch.w >> 16) & 0x7fff;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      uint64_t* own = slot(own_c, g);
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int hw = 0; hw < 2; ++hw) {
          const uint64_t w2 = (uint64_t)__float_as_uint(acc[g][t][2 * hw]) |
                              ((uint64_t)__float_as_uint(acc[g][t][2 * hw + 1]) << 32);
          __hip_atomic_store(own + 2 * t * 64 + hw, w2, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
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
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[g][t][e] = 0.0f;
    for (int c = 0; c < n_chunks; ++c) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const uint64_t* src = slot(c, g);
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
            acc[g][t][2 * hw] += __uint_as_float((uint32_t)p[t][hw]);
            acc[g][t][2 * hw + 1] += __uint_as_float((uint32_t)(p[t][hw] >> 32));
          }
      }
    }
  }

  // ---- epilogue: ln(2)/n_scale, LayerNorm over d_v, * U, store ------------
  {
    const float osc = a.out_scale;
    const int ln = opaque_lane();
    const int l16 = ln & 15, g4 = ln >> 4;
    const uint32_t e_lds = wave_rows ? ep_lds() : 0u;
    if (wave_rows && ln_ep) wait_vmem<0>();   // this wave's U rows have landed
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[g][t][e] *= osc;
      if (a.out_raw != nullptr && rvalid[g]) {
        char* rrow = reinterpret_cast<char*>(a.out_raw) +
                     ((int64_t)(seq0 + ig[g]) * a.ld_raw + (int64_t)h * 128) * 2;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (__bf16)acc[g][t][e];
          *reinterpret_cast<bf16x4*>(rrow + 2 * (16 * t + 4 * g4)) = o;
        }
      }
      float mean = 0.0f, rstd = 1.0f;
      if (ln_ep) {
        float sum = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) sum += acc[g][t][e];
        sum += __shfl_xor(sum, 16, 64);
        sum += __shfl_xor(sum, 32, 64);
        mean = sum * (1.0f / 128);
        float sq = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float c = acc[g][t][e] - mean;
            sq += c * c;
          }
        sq += __shfl_xor(sq, 16, 64);
        sq += __shfl_xor(sq, 32, 64);
        rstd = rsqrtf(sq * (1.0f / 128) + a.ln_eps);
      }
      if (wave_rows) {
        // y = (O - mean) * rstd * U in place of U: row 16 g + l16, columns
        // 16t + 4 g4 .. + 3
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const uint32_t off = e_lds + (uint32_t)((16 * g + l16) * ROWB) +
                               16u * (uint32_t)w32_kchunk(2 * t + (g4 >> 1), l16) +
                               8u * (uint32_t)(g4 & 1);
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = acc[g][t][e];
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
      }
    }
    if (wave_rows) {
      // whole rows out: lane l of store n writes physical chunk (64n + l) % 16
      // of row (64n + l) / 16, i.e. logical chunk ^ swizzle, rows of the tile only
      char* obase = reinterpret_cast<char*>(uni_ptr(
          reinterpret_cast<char*>(a.out) + ((int64_t)(seq0 + wr0) * a.ld_out + (int64_t)h * 128) * 2));
      const uint32_t ldo_b = (uint32_t)(a.ld_out * 2);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int m = 64 * n + ln, r = m >> 4;
        const uintx4 w4 = lds_ld<uintx4>(e_lds + 16u * (uint32_t)m);
        if (wr0 + r < i1)
          __builtin_nontemporal_store(
              w4, reinterpret_cast<uintx4*>(obase + ((uint32_t)r * ldo_b +
                                                     16u * (uint32_t)w32_kchunk(m & 15, r))));
      }
    }
  }

  // The LDS of this item is free again once every wave is here.
  stage_barrier();
  }  // units
  }  // planned workgroups
}

template <int POSM, bool TIME>
static hipError_t launch_w32_one(const AttnArgs& a, int n_wg, hipStream_t stream,
                                 hipEvent_t start, hipEvent_t stop) {
  auto kern = hstu_attn_fwd_w32_kernel<POSM, TIME>;
  if (start || stop)
    hipExtLaunchKernelGGL(kern, dim3((unsigned)n_wg), dim3(kW32Threads), 0, stream, start, stop,
                          0, a);
  else
    hipLaunchKernelGGL(kern, dim3((unsigned)n_wg), dim3(kW32Threads), 0, stream, a);
  return hipGetLastError();
}

template <int POSM, bool TIME>
static int w32_blocks_per_cu() {
  auto kern = hstu_attn_fwd_w32_kernel<POSM, TIME>;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, kW32Threads, 0) != hipSuccess)
    return -1;
  return nb;
}

bool attn_w32_supported(int dtype, int d_qk, int d_v) {
  return dtype == 1 && d_qk == 128 && d_v == 128;
}

int attn_w32_grid(int pos_len, int time_len, bool clamp) {
  const bool pos = pos_len > 0, tim = time_len > 0;
  int bpc;
  if (pos && clamp && tim) bpc = w32_blocks_per_cu<2, true>();
  else if (pos && clamp) bpc = w32_blocks_per_cu<2, false>();
  else if (pos && tim) bpc = w32_blocks_per_cu<1, true>();
  else if (pos) bpc = w32_blocks_per_cu<1, false>();
  else if (tim) bpc = w32_blocks_per_cu<0, true>();
  else bpc = w32_blocks_per_cu<0, false>();
  if (bpc <= 0) return -1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  return cus * bpc;
}

hipError_t launch_attn_w32(const AttnArgs& a, int n_wg, hipStream_t stream, hipEvent_t t0,
                           hipEvent_t t1) {
  const bool pos = a.pos_len > 0, tim = a.time_len > 0, cl = a.pos_clamp != 0;
  if (pos && cl && tim) return launch_w32_one<2, true>(a, n_wg, stream, t0, t1);
  if (pos && cl) return launch_w32_one<2, false>(a, n_wg, stream, t0, t1);
  if (pos && tim) return launch_w32_one<1, true>(a, n_wg, stream, t0, t1);
  if (pos) return launch_w32_one<1, false>(a, n_wg, stream, t0, t1);
  if (tim) return launch_w32_one<0, true>(a, n_wg, stream, t0, t1);
  return launch_w32_one<0, false>(a, n_wg, stream, t0, t1);
}

}  // namespace hstu
