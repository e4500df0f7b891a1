// attn_bwd.hip -- gfx950 (CDNA4) backward of the jagged HSTU attention.
//
// The forward computes, per (sequence, head) and allowed pair (i, j),
//   x_ij = alpha <q_i, k_j> + pos[min(|i-j|, P-1)] + time[bucket(|t_i - t_j|)]
//   a_ij = SiLU(x_ij) / n_scale,   o_i = sum_j a_ij v_j,   out_i = Norm(o_i) u_i
// (pointwise SiLU aggregation with position/time bias and the Norm-then-U
// gate of "HSTU tensor by tensor: SiLU aggregation, temporal bias and gating",
// sections "SiLU aggregation coefficients are not probabilities", "Relative
// time adds information content similarity lacks", "Similar shape, different
// aggregation").  Training the model end to end ("Scaling HSTU: ragged
// execution, candidate amortization and content features") needs its
// gradients, which follow by the chain rule:
//   gate   du_i, do_i from o_i, u_i and dout_i            (gate kernel)
//   da_ij = <do_i, v_j>,   ds_ij = da_ij SiLU'(x_ij) / n_scale on allowed pairs,
//   SiLU'(x) = sig(x) (1 + x (1 - sig(x))),
//   dq_i = alpha sum_j ds_ij k_j,   dk_j = alpha sum_i ds_ij q_i,
//   dv_j = sum_i a_ij do_i,   dpos[min(|i-j|, P-1)] += ds_ij,  dtime[..] += ds_ij.
// There is no softmax, hence no row statistics to keep: both passes simply
// recompute x from q and k.
//
// Two persistent bf16 MFMA kernels split the work so that every token
// gradient is written by exactly one workgroup (no atomics, deterministic):
//   dQ pass: query tiles of 128 rows (4 waves x 32), keys streamed 32 at a
//     time.  Per wave and key block: S^T = K Q^T and dA^T = V dO^T
//     (v_mfma_f32_32x32x16_bf16, fp32 accumulation), dS^T elementwise, then
//     dQ^T += K^T dS^T.  Q and dO stay in registers as B operands; K and V
//     come through LDS.
//   dK/dV pass: key tiles of 128 keys, query rows streamed 32 at a time.
//     S = Q K^T and dA = dO V^T, then A and dS elementwise, dV^T += dO^T A and
//     dK^T += Q^T dS.  K and V stay in registers; Q and dO come through LDS.
//     This pass also sums the table gradients: per pair into LDS histograms
//     (the position table by |i - j|, the time buckets per lane), written out
//     once per workgroup and added up in a fixed order by a small last kernel.
// In both passes the coefficient tile leaves the first MFMAs in accumulator
// layout, which is the B-operand layout of the aggregation MFMA once the
// staged tile's A operand is read transposed (ds_read_b64_tr_b16) in the
// accumulator's row order.  Tiles are staged by global_load_lds copies two
// steps ahead through three LDS buffers, one barrier per step.
//
// fp32 inputs (small head dims, parity runs) take two plain kernels with one
// wave per (token, head) instead; the table gradients are then accumulated
// with fp32 atomics.
#include <type_traits>

#include "hstu_device.hpp"

namespace hstu {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kStages = 3;                         // LDS buffers of the pipeline
constexpr int kStep = 32;                          // partner tokens per step
constexpr int kDiagN = kBM + kStep - 1;            // distinct i - j of a 128 x 32 block
constexpr int kDiagCp = (kDiagN + 63) / 64;        // 4-byte copies of 64 lanes
constexpr int kTsWave = kWaves - 1 - kDiagCp;      // wave that copies the timestamps
constexpr int64_t kT32Range = int64_t(1) << 30;    // |t - base| below this: 32-bit path
constexpr int kTimeBins = 64;                      // floor(log2(1 + dt)) of 64-bit dt
constexpr int kTabExtra = 64;                      // time-bin slots after the position bins
static_assert(kTsWave >= 0, "enough waves for the bias copies");

__device__ inline uint32_t lds_off(const void* p) { return (uint32_t)(uintptr_t)p; }
__device__ inline lds_shortx4* lds_ptr4(uint32_t off) { return (lds_shortx4*)(uintptr_t)off; }
template <typename V>
__device__ inline V lds_ld(uint32_t off) {
  return *(__attribute__((address_space(3))) const V*)(uintptr_t)off;
}
template <typename V>
__device__ inline void lds_st(uint32_t off, V v) {
  *(__attribute__((address_space(3))) V*)(uintptr_t)off = v;
}
__device__ inline uint64_t uni_ptr(const void* p) {
  const uint64_t x = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ inline int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// HBM -> LDS copies: lane l reads base + voff, its bytes land at `lds` +
// size * l.  From inline assembly so that the compiler neither waits for
// them nor counts them; every wait on them is an explicit wait_vmem.  `base`
// and `lds` are the same in every lane.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void lds_copy16(uint64_t base, uint32_t voff, uint32_t lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(m), "v"(voff), "s"(base) : "memory", "m0");
}
__device__ inline void lds_copy4(uint64_t base, uint32_t voff, uint32_t lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(m), "v"(voff), "s"(base) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N): all but the N most recent global memory operations of
// this wave have completed (they complete in order).
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N < 16, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(N | (7 << 4) | (15 << 8));
}
__device__ inline void wait_vmem_n(int n) {
  switch (n) {
    case 0: wait_vmem<0>(); break;
    case 1: wait_vmem<1>(); break;
    case 2: wait_vmem<2>(); break;
    case 3: wait_vmem<3>(); break;
    case 4: wait_vmem<4>(); break;
    case 5: wait_vmem<5>(); break;
    case 6: wait_vmem<6>(); break;
    default: wait_vmem<7>(); break;
  }
}

// Barrier that waits for this wave's LDS accesses only (lgkmcnt), not for the
// LDS copies of the steps ahead; the caller waited for the copies it needs.
__device__ inline void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool MAX>
__device__ inline int wave_reduce_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const int y = __shfl_xor(x, o, 64);
    x = MAX ? (y > x ? y : x) : (y < x ? y : x);
  }
  return uni(x);
}
__device__ inline uint32_t wave_min_u(uint32_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t y = (uint32_t)__shfl_xor((int)x, o, 64);
    x = y < x ? y : x;
  }
  return (uint32_t)uni((int)x);
}
__device__ inline uint32_t wave_max_u(uint32_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t y = (uint32_t)__shfl_xor((int)x, o, 64);
    x = y > x ? y : x;
  }
  return (uint32_t)uni((int)x);
}
__device__ inline float wave_sum_f(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Register r of a 32x32 accumulator (lane half hh) holds row 8(r/4) + 4hh + r%4.
__device__ constexpr int acc_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

// The lane index as a value the compiler cannot see through: offsets derived
// from it inside the step loop are recomputed there (a few VALU operations)
// instead of being hoisted and kept live in registers for every stage buffer.
__device__ inline int opaque_lane() {
  int l = (int)(threadIdx.x & 63);
  asm volatile("" : "+v"(l));
  return l;
}

// ---------------------------------------------------------------------------
// Scheduler: (sequence, tile) groups sorted by decreasing cost, one list per
// pass, by a counting sort over cost bins in one workgroup.
// ---------------------------------------------------------------------------
constexpr int kPlanT = 1024;
static_assert(kBwdCostBins == kPlanT, "one cost bin per scheduler thread");

__device__ inline int block_excl_scan_i(int x, int* ws, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) ws[wave] = inc;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kPlanT / 64; ++w) {
    const int s = ws[w];
    if (w < wave) pre += s;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return pre + inc - x;
}

__device__ inline int bwd_cost_q(const SeqGeom& g, int t) {
  const int i0 = t * kBM, i1 = min(i0 + kBM, g.L);
  int jlo, jhi;
  tile_key_range(g, i0, i1, jlo, jhi);
  return jhi / kStep - jlo / kStep + 3;
}
__device__ inline int bwd_cost_kv(const SeqGeom& g, int t) {
  const int j0 = t * kBM, j1 = min(j0 + kBM, g.L);
  int rlo, rhi;
  tile_row_range(g, j0, j1, rlo, rhi);
  return rhi / kStep - rlo / kStep + 3;
}

__global__ __launch_bounds__(kPlanT) void hstu_bwd_plan_kernel(BwdPlanArgs a) {
  __shared__ int hq[kBwdCostBins], hkv[kBwdCostBins];
  __shared__ int ws[kPlanT / 64];
  const int tid = threadIdx.x, B = a.num_seqs;
  hq[tid] = 0;
  hkv[tid] = 0;
  int run = 0;
  for (int base = 0; base < B; base += kPlanT) {
    const int b = base + tid;
    const int L = b < B ? a.offsets[b + 1] - a.offsets[b] : 0;
    int tot;
    const int ex = block_excl_scan_i((L + kBM - 1) / kBM, ws, tot);
    if (b < B) a.gstart[b] = run + ex;
    run += tot;
  }
  if (tid == 0) {
    a.gstart[B] = run;
    a.hdr[0] = run;
  }
  __syncthreads();
  const int G = run;
  auto group = [&](int g, int& b, int& t, SeqGeom& geo) {
    int lo = 0, hi = B - 1;   // last b with gstart[b] <= g
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.gstart[mid] <= g) lo = mid; else hi = mid - 1;
    }
    b = lo;
    t = g - a.gstart[b];
    const int L = a.offsets[b + 1] - a.offsets[b];
    geo = seq_geom(L, a.num_targets ? a.num_targets[b] : 0, a.contextual_len, a.max_attn_len);
  };
  for (int g = tid; g < G; g += kPlanT) {
    int b, t;
    SeqGeom geo;
    group(g, b, t, geo);
    atomicAdd(&hq[min(bwd_cost_q(geo, t), kBwdCostBins - 1)], 1);
    atomicAdd(&hkv[min(bwd_cost_kv(geo, t), kBwdCostBins - 1)], 1);
  }
  __syncthreads();
  {   // bin starts in decreasing cost order
    const int bin = kBwdCostBins - 1 - tid;
    int tot;
    const int xq = hq[bin], xkv = hkv[bin];
    const int eq = block_excl_scan_i(xq, ws, tot);
    const int ekv = block_excl_scan_i(xkv, ws, tot);
    hq[bin] = eq;
    hkv[bin] = ekv;
  }
  __syncthreads();
  for (int g = tid; g < G; g += kPlanT) {
    int b, t;
    SeqGeom geo;
    group(g, b, t, geo);
    const int pq = atomicAdd(&hq[min(bwd_cost_q(geo, t), kBwdCostBins - 1)], 1);
    const int pkv = atomicAdd(&hkv[min(bwd_cost_kv(geo, t), kBwdCostBins - 1)], 1);
    a.list_q[pq] = make_int2(b, t);
    a.list_kv[pkv] = make_int2(b, t);
  }
}

// ---------------------------------------------------------------------------
// Gate backward: out = xhat * u with xhat = (o - mean) * rstd over a group of
// `width` values (one head, or all heads of the token):
//   du = dout * xhat,  g = dout * u,  do = rstd (g - mean(g) - xhat mean(g xhat)).
// One wave per (token, group); three passes over the group's values (the
// re-reads hit the cache).
// ---------------------------------------------------------------------------
template <typename T, int EPC>
__device__ inline void ld_chunk(const T* p, float* x) {
  if constexpr (EPC == 8) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
  } else {
    const floatx4 v = *reinterpret_cast<const floatx4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = v[e];
  }
}
template <typename T, int EPC>
__device__ inline void st_chunk(T* p, const float* x) {
  if constexpr (EPC == 8) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)x[e];
    *reinterpret_cast<bf16x8*>(p) = v;
  } else {
    floatx4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = x[e];
    *reinterpret_cast<floatx4*>(p) = v;
  }
}

// G lanes share one group (G a power of two, G * CPL * EPC >= width); a wave
// holds 64 / G groups.  The values stay in registers between the passes.
template <typename T, int EPC, int G, int CPL>
__global__ __launch_bounds__(256) void hstu_gate_bwd_kernel(GateBwdArgs a) {
  const int lane = threadIdx.x & 63, sub = lane & (G - 1);
  const int64_t w = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / G) + lane / G;
  const bool live = w < (int64_t)a.n_tok * a.groups;
  const int64_t ww = live ? w : 0;   // dead groups compute on group 0 and store nothing
  const int64_t t = ww / a.groups;
  const int64_t col = (ww - t * a.groups) * (int64_t)a.width;
  const T* o = static_cast<const T*>(a.o) + t * a.ld_o + col;
  const T* u = static_cast<const T*>(a.u) + t * a.ld_u + col;
  const T* dy = static_cast<const T*>(a.dy) + t * a.ld_dy + col;
  const int chunks = a.width / EPC;
  const float inv_w = 1.0f / (float)a.width;
  auto gsum = [](float x) {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
  };
  float x[CPL][EPC], uu[CPL][EPC], yy[CPL][EPC];
  float sum = 0.0f;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int c = sub + G * k;
    if (c < chunks) {
      ld_chunk<T, EPC>(o + EPC * c, x[k]);
      ld_chunk<T, EPC>(u + EPC * c, uu[k]);
      ld_chunk<T, EPC>(dy + EPC * c, yy[k]);
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) x[k][e] = uu[k][e] = yy[k][e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) sum += x[k][e];
  }
  const float mean = gsum(sum) * inv_w;
  float sq = 0.0f, sg = 0.0f, sgx = 0.0f;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    if (sub + G * k >= chunks) continue;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const float xc = x[k][e] - mean, g = yy[k][e] * uu[k][e];
      sq += xc * xc;
      sg += g;
      sgx += g * xc;
    }
  }
  const float rstd = rsqrtf(gsum(sq) * inv_w + a.eps);
  const float mg = gsum(sg) * inv_w;
  const float mgx = gsum(sgx) * inv_w * rstd;   // mean(g * xhat)
  if (!live) return;
  T* du = static_cast<T*>(a.du) + t * a.ld_u + col;
  T* d_o = static_cast<T*>(a.d_o) + t * a.ld_o + col;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int c = sub + G * k;
    if (c >= chunks) continue;
    float r0[EPC], r1[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const float xh = (x[k][e] - mean) * rstd;
      r0[e] = yy[k][e] * xh;
      r1[e] = rstd * (yy[k][e] * uu[k][e] - mg - xh * mgx);
    }
    st_chunk<T, EPC>(du + EPC * c, r0);
    st_chunk<T, EPC>(d_o + EPC * c, r1);
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA passes.
// ---------------------------------------------------------------------------
template <int D>
struct BCfg {
  static constexpr int kRow = 2 * D;                      // bytes of a staged row
  static constexpr int kCh = D / 8;                       // 16-byte chunks per row
  static constexpr int kNC = D / 16;                      // MFMA steps over d
  static constexpr int kNDB = D / 32;                     // 32-wide blocks of d
  static constexpr int kTileCp = kStep * kCh / 64;        // 64-lane copies per tile
  static constexpr int kCpW = (kTileCp + kWaves - 1) / kWaves;
  static_assert(D == 64 || D == 128, "bf16 backward: d = 64 or 128");
  // XOR swizzle of a staged row's 16-byte chunks, one for both access
  // patterns: a row read touches one logical chunk of 8 consecutive rows per
  // LDS cycle (distinct banks), a transposed read 4 consecutive chunks of 4
  // rows (distinct banks as well).
  __device__ static int swz(int r) {
    return kCh >= 16 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
};

// DX: head size of the x rows (K or Q: d_qk), DY: of the y rows (V or dO: d_v).
template <int DX, int DY>
struct BStage {
  char x[kStep * 2 * DX];      // K (dQ pass) or Q (dK/dV pass) rows, chunks swizzled
  char y[kStep * 2 * DY];      // V or dO rows
  float diag[kDiagCp * 64];    // position bias by i - j (scaled), see diag_rel
  int64_t ts64[kStep];         // raw partner timestamps
  uint32_t ts32[kStep];        // partner timestamps relative to the item's base
  uint32_t tmin, tmax;         // range of ts32 over the valid partners
  int tbad;                    // some partner needs the 64-bit time path
  int pad_;
  float cpos[64];              // dQ pass, clamped positions: bias of key (lane % 32),
                               // pos[min(max(n_h - j, 0), P-1)] (scaled)
};

__host__ __device__ constexpr int copies_of_wave(int count, int w) {
  return count > w ? (count - w + kWaves - 1) / kWaves : 0;
}

// Shared pipeline machinery of both passes.  The fixed side (the item's 128
// tokens: query rows in the dQ pass, keys in the dK/dV pass) belongs to the
// lanes, 32 per wave; the partner side is streamed 32 tokens per step.
// diag: entry f of a step holds pos[min(|i - j|, P-1)] / am for
//   i - j = dc + ds * f  (dQ: dc = i0 - j0 + 127, ds = -1; dK/dV: dc = ib -
//   j0 - 127, ds = +1), and the lane of fixed token 32w + l32 finds register
//   r's partner at f = dbase + 8(r/4) + r%4, dbase = 127 - 32w - l32 + 4hh.
// CPS: the dQ pass with the position bias at clamped positions (each step
// also gathers the bias of its keys at the candidates' position n_h).
template <int DX, int DY, bool POS, bool TIME, bool CPS = false>
struct Pipe {
  using CX = BCfg<DX>;   // x rows (d_qk)
  using CY = BCfg<DY>;   // y rows (d_v)
  using SB = BStage<DX, DY>;
  SB* st;                 // kStages buffers
  const float* trev;      // trev[z] = time[min(31 - z, Tt - 1)], z = clz(1 + |dt|)
  const float* tful;      // tful[b] = time[min(b, Tt - 1)]
  int wave, lane;
  int P;
  float pscale;
  uint32_t xoff[CX::kCpW], yoff[CY::kCpW];
  uint32_t ldx_b, ldy_b;
  int my_copies;
  static constexpr bool cp_stage = POS && CPS;
  int n_h;   // history length of the current item (cp_stage)
  // fixed-side times
  int64_t tbase;
  uint32_t tf32;
  bool w_t_ok;
  uint32_t w_tmin, w_tmax;

  __device__ void init(SB* s, const float* tr, const float* tf, int w, int l, int pos_len,
                       float ps, int64_t ldx, int64_t ldy) {
    st = s;
    n_h = 0;
    trev = tr;
    tful = tf;
    wave = w;
    lane = l;
    P = pos_len;
    pscale = ps;
    ldx_b = (uint32_t)(ldx * 2);
    ldy_b = (uint32_t)(ldy * 2);
#pragma unroll
    for (int s2 = 0; s2 < CX::kCpW; ++s2) {
      const int m = 64 * (s2 * kWaves + wave) + lane, row = m / CX::kCh;
      xoff[s2] = (uint32_t)row * ldx_b + 16u * (uint32_t)((m % CX::kCh) ^ CX::swz(row));
    }
#pragma unroll
    for (int s2 = 0; s2 < CY::kCpW; ++s2) {
      const int m = 64 * (s2 * kWaves + wave) + lane, row = m / CY::kCh;
      yoff[s2] = (uint32_t)row * ldy_b + 16u * (uint32_t)((m % CY::kCh) ^ CY::swz(row));
    }
    my_copies = copies_of_wave(CX::kTileCp, wave) + copies_of_wave(CY::kTileCp, wave) +
                ((POS && wave > kTsWave) ? 1 : 0) +
                ((TIME && wave == kTsWave) ? 1 : 0) + ((cp_stage && wave == kTsWave) ? 1 : 0);
  }

  // Copy partner tokens [p0, p0 + 32) of sequence length L (rows past the
  // end repeat the last row: finite values whose coefficients are masked to
  // 0) and the step's position-bias values into buffer b.
  __device__ void issue(int b, uint64_t xbase, uint64_t ybase, int p0, int L, uint64_t pos_base,
                        int dc, int dsgn, uint64_t ts_base) {
    SB& sb = st[b];
    const bool whole = p0 + kStep <= L;
    const uint64_t xb = xbase + (uint64_t)p0 * ldx_b, yb = ybase + (uint64_t)p0 * ldy_b;
#pragma unroll
    for (int s2 = 0; s2 < CX::kCpW; ++s2) {
      const int n = s2 * kWaves + wave;
      if (n < CX::kTileCp) {
        uint32_t ox = xoff[s2];
        if (!whole) {
          const int m = 64 * n + lane, row = m / CX::kCh;
          const uint32_t rr = (uint32_t)min(row, L - 1 - p0);
          ox = rr * ldx_b + 16u * (uint32_t)((m % CX::kCh) ^ CX::swz(row));
        }
        lds_copy16(xb, ox, lds_off(sb.x) + 1024u * (uint32_t)n);
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < CY::kCpW; ++s2) {
      const int n = s2 * kWaves + wave;
      if (n < CY::kTileCp) {
        uint32_t oy = yoff[s2];
        if (!whole) {
          const int m = 64 * n + lane, row = m / CY::kCh;
          const uint32_t rr = (uint32_t)min(row, L - 1 - p0);
          oy = rr * ldy_b + 16u * (uint32_t)((m % CY::kCh) ^ CY::swz(row));
        }
        lds_copy16(yb, oy, lds_off(sb.y) + 1024u * (uint32_t)n);
      }
    }
    if constexpr (POS) {
      if (wave > kTsWave) {
        const int p = kWaves - 1 - wave;
        const int d = dc + dsgn * (64 * p + lane);
        const int ix = min(d < 0 ? -d : d, P - 1);
        lds_copy4(pos_base, 4u * (uint32_t)ix, lds_off(sb.diag) + 256u * (uint32_t)p);
      }
      if (cp_stage && wave == kTsWave) {   // bias of n_h - j (0 for candidate keys)
        const int d = n_h - (p0 + (lane & (kStep - 1)));
        const int ix = min(d > 0 ? d : 0, P - 1);
        lds_copy4(pos_base, 4u * (uint32_t)ix, lds_off(sb.cpos));
      }
    }
    if constexpr (TIME) {
      if (wave == kTsWave) {
        const int j = min(p0 + (lane >> 1), L - 1);
        lds_copy4(ts_base, 8u * (uint32_t)j + 4u * (uint32_t)(lane & 1), lds_off(sb.ts64));
      }
    }
  }

  // Once this wave's own copies of buffer b have landed: scale the position
  // bias it gathered; form the partner times relative to tbase, their range
  // and whether any needs the 64-bit path.
  __device__ void finish(int b, int p0, int L) {
    SB& sb = st[b];
    if constexpr (POS) {
      if (wave > kTsWave) {
        const int e = 64 * (kWaves - 1 - wave) + lane;
        if (e < kDiagN) sb.diag[e] *= pscale;
      }
      if (cp_stage && wave == kTsWave) sb.cpos[lane] *= pscale;
    }
    if constexpr (TIME) {
      if (wave == kTsWave) {
        const int kl = lane & (kStep - 1);
        const int64_t tj = sb.ts64[kl];
        const int64_t rel = tj - tbase;
        const bool ok = rel > -kT32Range && rel < kT32Range;
        const uint32_t t32 = ok ? uint32_t(rel + kT32Range) : 0u;
        const int nvalid = min(kStep, L - p0);
        if (lane < kStep) sb.ts32[kl] = t32;
        const bool bad = __ballot(!ok) != 0;
        // When the valid partner times ascend (as times along a sequence
        // usually do) their range is [first, last]; otherwise the step
        // claims every 32-bit time, so no pair is taken for a shared bucket.
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
  }

  // Fixed-side times of this lane's token (t_fix) and the wave's range.
  __device__ void set_fixed_times(int64_t base, int64_t t_fix, bool valid) {
    tbase = base;
    const int64_t rel = t_fix - base;
    const bool ok = rel > -kT32Range && rel < kT32Range;
    tf32 = ok ? uint32_t(rel + kT32Range) : 0u;
    w_t_ok = __all(ok);
    w_tmin = wave_min_u(valid ? tf32 : 0xffffffffu);
    w_tmax = wave_max_u(valid ? tf32 : 0u);
  }

  // The buckets the step's (fixed, partner) time gaps can fall in: every gap
  // of a valid pair lies in [dmin, dmax] of the two time ranges, so its
  // clz(1 + dt) lies in [z1, z0].  False when some time needs 64 bits.
  __device__ bool time_span(const SB& sb, int& z0, int& z1) const {
    if (!w_t_ok || uni(sb.tbad) != 0) return false;
    const uint32_t kmin = (uint32_t)uni((int)sb.tmin), kmax = (uint32_t)uni((int)sb.tmax);
    uint32_t dmin = 0;
    if (w_tmin > kmax) dmin = w_tmin - kmax;
    if (kmin > w_tmax) dmin = kmin - w_tmax;
    const uint32_t dmax = max(w_tmax > kmin ? w_tmax - kmin : 0u,
                              kmax > w_tmin ? kmax - w_tmin : 0u);
    z0 = uni(__builtin_clz(dmin + 1u));
    z1 = uni(__builtin_clz(dmax + 1u));
    return true;
  }

  // How a step's time bias is found, for this wave: 0 = no time bias, or
  // one bucket for every pair of the step (its value tb and bin cb); 3 = two
  // adjacent buckets, told apart by one compare per pair (tb and cb are the
  // lower one's, t_hi and t_thr the upper one's value and first gap + 1);
  // 1 = per pair from 32-bit times and the table; 2 = per pair from 64-bit
  // times.
  __device__ int time_mode(const SB& sb, float& tb, int& cb) {
    tb = 0.0f;
    cb = 0;
    if constexpr (TIME) {
      int z0, z1;
      if (!time_span(sb, z0, z1)) return 2;
      tb = __builtin_bit_cast(float, uni(__builtin_bit_cast(int, trev[z0])));
      cb = 31 - z0;
      if (z0 == z1) return 0;
      if (z0 != z1 + 1) return 1;
      t_hi = __builtin_bit_cast(float, uni(__builtin_bit_cast(int, trev[z1])));
      t_thr = 1u << (31 - z1);
      return 3;
    }
    return 0;
  }
  float t_hi;
  uint32_t t_thr;
  // Time bias and bin of register r's pair (modes 1, 2 and 3); t4 holds the
  // 32-bit partner times of registers 4(r/4) .. 4(r/4)+3.  Mode 3 takes cb
  // (the lower bin) and tb (its value).
  template <int MODE>
  __device__ float pair_time(const SB& sb, const uint4& t4, int r, int hh, int64_t t_fix64,
                             int& bin, int cb = 0, float tb = 0.0f) const {
    if constexpr (MODE == 1 || MODE == 3) {
      const int e = r & 3;
      const uint32_t tv = e == 0 ? t4.x : (e == 1 ? t4.y : (e == 2 ? t4.z : t4.w));
      const uint32_t d1 = (tf32 > tv ? tf32 - tv : tv - tf32) + 1u;
      if constexpr (MODE == 3) {
        const bool up = d1 >= t_thr;
        bin = cb + (up ? 1 : 0);
        return up ? t_hi : tb;
      }
      const int z = __builtin_clz(d1);
      bin = 31 - z;
      return trev[z];
    } else {
      const int64_t tj = sb.ts64[acc_row(r, hh)];
      const uint64_t dt = t_fix64 >= tj ? uint64_t(t_fix64) - uint64_t(tj)
                                        : uint64_t(tj) - uint64_t(t_fix64);
      const uint64_t d1 = dt + 1u;   // 0 only for a gap of 2^64 - 1
      bin = d1 ? 63 - __builtin_clzll(d1) : 63;
      return tful[bin];
    }
  }

  // Accumulator init: the step's position bias (or 0).
  __device__ floatx16 diag_init(const SB& sb, int dbase) const {
    floatx16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (POS) s[r] = sb.diag[dbase + 8 * (r >> 2) + (r & 3)];
      else s[r] = 0.0f;
    }
    return s;
  }

  // acc += tile rows (A, row reads) x f (B operands in registers), over the
  // d of side CC, with the operand reads issued in two halves.
  template <typename CC>
  __device__ static floatx16 contract(uint32_t tile, int l32, int hh, const bf16x8* f,
                                      floatx16 acc) {
    constexpr int NH = CC::kNC / 2;
    bf16x8 op[NH];
#pragma unroll
    for (int c = 0; c < NH; ++c) op[c] = row_op<CC>(tile, l32, hh, c);
#pragma unroll
    for (int c = 0; c < NH; ++c)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[c], f[c], acc, 0, 0, 0);
#pragma unroll
    for (int c = 0; c < NH; ++c) op[c] = row_op<CC>(tile, l32, hh, NH + c);
#pragma unroll
    for (int c = 0; c < NH; ++c)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[c], f[NH + c], acc, 0, 0, 0);
    return acc;
  }

  // Row-read A operand (rows l32 of a staged tile, logical chunk 2c + hh).
  template <typename CC>
  __device__ static bf16x8 row_op(uint32_t tile, int l32, int hh, int c) {
    return lds_ld<bf16x8>(tile + (uint32_t)(l32 * CC::kRow) +
                          16u * (uint32_t)((2 * c + hh) ^ CC::swz(l32)));
  }
  // Transposed A operand of d-block db and contraction block ins: lane
  // (e = 32 db + l32, half hh) gets the tile's rows 16 ins + 4hh + {0..3} and
  // 16 ins + 8 + 4hh + {0..3} at column e -- the accumulator rows of the
  // coefficients it multiplies.  ds_read_b64_tr_b16: in each 16-lane group,
  // lane 4e'+q reads 4 values of row e' at columns 4q..4q+3 of the group's 16
  // columns, and lane c of the group receives column c of the 4 rows.
  template <typename CC>
  __device__ static bf16x8 tr_op(uint32_t tile, int lane, int db, int ins) {
    const int gl = lane & 15, grp = lane >> 4, er = gl >> 2, h2 = lane >> 5;
    const int col = 32 * db + 16 * (grp & 1) + 4 * (gl & 3);
    const int r0 = 16 * ins + 4 * h2 + er, r1 = r0 + 8;
    const uint32_t a0 = tile + (uint32_t)(r0 * CC::kRow) +
                        16u * (uint32_t)((col >> 3) ^ CC::swz(r0)) + 2u * (uint32_t)(col & 7);
    const uint32_t a1 = tile + (uint32_t)(r1 * CC::kRow) +
                        16u * (uint32_t)((col >> 3) ^ CC::swz(r1)) + 2u * (uint32_t)(col & 7);
    const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr4(a0));
    const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr4(a1));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// SiLU and its derivative: sig = 1 / (1 + e^-x).
__device__ inline float sigm(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * x));
}

// CL: position bias at the clamped positions min(position, n_h).
template <int DQK, int DV, bool POS, bool TIME, bool CL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void
hstu_bwd_dq_kernel(BwdArgs a) {
  using CX = BCfg<DQK>;   // K rows
  using CY = BCfg<DV>;    // V rows
  using SB = BStage<DQK, DV>;
  using PP = Pipe<DQK, DV, POS, TIME, CL>;
  constexpr int NCX = CX::kNC, NCY = CY::kNC, NDB = CX::kNDB;
  __shared__ __align__(16) SB st[kStages];
  __shared__ float trev[32], tful[64];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = uni(tid >> 6);
  const int H = a.num_heads;
  const bool alpha_zero = a.alpha == 0.0f;
  const float am = alpha_zero ? 1.0f : a.alpha;
  if constexpr (TIME) {
    const int Tt = a.time_len;
    if (tid < 32) trev[tid] = a.time_table[min(31 - tid, Tt - 1)];
    if (tid < 64) tful[tid] = a.time_table[min(tid, Tt - 1)];
  }
  PP pp;
  pp.init(st, trev, tful, wave, lane, a.pos_len, 1.0f / am, a.ld_k, a.ld_v);
  const float out_scale = a.alpha * a.inv_scale;

  const int n_items = a.hdr[0] * H;
  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int2 gp = a.list[it / H];
    const int h = it - (it / H) * H;
    const int seq0 = a.offsets[gp.x];
    const int L = a.offsets[gp.x + 1] - seq0;
    const SeqGeom geo = seq_geom(L, a.num_targets ? a.num_targets[gp.x] : 0, a.contextual_len,
                                 a.max_attn_len);
    const int i0 = gp.y * kBM, i1 = min(i0 + kBM, L);
    int jlo, jhi;
    tile_key_range(geo, i0, i1, jlo, jhi);
    const int kt_lo = jlo / kStep, kt_hi = jhi / kStep;

    const int wr0 = i0 + 32 * wave, i = wr0 + l32;
    const bool row_valid = i < i1, wave_rows = wr0 < i1;
    pp.n_h = geo.n_h;
    // rows of candidates take the bias of the clamped positions from cpos
    const bool w_cand = PP::cp_stage && wave_rows && wr0 + 31 >= geo.n_h;
    int w_jmin, w_jmax, w_lomax, w_himin;
    const RowBounds rb = row_valid ? row_bounds(geo, i) : RowBounds{kEmptyLo, 0, -1};
    {
      const bool nonempty = rb.lo != kEmptyLo;
      const int hi = rb.lo + rb.span;
      int jmin = nonempty ? rb.lo : (rb.self_j >= 0 ? rb.self_j : 0x7fffffff);
      int jmax = nonempty ? max(hi, rb.self_j) : rb.self_j;
      if (!row_valid) {
        jmin = 0x7fffffff;
        jmax = -1;
      }
      w_jmin = wave_reduce_i<false>(jmin);
      w_jmax = wave_reduce_i<true>(jmax);
      w_lomax = wave_reduce_i<true>(row_valid ? rb.lo : 0x7fffffff);
      w_himin = wave_reduce_i<false>(row_valid && nonempty ? hi : -1);
    }

    const uint64_t kseq = uni_ptr(reinterpret_cast<const char*>(a.k) +
                                  ((int64_t)seq0 * a.ld_k + (int64_t)h * DQK) * 2);
    const uint64_t vseq = uni_ptr(reinterpret_cast<const char*>(a.v) +
                                  ((int64_t)seq0 * a.ld_v + (int64_t)h * DV) * 2);
    const uint64_t pos_base = POS ? uni_ptr(a.pos_table) : 0;
    const uint64_t ts_base = TIME ? uni_ptr(a.timestamps + seq0) : 0;
    auto issue = [&](int b, int kt) __attribute__((always_inline)) {
      const int j0 = kt * kStep;
      pp.issue(b, kseq, vseq, j0, L, pos_base, i0 - j0 + (kBM - 1), -1, ts_base);
    };

    issue(0, kt_lo);
    if (kt_lo + 1 <= kt_hi) issue(1, kt_lo + 1);
    // Q and dO rows of this lane (B operands), row times
    bf16x8 qf[NCX], dof[NCY];
    {
      const int ir = min(i, i1 - 1);
      const char* qrow = reinterpret_cast<const char*>(a.q) +
                         ((int64_t)(seq0 + ir) * a.ld_q + (int64_t)h * DQK) * 2;
      const char* drow = reinterpret_cast<const char*>(a.dout) +
                         ((int64_t)(seq0 + ir) * a.ld_do + (int64_t)h * DV) * 2;
      const bf16x8 z = {};
#pragma unroll
      for (int c = 0; c < NCX; ++c) {
        const bf16x8 qv = *reinterpret_cast<const bf16x8*>(qrow + 16 * (2 * c + hh));
        qf[c] = (row_valid && !alpha_zero) ? qv : z;
      }
#pragma unroll
      for (int c = 0; c < NCY; ++c) {
        const bf16x8 dv = *reinterpret_cast<const bf16x8*>(drow + 16 * (2 * c + hh));
        dof[c] = row_valid ? dv : z;
      }
    }
    int64_t ti64 = 0;
    if constexpr (TIME) {
      const int64_t base = a.timestamps[seq0 + i0];
      ti64 = a.timestamps[seq0 + min(i, i1 - 1)];
      wait_vmem<0>();
      pp.set_fixed_times(base, ti64, row_valid);
    }
    wait_vmem<0>();
    pp.finish(0, kt_lo * kStep, L);
    stage_barrier();

    floatx16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

    int b = 0;
    for (int kt = kt_lo; kt <= kt_hi; ++kt) {
      const int b1 = b == kStages - 1 ? 0 : b + 1, b2 = b1 == kStages - 1 ? 0 : b1 + 1;
      const bool more2 = kt + 2 <= kt_hi;
      if (more2) issue(b2, kt + 2);
      if (kt + 1 <= kt_hi) {
        wait_vmem_n(more2 ? pp.my_copies : 0);
        pp.finish(b1, (kt + 1) * kStep, L);
      }
      const int jb = kt * kStep;
      if (wave_rows && jb <= w_jmax && jb + kStep - 1 >= w_jmin) {
        const SB& sb = st[b];
        const uint32_t xt = lds_off(sb.x), yt = lds_off(sb.y);
        const int ol = opaque_lane(), ol32 = ol & 31, ohh = ol >> 5;
        floatx16 s = pp.diag_init(sb, (kBM - 1) - 32 * wave - ol32 + 4 * ohh);
        if (PP::cp_stage && w_cand) {
          const bool cr = i >= geo.n_h;
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = cr ? sb.cpos[acc_row(r, ohh)] : s[r];
        }
        s = PP::template contract<CX>(xt, ol32, ohh, qf, s);
        __builtin_amdgcn_sched_barrier(0);
        floatx16 da = {};
        da = PP::template contract<CY>(yt, ol32, ohh, dof, da);
        __builtin_amdgcn_sched_barrier(0);

        // dS^T = dA^T SiLU'(x), zero on illegal pairs (time bias, SiLU'
        // and mask fused per register)
        float ds[16];
        {
          float tb;
          int cbin;
          const int mode = pp.time_mode(sb, tb, cbin);
          const bool full = w_lomax <= jb && w_himin >= jb + kStep - 1;
          const int jl = jb + 4 * hh - rb.lo, js = jb + 4 * hh - rb.self_j;
          auto elem = [&](auto mc) __attribute__((always_inline)) {
            constexpr int MODE = decltype(mc)::value;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              uint4 t4 = {};
              if constexpr (MODE == 1 || MODE == 3)
                t4 = *reinterpret_cast<const uint4*>(&sb.ts32[8 * gq + 4 * hh]);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * gq + e;
                int bin;
                const float t =
                    MODE == 0 ? tb : pp.template pair_time<MODE>(sb, t4, r, hh, ti64, bin, cbin, tb);
                const float x = fmaf(s[r], am, t);
                const float sg = sigm(x);
                float d = da[r] * (sg * fmaf(x, 1.0f - sg, 1.0f));
                if (!full) {
                  const int kk = 8 * gq + e;
                  const bool ok = (uint32_t)(jl + kk) <= (uint32_t)rb.span || js + kk == 0;
                  d = ok ? d : 0.0f;
                }
                ds[r] = d;
              }
            }
          };
          if (mode == 0) elem(std::integral_constant<int, 0>{});
          else if (mode == 3) elem(std::integral_constant<int, 3>{});
          else if (mode == 1) elem(std::integral_constant<int, 1>{});
          else elem(std::integral_constant<int, 2>{});
        }
        bf16x8 pd[2];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pd[0][e] = (__bf16)ds[e];
          pd[1][e] = (__bf16)ds[8 + e];
        }
        __builtin_amdgcn_sched_barrier(0);
        // dQ^T += K^T dS^T, two d-blocks of operands in flight at a time
#pragma unroll
        for (int db = 0; db < NDB; db += 2) {
          bf16x8 kt4[4];
#pragma unroll
          for (int u2 = 0; u2 < 2; ++u2)
#pragma unroll
            for (int ins = 0; ins < 2; ++ins)
              kt4[2 * u2 + ins] = PP::template tr_op<CX>(xt, ol, db + u2, ins);
#pragma unroll
          for (int u2 = 0; u2 < 2; ++u2)
#pragma unroll
            for (int ins = 0; ins < 2; ++ins)
              acc[db + u2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt4[2 * u2 + ins], pd[ins],
                                                                    acc[db + u2], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (kt + 1 <= kt_hi) stage_barrier();
      b = b1;
    }

    // dq row i: acc[db][r] holds d-index 32 db + acc_row(r, hh)
    if (row_valid) {
      char* dst =
          reinterpret_cast<char*>(a.dq) + ((int64_t)(seq0 + i) * a.ld_q + (int64_t)h * DQK) * 2;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (__bf16)(acc[db][4 * g + e] * out_scale);
          *reinterpret_cast<bf16x4*>(dst + 2 * (32 * db + 8 * g + 4 * hh)) = o;
        }
    }
    stage_barrier();   // the next item's copies may refill every buffer
  }
}

// M: 0 = dK, dV and the table sums in one pass; 1 = dK and the table sums;
// 2 = dV only.  At d = 128 the fused pass would need more registers than two
// waves per SIMD leave (K and V operands plus two 32 x 128 fp32
// accumulators), so it runs as passes 1 and 2, which recompute S.
template <int DQK, int DVV, bool POS, bool TIME, int M, bool CL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void
hstu_bwd_dkv_kernel(BwdArgs a) {
  constexpr bool DK = M != 2, DV = M != 1, TABS = DK;
  using CX = BCfg<DQK>;   // Q rows
  using CY = BCfg<DVV>;   // dO rows
  using SB = BStage<DQK, DVV>;
  using PP = Pipe<DQK, DVV, POS, TIME>;
  constexpr int NCX = CX::kNC, NCY = CY::kNC, NDBX = CX::kNDB, NDBY = CY::kNDB;
  constexpr int NDBM = NDBX > NDBY ? NDBX : NDBY;
  __shared__ __align__(16) SB st[kStages];
  __shared__ float trev[32], tful[64];
  __shared__ float htime[(TIME && TABS) ? kTimeBins * 32 : 1];   // [bin][lane % 32]
  extern __shared__ float hpos[];                      // [pos_len] (POS && TABS only)

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = uni(tid >> 6);
  const int H = a.num_heads, P = a.pos_len;
  const bool alpha_zero = a.alpha == 0.0f;
  const float am = alpha_zero ? 1.0f : a.alpha;
  if constexpr (TIME) {
    const int Tt = a.time_len;
    if (tid < 32) trev[tid] = a.time_table[min(31 - tid, Tt - 1)];
    if (tid < 64) tful[tid] = a.time_table[min(tid, Tt - 1)];
    if constexpr (TABS)
      for (int e = tid; e < kTimeBins * 32; e += kThreads) htime[e] = 0.0f;
  }
  if constexpr (POS && TABS)
    for (int e = tid; e < P; e += kThreads) hpos[e] = 0.0f;
  PP pp;
  pp.init(st, trev, tful, wave, lane, P, 1.0f / am, a.ld_q, a.ld_do);
  const float k_scale = a.alpha * a.inv_scale, v_scale = a.inv_scale;

  const int n_items = a.hdr[0] * H;
  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int2 gp = a.list[it / H];
    const int h = it - (it / H) * H;
    const int seq0 = a.offsets[gp.x];
    const int L = a.offsets[gp.x + 1] - seq0;
    const SeqGeom geo = seq_geom(L, a.num_targets ? a.num_targets[gp.x] : 0, a.contextual_len,
                                 a.max_attn_len);
    const int j0 = gp.y * kBM, j1 = min(j0 + kBM, L);
    int rlo, rhi;
    tile_row_range(geo, j0, j1, rlo, rhi);
    const int st_lo = rlo / kStep, st_hi = rhi / kStep;

    const int wk0 = j0 + 32 * wave, j = wk0 + l32;
    const bool key_valid = j < j1, wave_keys = wk0 < j1;
    const RowBounds cb = key_valid ? col_bounds(geo, j) : RowBounds{kEmptyLo, 0, -1};
    // Position bias at clamped positions: candidate rows i >= n_h see this
    // lane's key j at pos[min(max(n_h - j, 0), P-1)] (one value per lane);
    // their share of the position-table gradient collects in cacc.
    constexpr bool clamp = POS && CL;
    int c_ix = 0;
    float c_bias = 0.0f, cacc = 0.0f;
    if constexpr (clamp) {
      const int d = geo.n_h - j;
      c_ix = min(d > 0 ? d : 0, P - 1);
      c_bias = a.pos_table[c_ix] * (1.0f / am);
    }
    int w_rmin, w_rmax, w_lomax, w_himin;
    {
      const bool nonempty = cb.lo != kEmptyLo;
      const int hi = cb.lo + cb.span;
      int rmin = nonempty ? cb.lo : (cb.self_j >= 0 ? cb.self_j : 0x7fffffff);
      int rmax = nonempty ? max(hi, cb.self_j) : cb.self_j;
      if (!key_valid) {
        rmin = 0x7fffffff;
        rmax = -1;
      }
      w_rmin = wave_reduce_i<false>(rmin);
      w_rmax = wave_reduce_i<true>(rmax);
      w_lomax = wave_reduce_i<true>(key_valid && nonempty ? cb.lo : 0x7fffffff);
      w_himin = wave_reduce_i<false>(key_valid && nonempty ? hi : -1);
    }

    const uint64_t qseq = uni_ptr(reinterpret_cast<const char*>(a.q) +
                                  ((int64_t)seq0 * a.ld_q + (int64_t)h * DQK) * 2);
    const uint64_t dseq = uni_ptr(reinterpret_cast<const char*>(a.dout) +
                                  ((int64_t)seq0 * a.ld_do + (int64_t)h * DVV) * 2);
    const uint64_t pos_base = POS ? uni_ptr(a.pos_table) : 0;
    const uint64_t ts_base = TIME ? uni_ptr(a.timestamps + seq0) : 0;
    auto issue = [&](int b, int stp) __attribute__((always_inline)) {
      const int ib = stp * kStep;
      pp.issue(b, qseq, dseq, ib, L, pos_base, ib - j0 - (kBM - 1), 1, ts_base);
    };

    issue(0, st_lo);
    if (st_lo + 1 <= st_hi) issue(1, st_lo + 1);
    // K and V rows of this lane's key (B operands), key times
    bf16x8 kf[NCX], vf[DK ? NCY : 1];
    {
      const int jr = min(j, j1 - 1);
      const char* krow = reinterpret_cast<const char*>(a.k) +
                         ((int64_t)(seq0 + jr) * a.ld_k + (int64_t)h * DQK) * 2;
      const char* vrow = reinterpret_cast<const char*>(a.v) +
                         ((int64_t)(seq0 + jr) * a.ld_v + (int64_t)h * DVV) * 2;
      const bf16x8 z = {};
#pragma unroll
      for (int c = 0; c < NCX; ++c) {
        const bf16x8 kv = *reinterpret_cast<const bf16x8*>(krow + 16 * (2 * c + hh));
        kf[c] = (key_valid && !alpha_zero) ? kv : z;
      }
      if constexpr (DK) {
#pragma unroll
        for (int c = 0; c < NCY; ++c) {
          const bf16x8 vv = *reinterpret_cast<const bf16x8*>(vrow + 16 * (2 * c + hh));
          vf[c] = key_valid ? vv : z;
        }
      }
    }
    int64_t tj64 = 0;
    if constexpr (TIME) {
      const int64_t base = a.timestamps[seq0 + j0];
      tj64 = a.timestamps[seq0 + min(j, j1 - 1)];
      wait_vmem<0>();
      pp.set_fixed_times(base, tj64, key_valid);
    }
    wait_vmem<0>();
    pp.finish(0, st_lo * kStep, L);
    stage_barrier();

    floatx16 acck[DK ? NDBX : 1], accv[DV ? NDBY : 1];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (DK)
#pragma unroll
        for (int db = 0; db < NDBX; ++db) acck[db][r] = 0.0f;
      if constexpr (DV)
#pragma unroll
        for (int db = 0; db < NDBY; ++db) accv[db][r] = 0.0f;
    }

    int b = 0;
    for (int stp = st_lo; stp <= st_hi; ++stp) {
      const int b1 = b == kStages - 1 ? 0 : b + 1, b2 = b1 == kStages - 1 ? 0 : b1 + 1;
      const bool more2 = stp + 2 <= st_hi;
      if (more2) issue(b2, stp + 2);
      if (stp + 1 <= st_hi) {
        wait_vmem_n(more2 ? pp.my_copies : 0);
        pp.finish(b1, (stp + 1) * kStep, L);
      }
      const int ib = stp * kStep;
      if (wave_keys && ib <= w_rmax && ib + kStep - 1 >= w_rmin) {
        const SB& sb = st[b];
        const uint32_t xt = lds_off(sb.x), yt = lds_off(sb.y);
        const int ol = opaque_lane(), ol32 = ol & 31, ohh = ol >> 5;
        // S[i][j] (rows in registers, this lane's key in the column)
        floatx16 s = pp.diag_init(sb, (kBM - 1) - 32 * wave - ol32 + 4 * ohh);
        const bool step_cand = clamp && ib + kStep - 1 >= geo.n_h;
        if (step_cand) {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = ib + acc_row(r, ohh) >= geo.n_h ? c_bias : s[r];
        }
        s = PP::template contract<CX>(xt, ol32, ohh, kf, s);
        __builtin_amdgcn_sched_barrier(0);
        floatx16 da = {};
        if constexpr (DK) {
          da = PP::template contract<CY>(yt, ol32, ohh, vf, da);
          __builtin_amdgcn_sched_barrier(0);
        }
        // A and dS (time bias, SiLU, SiLU', mask, bf16 packing and the table
        // sums fused per register group)
        bf16x8 pa[2], pd[2];
        {
          float tb;
          int cbin;
          const int mode = pp.time_mode(sb, tb, cbin);
          const bool full = w_lomax <= ib && w_himin >= ib + kStep - 1;
          const int il = ib + 4 * hh - cb.lo, is = ib + 4 * hh - cb.self_j;
          const int R0 = ib - wk0;   // i - j of register r: R0 + acc_row(r, hh) - l32
          // Time-bin sums: a lane's registers run over rows in increasing
          // order, along which the bin of |t_i - t_j| changes only a few
          // times when times grow with position, so each lane adds up runs
          // of equal bins and touches the LDS sums only where a run ends.
          auto tflush = [&](int bin, float v) __attribute__((always_inline)) {
            if (v != 0.0f)
              __hip_atomic_fetch_add(&htime[bin * 32 + ol32], v, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_WORKGROUP);
          };
          // Position-bin sums: the step's 32 x 32 block has 63 distinct
          // i - j = R0 + delta, delta = row - key in [-31, 31]; register 4g+e
          // of lane (c, hh) holds delta = 8g + 4hh + e - c.  Three rounds of
          // lane exchanges (ds_bpermute) gather the block into one value per
          // lane -- lane (c, 0) ends with delta = -c, lane (c, 1) with
          // delta = 32 - c -- so one LDS atomic per lane and step is left.
          // Round 1 (per group g): lane c adds register 4g+e of lane c+e, all
          // of delta 8g + 4hh - c (lo); past the wrap the key is c + e - 32
          // and delta 32 higher (hi).  Round 2: lane c adds group g's lo and
          // hi of lane c + 8g (delta 4hh - c, or 32 higher past the wrap).
          // Round 3 (after the groups) merges the two lane halves.
          float lo2 = 0.0f, hi2 = 0.0f;
          auto bperm = [](int src_lane, float v) __attribute__((always_inline)) {
            return __builtin_bit_cast(
                float, __builtin_amdgcn_ds_bpermute(4 * src_lane, __builtin_bit_cast(int, v)));
          };
          auto pgroup = [&](int g, const float* dg) __attribute__((always_inline)) {
            float A = dg[0], Bw = 0.0f;
#pragma unroll
            for (int e = 1; e < 4; ++e) {
              const float v = bperm(((ol32 + e) & 31) + 32 * ohh, dg[e]);
              if (ol32 + e >= 32) Bw += v; else A += v;
            }
            if (g == 0) {
              lo2 += A;
              hi2 += Bw;
            } else {
              const int src = ((ol32 + 8 * g) & 31) + 32 * ohh;
              const float a2 = bperm(src, A), b2 = bperm(src, Bw);
              if (ol32 + 8 * g >= 32) {
                hi2 += a2;
              } else {
                lo2 += a2;
                hi2 += b2;
              }
            }
          };
          auto elem = [&](auto mc) __attribute__((always_inline)) {
            constexpr int MODE = decltype(mc)::value;
            float run = 0.0f, run_hi = 0.0f;   // run_hi: bin cbin + 1 (mode 3)
            int prev = cbin;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              uint4 t4 = {};
              if constexpr (MODE == 1 || MODE == 3)
                t4 = *reinterpret_cast<const uint4*>(&sb.ts32[8 * gq + 4 * hh]);
              float dg[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * gq + e, kk = 8 * gq + e;
                int bin = 0;
                const float t =
                    MODE == 0 ? tb : pp.template pair_time<MODE>(sb, t4, r, hh, tj64, bin, cbin, tb);
                const float x = fmaf(s[r], am, t);
                const float sg = sigm(x);
                float aa = x * sg, d = DK ? da[r] * (sg * fmaf(x, 1.0f - sg, 1.0f)) : 0.0f;
                if (!full) {
                  const bool ok = (uint32_t)(il + kk) <= (uint32_t)cb.span || is + kk == 0;
                  aa = ok ? aa : 0.0f;
                  d = ok ? d : 0.0f;
                }
                if constexpr (DV) pa[gq >> 1][4 * (gq & 1) + e] = (__bf16)aa;
                if constexpr (DK) pd[gq >> 1][4 * (gq & 1) + e] = (__bf16)d;
                dg[e] = d;
                if constexpr (clamp && TABS) {
                  if (step_cand && ib + acc_row(r, hh) >= geo.n_h) {   // clamped index
                    cacc += d;
                    dg[e] = 0.0f;
                  }
                }
                if constexpr (TIME && TABS && MODE == 3) {
                  // two bins only: one sum each, no run breaks
                  const bool up = bin != cbin;
                  run_hi += up ? d : 0.0f;
                  run += up ? 0.0f : d;
                } else if constexpr (TIME && TABS) {
                  if constexpr (MODE != 0) {
                    if (r == 0) {
                      prev = bin;
                    } else if (bin != prev) {
                      tflush(prev, run);
                      run = 0.0f;
                      prev = bin;
                    }
                  }
                  run += d;
                }
              }
              if constexpr (POS && TABS) pgroup(gq, dg);
            }
            if constexpr (TIME && TABS) tflush(prev, run);
            if constexpr (TIME && TABS && MODE == 3) tflush(cbin + 1, run_hi);
          };
          if (mode == 0) elem(std::integral_constant<int, 0>{});
          else if (mode == 3) elem(std::integral_constant<int, 3>{});
          else if (mode == 1) elem(std::integral_constant<int, 1>{});
          else elem(std::integral_constant<int, 2>{});
          if constexpr (POS && TABS) {
            // round 3: lane (c, 0) adds lane (c + 4, 1)'s lo (delta -c);
            // lane (c, 1) takes lane (c, 0)'s hi and, from lane (c + 4, 1),
            // its hi -- or past the wrap (c >= 28) the lo of lane c - 28
            const int s4 = ((ol32 + 4) & 31) + 32;
            const float x = bperm(s4, lo2);
            const float y = bperm(ol32, hi2);
            const float z = bperm(s4, ol32 < 4 ? lo2 : hi2);
            const float pacc = ohh ? y + z : lo2 + (ol32 < 28 ? x : 0.0f);
            const int rel = R0 + (ohh ? 32 - ol32 : -ol32);
            if (pacc != 0.0f)
              __hip_atomic_fetch_add(&hpos[min(rel < 0 ? -rel : rel, P - 1)], pacc,
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // dV^T += dO^T A and dK^T += Q^T dS, one d-block of operands at a time
#pragma unroll
        for (int db = 0; db < NDBM; ++db) {
          const bool dvb = DV && db < NDBY, dkb = DK && db < NDBX;   // compile-time after unrolling
          bf16x8 t4[4];
#pragma unroll
          for (int ins = 0; ins < 2; ++ins) {
            if (dvb) t4[ins] = PP::template tr_op<CY>(yt, ol, db, ins);
            if (dkb) t4[2 + ins] = PP::template tr_op<CX>(xt, ol, db, ins);
          }
#pragma unroll
          for (int ins = 0; ins < 2; ++ins) {
            if constexpr (DV) {
              if (dvb)
                accv[db < NDBY ? db : 0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    t4[ins], pa[ins], accv[db < NDBY ? db : 0], 0, 0, 0);
            }
            if constexpr (DK) {
              if (dkb)
                acck[db < NDBX ? db : 0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    t4[2 + ins], pd[ins], acck[db < NDBX ? db : 0], 0, 0, 0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (stp + 1 <= st_hi) stage_barrier();
      b = b1;
    }

    if constexpr (clamp && TABS) {
      if (key_valid && cacc != 0.0f)
        __hip_atomic_fetch_add(&hpos[c_ix], cacc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (key_valid) {
      char* dk =
          reinterpret_cast<char*>(a.dk) + ((int64_t)(seq0 + j) * a.ld_k + (int64_t)h * DQK) * 2;
      char* dv =
          reinterpret_cast<char*>(a.dv) + ((int64_t)(seq0 + j) * a.ld_v + (int64_t)h * DVV) * 2;
      if constexpr (DK) {
#pragma unroll
        for (int db = 0; db < NDBX; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            bf16x4 ok4;
#pragma unroll
            for (int e = 0; e < 4; ++e) ok4[e] = (__bf16)(acck[db][4 * g + e] * k_scale);
            *reinterpret_cast<bf16x4*>(dk + 2 * (32 * db + 8 * g + 4 * hh)) = ok4;
          }
      }
      if constexpr (DV) {
#pragma unroll
        for (int db = 0; db < NDBY; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            bf16x4 ov4;
#pragma unroll
            for (int e = 0; e < 4; ++e) ov4[e] = (__bf16)(accv[db][4 * g + e] * v_scale);
            *reinterpret_cast<bf16x4*>(dv + 2 * (32 * db + 8 * g + 4 * hh)) = ov4;
          }
      }
    }
    stage_barrier();
  }

  // this workgroup's table sums
  __syncthreads();
  if constexpr (TABS && (POS || TIME)) {
    float* part = a.tab_part + (size_t)blockIdx.x * (size_t)(P + kTabExtra);
    if constexpr (POS)
      for (int e = tid; e < P; e += kThreads) part[e] = hpos[e];
    if constexpr (TIME) {
      if (tid < kTimeBins) {
        float t = 0.0f;
        for (int l = 0; l < 32; ++l) t += htime[tid * 32 + l];
        part[P + tid] = t;
      }
    }
  }
}

// Table gradients: entry e = scale * sum over the workgroups' rows, in a
// fixed order.  Stage 1: workgroup (x, y) sums rows [64y, 64y + 64) of
// entries [64x, 64x + 64) (4 row slices of 16, combined in order); stage 2
// sums the row blocks and folds time bins past Tt - 1 into the last entry.
__global__ __launch_bounds__(256) void hstu_tab_reduce1_kernel(TabReduceArgs a) {
  __shared__ float red[4][64];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + tx;
  const int r0 = blockIdx.y * 64 + ty * 16;
  float t = 0.0f;
  if (e < a.stride) {
#pragma unroll 4
    for (int r = r0; r < min(r0 + 16, a.n_part); ++r) t += a.part[(size_t)r * a.stride + e];
  }
  red[ty][tx] = t;
  __syncthreads();
  if (ty == 0 && e < a.stride)
    a.part2[(size_t)blockIdx.y * a.stride + e] = ((red[0][tx] + red[1][tx]) + red[2][tx]) + red[3][tx];
}

__global__ __launch_bounds__(256) void hstu_tab_reduce2_kernel(TabReduceArgs a) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int nb = (a.n_part + 63) / 64;
  auto col = [&](int c) {
    float t = 0.0f;
    for (int b = 0; b < nb; ++b) t += a.part2[(size_t)b * a.stride + c];
    return t;
  };
  if (e < a.pos_len) {
    a.dpos[e] = col(e) * a.scale;
  } else if (e < a.pos_len + a.time_len) {
    const int tb = e - a.pos_len;
    float t = col(a.pos_len + tb);
    if (tb == a.time_len - 1)
      for (int bb = tb + 1; bb < kTimeBins; ++bb) t += col(a.pos_len + bb);
    a.dtime[tb] = t * a.scale;
  }
}

__global__ __launch_bounds__(256) void hstu_tab64_finish_kernel(const double* t, float* dpos,
                                                                float* dtime, int P, int Tt) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e < P) dpos[e] = (float)t[e];
  else if (e < P + Tt) dtime[e - P] = (float)t[e];
}

__global__ __launch_bounds__(256) void hstu_fill_zero_kernel(float* p, int64_t n) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n) p[e] = 0.0f;
}

// ---------------------------------------------------------------------------
// Per-token passes: one wave per (token, head), lanes over the head dimension,
// fp32 arithmetic on inputs of element type T (fp32, or bf16 for the head
// size the matrix-core passes are not built for).
// ---------------------------------------------------------------------------
template <typename T>
__device__ inline float elt(const void* p, int64_t ix) {
  return (float)static_cast<const T*>(p)[ix];
}
__device__ inline int seq_of(const int32_t* offsets, int num_seqs, int t) {
  int lo = 0, hi = num_seqs - 1;   // last b with offsets[b] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Position of token x for the position bias: x, or with the bias at clamped
// positions min(x, n_h).
__device__ inline int bias_pos(const BwdArgs& a, const SeqGeom& g, int x) {
  return a.pos_clamp && x > g.n_h ? g.n_h : x;
}

// Score of (i, j) of one head: alpha <qi, kj> + biases (lanes hold e = lane + 64 m);
// i and j are the bias positions of the pair.
template <int E>
__device__ inline float f32_score(const BwdArgs& a, const float* qi, const float* kj, int i, int j,
                                  int64_t ti, int64_t tj, int& pidx, int& tidx) {
  float d = 0.0f;
#pragma unroll
  for (int m = 0; m < E; ++m) d += qi[m] * kj[m];
  float s = a.alpha * wave_sum_f(d);
  if (a.pos_len > 0) {
    const int r = i >= j ? i - j : j - i;
    pidx = min(r, a.pos_len - 1);
    s += a.pos_table[pidx];
  }
  if (a.time_len > 0) {
    const uint64_t dt = ti >= tj ? uint64_t(ti) - uint64_t(tj) : uint64_t(tj) - uint64_t(ti);
    const uint64_t d1 = dt + 1u;
    tidx = min(d1 ? 63 - __builtin_clzll(d1) : 63, a.time_len - 1);
    s += a.time_table[tidx];
  }
  return s;
}

template <int D, typename T>
__global__ __launch_bounds__(256) void hstu_bwd_dq_f32_kernel(BwdArgs a, int num_seqs) {
  constexpr int E = (D + 63) / 64;
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (int64_t)a.n_tok * a.num_heads) return;
  const int tok = (int)(w / a.num_heads), h = (int)(w - (int64_t)tok * a.num_heads);
  const int b = seq_of(a.offsets, num_seqs, tok);
  const int seq0 = a.offsets[b], L = a.offsets[b + 1] - seq0, i = tok - seq0;
  const SeqGeom geo = seq_geom(L, a.num_targets ? a.num_targets[b] : 0, a.contextual_len,
                               a.max_attn_len);
  const RowBounds rb = row_bounds(geo, i);
  float qi[E], doi[E], acc[E];
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const int e = lane + 64 * m;
    qi[m] = e < D ? elt<T>(a.q, (int64_t)tok * a.ld_q + h * D + e) : 0.0f;
    doi[m] = e < D ? elt<T>(a.dout, (int64_t)tok * a.ld_do + h * D + e) : 0.0f;
    acc[m] = 0.0f;
  }
  const int64_t ti = a.time_len > 0 ? a.timestamps[tok] : 0;
  const int n_range = rb.lo != kEmptyLo ? rb.span + 1 : 0;
  for (int n = 0; n < n_range + (rb.self_j >= 0 ? 1 : 0); ++n) {
    const int j = n < n_range ? rb.lo + n : rb.self_j;
    float kj[E], vj[E];
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const int e = lane + 64 * m;
      kj[m] = e < D ? elt<T>(a.k, (int64_t)(seq0 + j) * a.ld_k + h * D + e) : 0.0f;
      vj[m] = e < D ? elt<T>(a.v, (int64_t)(seq0 + j) * a.ld_v + h * D + e) : 0.0f;
    }
    int pidx = 0, tidx = 0;
    const int64_t tj = a.time_len > 0 ? a.timestamps[seq0 + j] : 0;
    const float s = f32_score<E>(a, qi, kj, bias_pos(a, geo, i), bias_pos(a, geo, j), ti, tj, pidx, tidx);
    float dd = 0.0f;
#pragma unroll
    for (int m = 0; m < E; ++m) dd += doi[m] * vj[m];
    const float da = wave_sum_f(dd);
    const float sg = 1.0f / (1.0f + expf(-s));
    const float ds = da * sg * (1.0f + s * (1.0f - sg)) * a.inv_scale;
#pragma unroll
    for (int m = 0; m < E; ++m) acc[m] += a.alpha * ds * kj[m];
    if (lane == 0) {
      // fp64 sums: their rounding does not depend on the order of arrival
      if (a.pos_len > 0) atomicAdd(&a.tab64[pidx], (double)ds);
      if (a.time_len > 0) atomicAdd(&a.tab64[a.pos_len + tidx], (double)ds);
    }
  }
  T* dq = static_cast<T*>(a.dq);
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const int e = lane + 64 * m;
    if (e < D) dq[(int64_t)tok * a.ld_q + h * D + e] = (T)acc[m];
  }
}

template <int D, typename T>
__global__ __launch_bounds__(256) void hstu_bwd_dkv_f32_kernel(BwdArgs a, int num_seqs) {
  constexpr int E = (D + 63) / 64;
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (int64_t)a.n_tok * a.num_heads) return;
  const int tok = (int)(w / a.num_heads), h = (int)(w - (int64_t)tok * a.num_heads);
  const int b = seq_of(a.offsets, num_seqs, tok);
  const int seq0 = a.offsets[b], L = a.offsets[b + 1] - seq0, j = tok - seq0;
  const SeqGeom geo = seq_geom(L, a.num_targets ? a.num_targets[b] : 0, a.contextual_len,
                               a.max_attn_len);
  const RowBounds cb = col_bounds(geo, j);
  float kj[E], vj[E], ak[E], av[E];
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const int e = lane + 64 * m;
    kj[m] = e < D ? elt<T>(a.k, (int64_t)tok * a.ld_k + h * D + e) : 0.0f;
    vj[m] = e < D ? elt<T>(a.v, (int64_t)tok * a.ld_v + h * D + e) : 0.0f;
    ak[m] = 0.0f;
    av[m] = 0.0f;
  }
  const int64_t tj = a.time_len > 0 ? a.timestamps[tok] : 0;
  const int n_range = cb.lo != kEmptyLo ? cb.span + 1 : 0;
  for (int n = 0; n < n_range + (cb.self_j >= 0 ? 1 : 0); ++n) {
    const int i = n < n_range ? cb.lo + n : cb.self_j;
    float qi[E], doi[E];
#pragma unroll
    for (int m = 0; m < E; ++m) {
      const int e = lane + 64 * m;
      qi[m] = e < D ? elt<T>(a.q, (int64_t)(seq0 + i) * a.ld_q + h * D + e) : 0.0f;
      doi[m] = e < D ? elt<T>(a.dout, (int64_t)(seq0 + i) * a.ld_do + h * D + e) : 0.0f;
    }
    int pidx = 0, tidx = 0;
    const int64_t ti = a.time_len > 0 ? a.timestamps[seq0 + i] : 0;
    const float s = f32_score<E>(a, qi, kj, bias_pos(a, geo, i), bias_pos(a, geo, j), ti, tj, pidx, tidx);
    float dd = 0.0f;
#pragma unroll
    for (int m = 0; m < E; ++m) dd += doi[m] * vj[m];
    const float da = wave_sum_f(dd);
    const float sg = 1.0f / (1.0f + expf(-s));
    const float coef = s * sg * a.inv_scale;
    const float ds = da * sg * (1.0f + s * (1.0f - sg)) * a.inv_scale;
#pragma unroll
    for (int m = 0; m < E; ++m) {
      av[m] += coef * doi[m];
      ak[m] += a.alpha * ds * qi[m];
    }
  }
  T* dk = static_cast<T*>(a.dk);
  T* dv = static_cast<T*>(a.dv);
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const int e = lane + 64 * m;
    if (e < D) {
      dk[(int64_t)tok * a.ld_k + h * D + e] = (T)ak[m];
      dv[(int64_t)tok * a.ld_v + h * D + e] = (T)av[m];
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// Which backward kernel: 0 = dQ, 1 = the pass that sums the tables (dK, or
// dK and dV fused), 2 = the dV-only pass (d = 128).
// The dK/dV pass: fused (0) when both head sizes are 64; with a 128-wide
// side the two accumulators need more registers than two waves per SIMD
// leave, so dK (with the table sums, 1) and dV (2) run as two passes.
template <int DQK, int DV>
constexpr int kv_mode_tab() { return (DQK == 128 || DV == 128) ? 1 : 0; }

template <bool POS>
size_t dkv_dyn_lds(int which, int pos_len) {
  return (POS && which == 1) ? sizeof(float) * (size_t)pos_len : 0;
}

template <int DQK, int DV, bool POS, bool TIME, bool CL>
int bpc_one(int which, int pos_len) {
  int nb = 0;
  hipError_t e;
  const size_t dyn = dkv_dyn_lds<POS>(which, pos_len);
  if (which == 1)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, hstu_bwd_dkv_kernel<DQK, DV, POS, TIME, kv_mode_tab<DQK, DV>(), CL>, kThreads, dyn);
  else if (which == 2)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, hstu_bwd_dkv_kernel<DQK, DV, POS, TIME, 2, CL>, kThreads, 0);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, hstu_bwd_dq_kernel<DQK, DV, POS, TIME, CL>, kThreads, 0);
  return e == hipSuccess ? nb : -1;
}

template <int DQK, int DV>
int bpc_d(int which, int pos_len, int time_len, bool clamp) {
  const bool pos = pos_len > 0, tim = time_len > 0, cl = pos && clamp;
  if (cl && tim) return bpc_one<DQK, DV, true, true, true>(which, pos_len);
  if (cl) return bpc_one<DQK, DV, true, false, true>(which, pos_len);
  if (pos && tim) return bpc_one<DQK, DV, true, true, false>(which, pos_len);
  if (pos) return bpc_one<DQK, DV, true, false, false>(which, pos_len);
  if (tim) return bpc_one<DQK, DV, false, true, false>(which, pos_len);
  return bpc_one<DQK, DV, false, false, false>(which, pos_len);
}

template <int DQK, int DV, bool POS, bool TIME, bool CL>
hipError_t launch_mfma_one(const BwdArgs& a, int which, int n_wg, hipStream_t stream) {
  const size_t dyn = dkv_dyn_lds<POS>(which, a.pos_len);
  if (which == 1)
    hipLaunchKernelGGL((hstu_bwd_dkv_kernel<DQK, DV, POS, TIME, kv_mode_tab<DQK, DV>(), CL>),
                       dim3((unsigned)n_wg), dim3(kThreads), dyn, stream, a);
  else if (which == 2)
    hipLaunchKernelGGL((hstu_bwd_dkv_kernel<DQK, DV, POS, TIME, 2, CL>), dim3((unsigned)n_wg),
                       dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((hstu_bwd_dq_kernel<DQK, DV, POS, TIME, CL>), dim3((unsigned)n_wg),
                       dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t launch_mfma_d(const BwdArgs& a, int which, int n_wg, hipStream_t stream) {
  if (which == 2 && kv_mode_tab<DQK, DV>() == 0) return hipSuccess;   // fused in pass 1
  const bool pos = a.pos_len > 0, tim = a.time_len > 0, cl = pos && a.pos_clamp != 0;
  if (cl && tim) return launch_mfma_one<DQK, DV, true, true, true>(a, which, n_wg, stream);
  if (cl) return launch_mfma_one<DQK, DV, true, false, true>(a, which, n_wg, stream);
  if (pos && tim) return launch_mfma_one<DQK, DV, true, true, false>(a, which, n_wg, stream);
  if (pos) return launch_mfma_one<DQK, DV, true, false, false>(a, which, n_wg, stream);
  if (tim) return launch_mfma_one<DQK, DV, false, true, false>(a, which, n_wg, stream);
  return launch_mfma_one<DQK, DV, false, false, false>(a, which, n_wg, stream);
}

template <int D, typename T>
hipError_t launch_f32_d(const BwdArgs& a, bool kv, int num_seqs, hipStream_t stream) {
  const int64_t waves = (int64_t)a.n_tok * a.num_heads;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  if (kv)
    hipLaunchKernelGGL((hstu_bwd_dkv_f32_kernel<D, T>), grid, block, 0, stream, a, num_seqs);
  else
    hipLaunchKernelGGL((hstu_bwd_dq_f32_kernel<D, T>), grid, block, 0, stream, a, num_seqs);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_plan(const BwdPlanArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(hstu_bwd_plan_kernel, dim3(1), dim3(kPlanT), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int EPC, int G, int CPL>
static hipError_t launch_gate_one(const GateBwdArgs& a, hipStream_t stream) {
  const int64_t groups = (int64_t)a.n_tok * a.groups;
  const int64_t waves = (groups + 64 / G - 1) / (64 / G);
  hipLaunchKernelGGL((hstu_gate_bwd_kernel<T, EPC, G, CPL>), dim3((unsigned)((waves + 3) / 4)),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int EPC>
static hipError_t launch_gate_t(const GateBwdArgs& a, hipStream_t stream) {
  const int chunks = a.width / EPC;
  if (chunks <= 2) return launch_gate_one<T, EPC, 2, 1>(a, stream);
  if (chunks <= 4) return launch_gate_one<T, EPC, 4, 1>(a, stream);
  if (chunks <= 8) return launch_gate_one<T, EPC, 8, 1>(a, stream);
  if (chunks <= 16) return launch_gate_one<T, EPC, 16, 1>(a, stream);
  if (chunks <= 32) return launch_gate_one<T, EPC, 32, 1>(a, stream);
  if (chunks <= 64) return launch_gate_one<T, EPC, 64, 1>(a, stream);
  if (chunks <= 128) return launch_gate_one<T, EPC, 64, 2>(a, stream);
  if (chunks <= 256) return launch_gate_one<T, EPC, 64, 4>(a, stream);
  if (chunks <= 512) return launch_gate_one<T, EPC, 64, 8>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_gate_bwd(const GateBwdArgs& a, int dtype, hipStream_t stream) {
  if ((int64_t)a.n_tok * a.groups <= 0) return hipSuccess;
  return dtype == 1 ? launch_gate_t<__bf16, 8>(a, stream) : launch_gate_t<float, 4>(a, stream);
}

int bwd_grid(int dtype, int d_qk, int d_v, int pos_len, int time_len, int which,
             bool clamp) {
  if (dtype != 1) return 1;   // fp32 kernels are not persistent
  int bpc = -1;
  if (d_qk == 128 && d_v == 128) {
    bpc = bpc_d<128, 128>(which, pos_len, time_len, clamp);
  } else if (d_qk == 64 && d_v == 64) {
    if (which == 2) return 0;   // no separate dV pass
    bpc = bpc_d<64, 64>(which, pos_len, time_len, clamp);
  } else if (d_qk == 64 && d_v == 128) {
    bpc = bpc_d<64, 128>(which, pos_len, time_len, clamp);
  } else if (d_qk == 128 && d_v == 64) {
    bpc = bpc_d<128, 64>(which, pos_len, time_len, clamp);
  }
  if (bpc <= 0) return -1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  const int g = cus * bpc;
  return g < kMaxGrid ? g : kMaxGrid;
}

// Head sizes the backward is built for: bf16 MFMA passes for d_qk, d_v in
// {64, 128} (equal or not); the per-token kernels for fp32 with d_qk == d_v
// in {8, 64, 128} and for bf16 with d_qk = d_v = 256.
bool bwd_supported(int dtype, int d_qk, int d_v) {
  if (dtype == 1)
    return ((d_qk == 64 || d_qk == 128) && (d_v == 64 || d_v == 128)) ||
           (d_qk == 256 && d_v == 256);
  if (dtype == 0) return d_qk == d_v && (d_qk == 8 || d_qk == 64 || d_qk == 128);
  return false;
}

bool bwd_per_token(int dtype, int d_qk, int d_v) {
  return dtype != 1 || (d_qk == 256 && d_v == 256);
}

hipError_t launch_bwd(const BwdArgs& a, int dtype, int d_qk, int d_v, int which, int n_wg,
                      hipStream_t stream) {
  if (dtype == 1 && d_qk == 256 && d_v == 256) {   // per-token kernels, n_wg = sequences
    if (which == 2) return hipSuccess;
    return launch_f32_d<256, __bf16>(a, which == 1, n_wg, stream);
  }
  if (dtype == 1) {
    if (d_qk == 128 && d_v == 128) return launch_mfma_d<128, 128>(a, which, n_wg, stream);
    if (d_qk == 64 && d_v == 64) return launch_mfma_d<64, 64>(a, which, n_wg, stream);
    if (d_qk == 64 && d_v == 128) return launch_mfma_d<64, 128>(a, which, n_wg, stream);
    if (d_qk == 128 && d_v == 64) return launch_mfma_d<128, 64>(a, which, n_wg, stream);
    return hipErrorInvalidValue;
  }
  // fp32: one kernel per side; n_wg carries the number of sequences
  if (which == 2) return hipSuccess;
  if (d_qk != d_v) return hipErrorInvalidValue;
  const bool kv = which == 1;
  if (d_qk == 128) return launch_f32_d<128, float>(a, kv, n_wg, stream);
  if (d_qk == 64) return launch_f32_d<64, float>(a, kv, n_wg, stream);
  if (d_qk == 8) return launch_f32_d<8, float>(a, kv, n_wg, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_tab_reduce(const TabReduceArgs& a, hipStream_t stream) {
  const int n = a.pos_len + a.time_len;
  if (n <= 0 || a.n_part <= 0) return hipSuccess;
  hipLaunchKernelGGL(hstu_tab_reduce1_kernel,
                     dim3((unsigned)((a.stride + 63) / 64), (unsigned)((a.n_part + 63) / 64)),
                     dim3(256), 0, stream, a);
  hipLaunchKernelGGL(hstu_tab_reduce2_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_tab64_finish(const double* tab64, float* dpos, float* dtime, int pos_len,
                               int time_len, hipStream_t stream) {
  const int n = pos_len + time_len;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(hstu_tab64_finish_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     stream, tab64, dpos, dtime, pos_len, time_len);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(hstu_fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     stream, p, n);
  return hipGetLastError();
}

}  // namespace hstu
