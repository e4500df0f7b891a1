// attn_common.hpp -- device helpers shared by the gfx950 attention forward
// kernels: operand vector types, HBM -> LDS copies (global_load_lds), explicit
// memory-counter waits, the pipeline barrier, wave reductions, the staged-row
// swizzles and the SiLU in log2 units.
#pragma once

#include <type_traits>

#include "hstu_device.hpp"

namespace hstu {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int uintx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaskedX = -1.0e30f;   // SiLU argument of an illegal pair
constexpr int64_t kT32Range = int64_t(1) << 30;  // |t - base| below this: 32-bit path
constexpr int kDiag = kBM + kBN - 1;             // distinct i - j of a 128 x 32 block
constexpr int kDiagCopies = (kDiag + 63) / 64;   // 4-byte LDS copies of 64 lanes

// XOR swizzle of the 16-byte chunks of a staged row of CH chunks: the rows a
// wave touches at one chunk position fall on distinct LDS banks.
template <int CH>
__device__ inline int row_swz(int row) {
  return CH >= 16 ? (row & 15) : (CH >= 2 ? ((row >> 1) & (CH - 1)) : 0);
}

template <typename T, int DQK, int DV>
struct Cfg {
  static constexpr bool kBf16 = std::is_same<T, __bf16>::value;
  static constexpr int kEs = (int)sizeof(T);
  static constexpr int kStep = kBf16 ? 16 : 2;          // MFMA contraction depth
  static constexpr int kKRow = DQK * kEs;               // staged row bytes
  static constexpr int kVRow = DV * kEs;
  static constexpr int kKCh = kKRow / 16;               // 16-byte chunks per row
  static constexpr int kVCh = kVRow / 16;
  static constexpr int kNK = kBN * kKCh / 64;           // 64-lane copies per K stage
  static constexpr int kNV = kBN * kVCh / 64;
  static constexpr int kNKC = DQK / kStep;              // MFMA steps of the scores
  static constexpr int kNDB = (DV + 31) / 32;           // 32-wide d_v blocks of O^T
  static_assert(kKRow % 16 == 0 && kVRow % 16 == 0, "rows are whole 16-byte chunks");
  static_assert(kBN * kKCh % 64 == 0 && kBN * kVCh % 64 == 0, "stage is whole copies");
  static_assert(DQK % kStep == 0 && DV % 4 == 0 && (!kBf16 || DV % 32 == 0), "shape");
  // The Q tile and the epilogue stage 32 rows per wave in half of the K+V
  // space of a stage buffer, which holds 64 rows of d_qk when d_qk <= d_v and
  // 64 rows of d_v when d_v <= d_qk; otherwise that side goes directly
  // between HBM and registers (Q operands loaded per lane; U loaded and the
  // output stored 4 values per lane).
  static constexpr bool kQLds = kKRow <= kVRow;
  static constexpr bool kEpLds = kVRow <= kKRow;
  // XOR swizzles of a row's 16-byte chunks (always below the number of
  // chunks, so they permute the row).  K: one read touches the same logical
  // chunk of 16 consecutive rows per LDS cycle.  V (bf16): a transposed read
  // of one lane half touches 4 rows x 4 chunks; (fp32): two rows 4 apart.
  __device__ static int kswz(int row) {
    return kKCh >= 16 ? (row & 15) : (kKCh >= 2 ? ((row >> 1) & (kKCh - 1)) : 0);
  }
  __device__ static int vswz(int row) {
    if constexpr (kBf16) return kVCh >= 16 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
    return kVCh >= 16 ? 8 * ((row >> 2) & 1) : 0;
  }
};

struct TimeTables {
  float trev[32];   // trev[z] = log2e * time[min(31 - z, Tt - 1)], z = clz(1 + |dt|)
  float tful[64];   // tful[b] = log2e * time[min(b, Tt - 1)]
};

// LDS byte offset of a __shared__ object's (generic) address: the LDS
// aperture is 4 GiB aligned, so the offset is the address's low 32 bits.
__device__ inline uint32_t lds_off(const void* p) { return (uint32_t)(uintptr_t)p; }
// LDS pointer from an LDS byte offset.
__device__ inline lds_shortx4* lds_ptr4(uint32_t off) { return (lds_shortx4*)(uintptr_t)off; }
// Typed LDS access by byte offset.
template <typename V>
__device__ inline V lds_ld(uint32_t off) {
  return *(__attribute__((address_space(3))) const V*)(uintptr_t)off;
}
template <typename V>
__device__ inline void lds_st(uint32_t off, V v) {
  *(__attribute__((address_space(3))) V*)(uintptr_t)off = v;
}

// A pointer that is the same in every lane, as a scalar-register value.
__device__ inline uint64_t uni_ptr(const void* p) {
  const uint64_t x = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// HBM -> LDS copies (global_load_lds): lane l reads base + voff and its bytes
// land at LDS offset `lds` + size * l.  Issued from inline assembly on
// purpose: the compiler then neither waits for them before unrelated LDS
// reads nor folds them into its own vmcnt accounting; every wait on them is
// an explicit wait_vmem below.  They write no registers.  M0 is a reserved
// register, so clobbering it is harmless; the warning about it is silenced.
// `base` and `lds` must be the same in every lane.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void lds_copy16(uint64_t base, uint32_t voff, uint32_t lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(m), "v"(voff), "s"(base) : "memory", "m0");
}
// The same, non-temporal (`nt`): for data that nothing reads again soon (a
// query tile, U rows, the keys and values of a short sequence), so that it
// does not push reused key/value tiles out of the caches.
__device__ inline void lds_copy16_nt(uint64_t base, uint32_t voff, uint32_t lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :: "s"(m), "v"(voff), "s"(base) : "memory", "m0");
}
__device__ inline void lds_copy4(uint64_t base, uint32_t voff, uint32_t lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(m), "v"(voff), "s"(base) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N): all but the N most recent global memory operations
// (loads, stores, LDS copies) of this wave are done (they complete in order).
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// The same for a wave-uniform count below 8.
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

// Workgroup barrier for the pipeline.  __syncthreads() carries a release
// fence that waits for every outstanding LDS copy, which would drain the
// copies of the stages ahead; here the caller has already waited for the
// copies that must have landed (vmcnt) and this waits for its own LDS
// accesses (lgkmcnt), and the empty asm statements keep the compiler from
// moving memory accesses across the barrier.
__device__ inline void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt untouched
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ inline int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Minimum / maximum over the 64 lanes of a wave (all lanes active), returned
// in a scalar register.  Data-parallel-primitive (DPP) row shifts build a
// running reduction within each 16-lane row (lane 15 ends with the row's
// value), then row broadcasts carry rows 0..2 into lane 63: a handful of
// register-to-register moves instead of LDS round trips.
template <bool MAX, typename V>
__device__ inline V wave_reduce(V x) {
  static_assert(sizeof(V) == 4, "32-bit values");
  auto op = [](V a, V b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  auto dpp = [](V v, auto ctrl, auto rows) {
    return __builtin_bit_cast(
        V, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                       decltype(ctrl)::value, decltype(rows)::value, 0xf,
                                       false));
  };
  x = op(x, dpp(x, std::integral_constant<int, 0x111>{}, std::integral_constant<int, 0xf>{}));
  x = op(x, dpp(x, std::integral_constant<int, 0x112>{}, std::integral_constant<int, 0xf>{}));
  x = op(x, dpp(x, std::integral_constant<int, 0x114>{}, std::integral_constant<int, 0xf>{}));
  x = op(x, dpp(x, std::integral_constant<int, 0x118>{}, std::integral_constant<int, 0xf>{}));
  x = op(x, dpp(x, std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xa>{}));
  x = op(x, dpp(x, std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xc>{}));
  return __builtin_bit_cast(V, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
template <typename V>
__device__ inline V wave_min(V v) { return wave_reduce<false>(v); }
template <typename V>
__device__ inline V wave_max(V v) { return wave_reduce<true>(v); }

// Register r of a 32x32 accumulator (lane half hh) holds row 8(r/4) + 4hh + r%4.
__device__ constexpr int acc_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

// SiLU(x) * log2(e) = x2 / (1 + 2^-x2)
__device__ inline float silu2(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x));
}

}  // namespace hstu
