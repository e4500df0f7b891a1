// Host-side memory-safety checks, built with AddressSanitizer (host code
// only; the HIP library's sources are compiled host-only, so no device code
// exists and nothing is launched):
//   * every C-ABI entry point on arguments the host rejects before any HIP
//     call (null, misaligned and out-of-range pointers, strides, sizes,
//     tables, workspace sizes, unsupported shapes), with the error message
//     read back each time;
//   * the fp64 C oracle's forward and backward on small ragged batches with
//     every mask rule, both bias tables and both position-bias readings.
// Prints "ok: N checks" and exits 0, or names the first failed check and
// exits 1.  The sanitizer aborts on any invalid access or leak.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "hstu_attn.h"

extern "C" {
int hstu_oracle_fwd(int num_seqs, const int32_t* offsets, int num_heads, int d_qk, int d_v,
                    const double* q, int64_t ld_q, const double* k, int64_t ld_k,
                    const double* v, int64_t ld_v, const double* u, int64_t ld_u,
                    const int64_t* timestamps, const int32_t* num_targets,
                    int contextual_len, int max_attn_len, double alpha, double n_scale,
                    const double* pos_table, int pos_len, const double* time_table,
                    int time_len, double eps, int epilogue, double* out, int64_t ld_out,
                    const unsigned char* row_select, int nthreads, int pos_clamp);
int hstu_oracle_bwd(int num_seqs, const int32_t* offsets, int num_heads, int d_qk, int d_v,
                    const double* q, int64_t ld_q, const double* k, int64_t ld_k,
                    const double* v, int64_t ld_v, const double* u, int64_t ld_u,
                    const int64_t* timestamps, const int32_t* num_targets,
                    int contextual_len, int max_attn_len, double alpha, double n_scale,
                    const double* pos_table, int pos_len, const double* time_table,
                    int time_len, double eps, int epilogue, const double* dout,
                    int64_t ld_out, double* dq, double* dk, double* dv, double* du,
                    double* dpos, double* dtime, int nthreads, int pos_clamp);
}

static int g_checks = 0;
#define CHECK(cond)                                                              \
  do {                                                                           \
    ++g_checks;                                                                  \
    if (!(cond)) {                                                               \
      std::printf("FAILED %s:%d: %s (last error: %s)\n", __FILE__, __LINE__, #cond, \
                  hstu_last_error());                                            \
      std::exit(1);                                                              \
    }                                                                            \
  } while (0)

// An aligned address the host never dereferences (the library only checks
// pointers on these paths).
static void* const kFake = reinterpret_cast<void*>(uintptr_t(0x10000));
static void* at(size_t off) { return reinterpret_cast<char*>(kFake) + off; }

static hstu_attn_desc base_desc() {
  hstu_attn_desc d;
  std::memset(&d, 0, sizeof(d));
  d.num_seqs = 2; d.total_tokens = 100; d.num_heads = 4; d.d_qk = 128; d.d_v = 128;
  d.dtype = HSTU_DTYPE_BF16;
  d.ld_q = d.ld_k = d.ld_v = d.ld_u = d.ld_out = 512;
  d.ln_eps = 1e-5f; d.epilogue = HSTU_EPILOGUE_LN_U;
  return d;
}

// The message of a failed call: set, bounded and readable to its end.
static void check_message() {
  const char* m = hstu_last_error();
  CHECK(m != nullptr);
  const size_t n = std::strlen(m);
  CHECK(n > 0 && n < 4096);
}

static int fwd(const hstu_attn_desc& d, void* q, void* out, void* ws, size_t wsb,
               float n_scale = 10.f, const float* pos = nullptr, const float* tim = nullptr,
               const int64_t* ts = nullptr) {
  return hstu_jagged_attn_fwd(&d, q, kFake, kFake, kFake, static_cast<const int32_t*>(kFake),
                              ts, nullptr, 0, 0, 0.1f, n_scale, pos, tim, out, ws, wsb, nullptr);
}

static void abi_checks() {
  // supported shapes
  CHECK(hstu_jagged_attn_supported(HSTU_DTYPE_BF16, 128, 128) == 1);
  CHECK(hstu_jagged_attn_supported(HSTU_DTYPE_BF16, 256, 256) == 1);
  CHECK(hstu_jagged_attn_supported(HSTU_DTYPE_F32, 8, 8) == 1);
  CHECK(hstu_jagged_attn_supported(HSTU_DTYPE_BF16, 8, 8) == 0);
  CHECK(hstu_jagged_attn_supported(7, 128, 128) == 0);
  CHECK(hstu_jagged_attn_supported(HSTU_DTYPE_BF16, -128, 128) == 0);

  // workspace sizing: valid descs give a size, bad ones 0 with a message
  hstu_attn_desc d = base_desc();
  const size_t ws = hstu_jagged_attn_workspace_bytes(&d);
  CHECK(ws > 0);
  CHECK(hstu_jagged_attn_bwd_workspace_bytes(&d) > 0);
  CHECK(hstu_jagged_attn_workspace_bytes(nullptr) == 0);
  check_message();
  const int32_t bad_ints[] = {-1, 0, INT32_MIN};
  for (int32_t x : bad_ints) {
    hstu_attn_desc b = base_desc();
    b.num_heads = x;
    CHECK(hstu_jagged_attn_workspace_bytes(&b) == 0);
    check_message();
    b = base_desc();
    b.ld_q = x;
    CHECK(hstu_jagged_attn_workspace_bytes(&b) == 0);
    check_message();
  }
  {
    hstu_attn_desc b = base_desc();
    b.num_seqs = -3;
    CHECK(hstu_jagged_attn_workspace_bytes(&b) == 0);
    b = base_desc();
    b.total_tokens = INT32_MAX;   // huge but valid: the size must not overflow to small
    const size_t big = hstu_jagged_attn_workspace_bytes(&b);
    CHECK(big == 0 || big >= ws);
    b = base_desc();
    b.ln_eps = NAN;
    CHECK(hstu_jagged_attn_workspace_bytes(&b) == 0);
    b = base_desc();
    b.epilogue = 9;
    CHECK(hstu_jagged_attn_workspace_bytes(&b) == 0);
    b = base_desc();
    b.d_qk = 96;                  // unsupported shape
    CHECK(hstu_jagged_attn_workspace_bytes(&b) == 0);
  }

  // forward: each rejected before any HIP call
  CHECK(fwd(d, nullptr, kFake, kFake, ws) == HSTU_ERR_INVALID_ARG);
  check_message();
  CHECK(fwd(d, at(2), kFake, kFake, ws) == HSTU_ERR_INVALID_ARG);     // misaligned q
  check_message();
  CHECK(fwd(d, kFake, nullptr, kFake, ws) == HSTU_ERR_INVALID_ARG);
  CHECK(fwd(d, kFake, kFake, nullptr, ws) == HSTU_ERR_WORKSPACE);
  CHECK(fwd(d, kFake, kFake, kFake, ws - 1) == HSTU_ERR_WORKSPACE);
  check_message();
  CHECK(fwd(d, kFake, kFake, kFake, ws, 0.f) == HSTU_ERR_INVALID_ARG);
  CHECK(fwd(d, kFake, kFake, kFake, ws, NAN) == HSTU_ERR_INVALID_ARG);
  {
    hstu_attn_desc b = base_desc();
    b.pos_table_len = 16;         // length without a table
    CHECK(fwd(b, kFake, kFake, kFake, ws) == HSTU_ERR_INVALID_ARG);
    b.pos_table_len = 1 << 20;    // longer than the kernels take
    CHECK(fwd(b, kFake, kFake, kFake, 1u << 30, 10.f, static_cast<const float*>(kFake)) ==
          HSTU_ERR_UNSUPPORTED);
    check_message();
    b = base_desc();
    b.time_table_len = 64;        // time table without timestamps
    CHECK(fwd(b, kFake, kFake, kFake, 1u << 30, 10.f, nullptr,
              static_cast<const float*>(kFake)) == HSTU_ERR_INVALID_ARG);
    b = base_desc();
    b.ld_v = 100;                 // stride below H * d_v
    CHECK(fwd(b, kFake, kFake, kFake, 1u << 30) == HSTU_ERR_INVALID_ARG);
    b = base_desc();
    b.ld_out = 513;               // stride not a multiple of 16 bytes
    CHECK(fwd(b, kFake, kFake, kFake, 1u << 30) == HSTU_ERR_INVALID_ARG);
    check_message();
  }
  CHECK(hstu_jagged_attn_plan(&d, nullptr, nullptr, 0, 0, kFake, ws, nullptr) ==
        HSTU_ERR_INVALID_ARG);
  CHECK(hstu_jagged_attn_plan(&d, static_cast<const int32_t*>(kFake), nullptr, -1, 0, kFake, ws,
                              nullptr) == HSTU_ERR_INVALID_ARG);
  CHECK(hstu_jagged_attn_run(&d, kFake, kFake, kFake, kFake, static_cast<const int32_t*>(kFake),
                             nullptr, nullptr, 0, -5, 0.1f, 10.f, nullptr, nullptr, kFake, kFake,
                             ws, nullptr) == HSTU_ERR_INVALID_ARG);
  CHECK(hstu_jagged_attn_run_timed(&d, kFake, kFake, kFake, kFake,
                                   static_cast<const int32_t*>(kFake), nullptr, nullptr, 0, 0,
                                   0.1f, 10.f, nullptr, nullptr, kFake, nullptr, 0, nullptr,
                                   nullptr, nullptr) == HSTU_ERR_WORKSPACE);
  CHECK(hstu_jagged_attn_plan_candidates(&d, nullptr, nullptr, 0, 0, kFake, ws, nullptr) ==
        HSTU_ERR_INVALID_ARG);
  CHECK(hstu_jagged_attn_plan_candidates(&d, static_cast<const int32_t*>(kFake), nullptr, 0, 0,
                                         kFake, 16, nullptr) == HSTU_ERR_WORKSPACE);
  CHECK(hstu_jagged_attn_fwd_candidates(&d, kFake, kFake, at(4), kFake,
                                        static_cast<const int32_t*>(kFake), nullptr, nullptr, 0,
                                        0, 0.1f, 10.f, nullptr, nullptr, kFake, kFake, ws,
                                        nullptr) == HSTU_ERR_INVALID_ARG);   // misaligned v
  CHECK(hstu_jagged_attn_fwd_noalloc(&d, nullptr, kFake, kFake, kFake,
                                     static_cast<const int32_t*>(kFake), nullptr, nullptr, 0, 0,
                                     0.1f, 10.f, nullptr, nullptr, kFake, nullptr) ==
        HSTU_ERR_INVALID_ARG);
  CHECK(hstu_jagged_attn_fwd_train(&d, kFake, kFake, kFake, kFake,
                                   static_cast<const int32_t*>(kFake), nullptr, nullptr, 0, 0,
                                   0.1f, 10.f, nullptr, nullptr, kFake, at(8), kFake, ws,
                                   nullptr) == HSTU_ERR_INVALID_ARG);   // misaligned o_raw
  check_message();

  // kernel choice (host only)
  CHECK(hstu_jagged_attn_set_fwd_kernel(99) == HSTU_ERR_INVALID_ARG);
  CHECK(hstu_jagged_attn_set_fwd_kernel(HSTU_FWD_KERNEL_FOUR_WAVE) == HSTU_OK);
  CHECK(hstu_jagged_attn_fwd_kernel_of(&d) == HSTU_FWD_KERNEL_FOUR_WAVE);
  CHECK(hstu_jagged_attn_set_fwd_kernel(HSTU_FWD_KERNEL_AUTO) == HSTU_OK);
  CHECK(hstu_jagged_attn_fwd_kernel_of(&d) == HSTU_FWD_KERNEL_SIXTEEN_ROW);
  CHECK(hstu_jagged_attn_fwd_kernel_of(nullptr) == -1);

  // backward
  auto bwd = [&](const hstu_attn_desc& b, void* dq, void* ws_p, size_t wsb) {
    return hstu_jagged_attn_bwd(&b, kFake, kFake, kFake, kFake,
                                static_cast<const int32_t*>(kFake), nullptr, nullptr, 0, 0,
                                0.1f, 10.f, nullptr, nullptr, kFake, nullptr, dq, kFake, kFake,
                                kFake, nullptr, nullptr, ws_p, wsb, nullptr);
  };
  const size_t bws = hstu_jagged_attn_bwd_workspace_bytes(&d);
  CHECK(bwd(d, nullptr, kFake, bws) == HSTU_ERR_INVALID_ARG);
  CHECK(bwd(d, kFake, nullptr, bws) == HSTU_ERR_WORKSPACE);
  CHECK(bwd(d, kFake, kFake, bws - 1) == HSTU_ERR_WORKSPACE);
  {
    hstu_attn_desc b = base_desc();
    b.d_qk = 256;
    b.ld_q = b.ld_k = 1024;
    CHECK(bwd(b, kFake, kFake, 1u << 30) == HSTU_ERR_UNSUPPORTED);   // no such forward
    check_message();
    b = base_desc();
    b.d_qk = b.d_v = 256;   // per-token backward: its workspace is checked before any HIP call
    b.ld_q = b.ld_k = b.ld_v = b.ld_u = b.ld_out = 1024;
    const size_t bws256 = hstu_jagged_attn_bwd_workspace_bytes(&b);
    CHECK(bws256 > 0);
    CHECK(bwd(b, kFake, kFake, bws256 - 1) == HSTU_ERR_WORKSPACE);
    check_message();
    b = base_desc();
    b.pos_clamp = 2;   // a flag: 0 or 1
    CHECK(bwd(b, kFake, kFake, 1u << 30) == HSTU_ERR_INVALID_ARG);
  }

  // layer
  hstu_layer_desc ld;
  std::memset(&ld, 0, sizeof(ld));
  ld.num_seqs = 2; ld.total_tokens = 100; ld.num_heads = 4; ld.d_qk = 128; ld.d_v = 128;
  ld.hidden = 512; ld.ln_eps = 1e-5f;
  const size_t lws = hstu_layer_workspace_bytes(&ld);
  CHECK(lws > 0);
  auto layer = [&](const hstu_layer_desc& b, void* x, size_t wsb) {
    return hstu_layer_fwd(&b, x, kFake, kFake, kFake, static_cast<const int32_t*>(kFake),
                          nullptr, nullptr, 0, 0, 0.1f, 10.f, nullptr, nullptr, kFake, kFake, wsb,
                          nullptr);
  };
  CHECK(layer(ld, nullptr, lws) == HSTU_ERR_INVALID_ARG);
  CHECK(layer(ld, kFake, lws - 1) == HSTU_ERR_WORKSPACE);
  {
    hstu_layer_desc b = ld;
    b.hidden = 500;
    CHECK(hstu_layer_workspace_bytes(&b) == 0);
    check_message();
    CHECK(layer(b, kFake, 1u << 30) == HSTU_ERR_UNSUPPORTED);
  }
  CHECK(hstu_layer_workspace_bytes(nullptr) == 0);
}

// ---- oracle ---------------------------------------------------------------
static void oracle_case(const std::vector<int32_t>& lengths, int H, int d, int W, int c,
                        bool targets, bool clamp, uint32_t seed) {
  const int B = (int)lengths.size();
  std::vector<int32_t> off(B + 1, 0), nt(B, 0);
  for (int b = 0; b < B; ++b) off[b + 1] = off[b] + lengths[b];
  const int N = off[B];
  std::mt19937 rng(seed);
  std::normal_distribution<double> nd(0.0, 1.0);
  std::uniform_int_distribution<int> ud(0, 9);
  for (int b = 0; b < B; ++b) nt[b] = targets ? ud(rng) : 0;
  const int64_t ld = (int64_t)H * d;
  const size_t n_el = (size_t)std::max(N, 1) * ld;   // one row at least: non-null buffers
  std::vector<double> q(n_el), k(n_el), v(n_el), u(n_el), out(n_el, 0.0);
  for (auto* x : {&q, &k, &v, &u})
    for (auto& e : *x) e = nd(rng);
  std::vector<int64_t> ts(std::max(N, 1));
  int64_t t = 1700000000;
  for (int i = 0; i < N; ++i) ts[i] = (t += ud(rng) * 1000);
  const int P = 40, T = 64;
  std::vector<double> pos(P), tim(T);
  for (auto& e : pos) e = 0.1 * nd(rng);
  for (auto& e : tim) e = 0.1 * nd(rng);
  for (int ep = 0; ep < 3; ++ep) {
    CHECK(hstu_oracle_fwd(B, off.data(), H, d, d, q.data(), ld, k.data(), ld, v.data(), ld,
                          u.data(), ld, ts.data(), targets ? nt.data() : nullptr, c, W, 0.3,
                          64.0, pos.data(), P, tim.data(), T, 1e-5, ep, out.data(), ld, nullptr,
                          1, clamp ? 1 : 0) == 0);
    for (double e : out) CHECK(std::isfinite(e));
  }
  std::vector<double> dout(n_el), dq(n_el), dk(n_el), dv(n_el), du(n_el), dpos(P), dtime(T);
  for (auto& e : dout) e = nd(rng);
  for (int ep = 0; ep < 3; ++ep) {
    CHECK(hstu_oracle_bwd(B, off.data(), H, d, d, q.data(), ld, k.data(), ld, v.data(), ld,
                          u.data(), ld, ts.data(), targets ? nt.data() : nullptr, c, W, 0.3,
                          64.0, pos.data(), P, tim.data(), T, 1e-5, ep, dout.data(), ld,
                          dq.data(), dk.data(), dv.data(), du.data(), dpos.data(), dtime.data(),
                          1, clamp ? 1 : 0) == 0);
    for (auto* x : {&dq, &dk, &dv, &du, &dpos, &dtime})
      for (double e : *x) CHECK(std::isfinite(e));
  }
  // a bad argument is refused, not read past
  CHECK(hstu_oracle_fwd(B, off.data(), 0, d, d, q.data(), ld, k.data(), ld, v.data(), ld,
                        u.data(), ld, nullptr, nullptr, 0, 0, 0.3, 64.0, nullptr, 0, nullptr, 0,
                        1e-5, 0, out.data(), ld, nullptr, 1, 0) == -1);
}

static void oracle_checks() {
  oracle_case({0, 1, 2, 33, 70, 0}, 2, 8, 0, 0, false, false, 1);
  oracle_case({5, 40, 17}, 1, 16, 7, 3, true, false, 2);
  oracle_case({64, 1, 30}, 3, 8, 0, 2, true, true, 3);
  oracle_case({}, 1, 8, 0, 0, false, false, 4);
}

int main() {
  abi_checks();
  oracle_checks();
  std::printf("ok: %d checks\n", g_checks);
  return 0;
}
