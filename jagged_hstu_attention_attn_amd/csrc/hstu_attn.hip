// hstu_attn.hip -- host side of the C ABI declared in include/hstu_attn.h:
// argument validation (before any HIP call), workspace sizing, launches of the
// scheduler and attention kernels on the caller's stream, error reporting.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <mutex>
#include <cstdio>
#include <cstring>

#include "hstu_attn.h"
#include "gemm.hpp"
#include "hstu_device.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

size_t elem_size(int32_t dtype) { return dtype == HSTU_DTYPE_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Work-list layout of a forward call.  Partial-output slots are reserved
// only when an item of the batch can be split along its keys (some sequence
// may reach kMinSplitTokens) and the call allows splitting.
hstu::PlanLayout fwd_layout(const hstu_attn_desc* d, bool no_split = false) {
  const bool splits = !no_split && (int64_t)d->total_tokens >= hstu::kMinSplitTokens;
  return hstu::plan_layout(d->num_seqs, d->total_tokens, d->num_heads, d->d_v, splits);
}

constexpr int64_t kMaxRowBytes = int64_t(1) << 24;   // bytes of one token row, any tensor

int check_desc(const hstu_attn_desc* d) {
  if (!d) return fail(HSTU_ERR_INVALID_ARG, "desc is NULL");
  if (d->num_seqs < 0) return fail(HSTU_ERR_INVALID_ARG, "num_seqs < 0 (%d)", d->num_seqs);
  if (d->total_tokens < 0)
    return fail(HSTU_ERR_INVALID_ARG, "total_tokens < 0 (%d)", d->total_tokens);
  if (d->num_heads < 1) return fail(HSTU_ERR_INVALID_ARG, "num_heads < 1 (%d)", d->num_heads);
  if (d->dtype != HSTU_DTYPE_F32 && d->dtype != HSTU_DTYPE_BF16)
    return fail(HSTU_ERR_INVALID_ARG, "unknown dtype %d", d->dtype);
  if (d->epilogue != HSTU_EPILOGUE_LN_U && d->epilogue != HSTU_EPILOGUE_NONE &&
      d->epilogue != HSTU_EPILOGUE_LN_ALL_U)
    return fail(HSTU_ERR_INVALID_ARG, "unknown epilogue %d", d->epilogue);
  if (d->pos_clamp != 0 && d->pos_clamp != 1)
    return fail(HSTU_ERR_INVALID_ARG, "pos_clamp must be 0 or 1 (%d)", d->pos_clamp);
  if (d->d_qk <= 0 || d->d_v <= 0)
    return fail(HSTU_ERR_INVALID_ARG, "d_qk and d_v must be positive (%d, %d)", d->d_qk, d->d_v);
  if (!hstu::attn_supported(d->dtype, d->d_qk, d->d_v))
    return fail(HSTU_ERR_UNSUPPORTED, "unsupported (dtype=%d, d_qk=%d, d_v=%d)", d->dtype,
                d->d_qk, d->d_v);
  if (d->pos_table_len < 0 || d->time_table_len < 0)
    return fail(HSTU_ERR_INVALID_ARG, "negative table length");
  if (d->pos_table_len > hstu::kPosMax)
    return fail(HSTU_ERR_UNSUPPORTED, "pos_table_len %d exceeds %d", d->pos_table_len,
                hstu::kPosMax);
  if (!(d->ln_eps > 0.0f) || !std::isfinite(d->ln_eps))
    return fail(HSTU_ERR_INVALID_ARG, "ln_eps must be positive and finite");
  if (d->epilogue == HSTU_EPILOGUE_LN_ALL_U &&
      (int64_t)d->num_heads * d->d_v > hstu::ln_all_heads_max_width(d->dtype))
    return fail(HSTU_ERR_UNSUPPORTED, "LayerNorm over all heads supports H*d_v <= %d",
                hstu::ln_all_heads_max_width(d->dtype));
  const int64_t H = d->num_heads;
  const size_t es = elem_size(d->dtype);
  struct {
    const char* name;
    int64_t ld;
    int64_t need;
  } lds[] = {{"ld_q", d->ld_q, H * d->d_qk}, {"ld_k", d->ld_k, H * d->d_qk},
             {"ld_v", d->ld_v, H * d->d_v},  {"ld_u", d->ld_u, H * d->d_v},
             {"ld_out", d->ld_out, H * d->d_v}};
  for (auto& x : lds) {
    if (x.name[3] == 'u' && d->epilogue == HSTU_EPILOGUE_NONE) continue;  // u unused
    if (x.ld < x.need)
      return fail(HSTU_ERR_INVALID_ARG, "%s = %lld is below H*d = %lld", x.name,
                  (long long)x.ld, (long long)x.need);
    if ((x.ld * (int64_t)es) % 16 != 0)
      return fail(HSTU_ERR_INVALID_ARG, "%s * element size must be a multiple of 16 bytes",
                  x.name);
    // the kernels form a copy's offset within a tile as a 32-bit row * stride
    // (rows below 256), so a token row may span at most 16 MiB
    if (x.ld * (int64_t)es > kMaxRowBytes)
      return fail(HSTU_ERR_UNSUPPORTED, "%s * element size = %lld bytes exceeds %lld", x.name,
                  (long long)(x.ld * (int64_t)es), (long long)kMaxRowBytes);
  }
  const hstu::PlanLayout pl = fwd_layout(d);
  if (2 * pl.units_max > 0x7fffffffLL || (int64_t)d->num_seqs * H > 0x7fffffffLL)
    return fail(HSTU_ERR_UNSUPPORTED, "too many work items (%lld)", (long long)pl.items_max);
  return HSTU_OK;
}

int check_plan_args(const hstu_attn_desc* d, const int32_t* offsets, int32_t contextual_len,
                    int32_t max_attn_len, const void* ws, size_t ws_bytes,
                    bool no_split = false) {
  if (d->num_seqs > 0 && !offsets) return fail(HSTU_ERR_INVALID_ARG, "offsets is NULL");
  if (contextual_len < 0) return fail(HSTU_ERR_INVALID_ARG, "contextual_len < 0");
  if (max_attn_len < 0) return fail(HSTU_ERR_INVALID_ARG, "max_attn_len < 0");
  const size_t need = fwd_layout(d, no_split).total;
  if (!ws) return fail(HSTU_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (ws_bytes < need)
    return fail(HSTU_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, need);
  if (!aligned16(ws)) return fail(HSTU_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  return HSTU_OK;
}

int check_run_args(const hstu_attn_desc* d, const void* q, const void* k, const void* v,
                   const void* u, const int64_t* timestamps, float alpha, float n_scale,
                   const float* pos_table, const float* time_table, const void* out) {
  struct {
    const char* name;
    const void* p;
  } ptrs[] = {{"q", q}, {"k", k}, {"v", v}, {"out", out}, {"u", u}};
  for (auto& x : ptrs) {
    if (x.name[0] == 'u' && d->epilogue == HSTU_EPILOGUE_NONE) continue;
    if (!x.p) return fail(HSTU_ERR_INVALID_ARG, "%s is NULL", x.name);
    if (!aligned16(x.p)) return fail(HSTU_ERR_INVALID_ARG, "%s is not 16-byte aligned", x.name);
  }
  if ((pos_table == nullptr) != (d->pos_table_len == 0))
    return fail(HSTU_ERR_INVALID_ARG, "pos_table and pos_table_len disagree");
  if ((time_table == nullptr) != (d->time_table_len == 0))
    return fail(HSTU_ERR_INVALID_ARG, "time_table and time_table_len disagree");
  if (time_table && !timestamps)
    return fail(HSTU_ERR_INVALID_ARG, "a time bias needs timestamps");
  if (!(n_scale > 0.0f) || !std::isfinite(n_scale))
    return fail(HSTU_ERR_INVALID_ARG, "n_scale must be positive and finite");
  if (!std::isfinite(alpha)) return fail(HSTU_ERR_INVALID_ARG, "alpha must be finite");
  return HSTU_OK;
}

// Which forward kernel runs: HSTU_FWD_KERNEL_AUTO takes the sixteen-row
// kernel where it is built (bf16, d = 128) and the four-wave kernel
// elsewhere; the eight-wave kernel runs only when chosen explicitly.
std::atomic<int> g_fwd_kernel{HSTU_FWD_KERNEL_AUTO};

int fwd_kernel_choice(const hstu_attn_desc* d, bool transposed = false) {
  if (transposed) return HSTU_FWD_KERNEL_SIXTEEN_ROW;   // the only kernel with that walk
  const int mode = g_fwd_kernel.load(std::memory_order_relaxed);
  if (mode == HSTU_FWD_KERNEL_EIGHT_WAVE && hstu::attn_pp_supported(d->dtype, d->d_qk, d->d_v))
    return HSTU_FWD_KERNEL_EIGHT_WAVE;
  const bool w16 = hstu::attn_w16_supported(d->dtype, d->d_qk, d->d_v);
  if (mode == HSTU_FWD_KERNEL_SIXTEEN_ROW && w16) return HSTU_FWD_KERNEL_SIXTEEN_ROW;
  if (mode == HSTU_FWD_KERNEL_THIRTYTWO_ROW && hstu::attn_w32_supported(d->dtype, d->d_qk, d->d_v))
    return HSTU_FWD_KERNEL_THIRTYTWO_ROW;
  if (mode == HSTU_FWD_KERNEL_AUTO && w16 && hstu::kW16Auto) return HSTU_FWD_KERNEL_SIXTEEN_ROW;
  return HSTU_FWD_KERNEL_FOUR_WAVE;
}

// Workgroups of the persistent attention launch: CUs x resident workgroups
// per CU (cached per device and kernel variant), between 8 (one per XCD) and
// kMaxGrid (the most a plan serves).  <= 0 on a HIP error.
int persistent_grid(const hstu_attn_desc* d, bool transposed = false) {
  struct Entry {
    int dev, dtype, d_qk, d_v, pos_len, has_time, clamp, kern, grid;
  };
  static thread_local Entry cache[16];
  static thread_local int cache_n = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const int has_time = d->time_table_len > 0;
  const int clamp = d->pos_clamp != 0 && d->pos_table_len > 0;
  const int kern = fwd_kernel_choice(d, transposed) + (transposed ? 100 : 0);   // cache key
  int g = -1;
  for (int i = 0; i < cache_n && i < 16; ++i) {
    const Entry& e = cache[i];
    if (e.dev == dev && e.dtype == d->dtype && e.d_qk == d->d_qk && e.d_v == d->d_v &&
        e.pos_len == d->pos_table_len && e.has_time == has_time && e.clamp == clamp &&
        e.kern == kern) {
      g = e.grid;
      break;
    }
  }
  if (g < 0) {
    g = kern == HSTU_FWD_KERNEL_EIGHT_WAVE
            ? hstu::attn_pp_grid(d->pos_table_len, d->time_table_len, clamp != 0)
        : kern == HSTU_FWD_KERNEL_SIXTEEN_ROW || transposed
            ? hstu::attn_w16_grid(d->pos_table_len, d->time_table_len, clamp != 0, transposed)
        : kern == HSTU_FWD_KERNEL_THIRTYTWO_ROW
            ? hstu::attn_w32_grid(d->pos_table_len, d->time_table_len, clamp != 0)
            : hstu::attn_grid(d->dtype, d->d_qk, d->d_v, d->pos_table_len, d->time_table_len,
                              clamp != 0);
    if (g <= 0) return g;
    cache[cache_n % 16] =
        Entry{dev, d->dtype, d->d_qk, d->d_v, d->pos_table_len, has_time, clamp, kern, g};
    ++cache_n;
  }
  // at least one workgroup per XCD, at most what a plan serves
  return g < hstu::kXcds ? hstu::kXcds : (g < hstu::kMaxGrid ? g : hstu::kMaxGrid);
}

struct PlanPtrs {
  int32_t* hdr;
  int4* units;
  int32_t* wg;
  int32_t* counters;
  float* partials;
  int32_t* seq;
  char* items;
  int64_t slot_floats;
};

PlanPtrs plan_ptrs(const hstu_attn_desc* d, void* ws, bool no_split = false) {
  const hstu::PlanLayout pl = fwd_layout(d, no_split);
  char* base = static_cast<char*>(ws);
  PlanPtrs p;
  p.hdr = reinterpret_cast<int32_t*>(base + pl.hdr_off);
  p.units = reinterpret_cast<int4*>(base + pl.units_off);
  p.wg = reinterpret_cast<int32_t*>(base + pl.wg_off);
  p.counters = reinterpret_cast<int32_t*>(base + pl.ctr_off);
  p.partials = reinterpret_cast<float*>(base + pl.part_off);
  p.seq = reinterpret_cast<int32_t*>(base + pl.seq_off);
  p.items = base + pl.item_off;
  p.slot_floats = pl.slot_floats;
  return p;
}

}  // namespace

extern "C" {

int hstu_jagged_attn_supported(int32_t dtype, int32_t d_qk, int32_t d_v) {
  return hstu::attn_supported(dtype, d_qk, d_v) ? 1 : 0;
}

size_t hstu_jagged_attn_workspace_bytes(const hstu_attn_desc* desc) {
  if (check_desc(desc) != HSTU_OK) return 0;
  return fwd_layout(desc).total;
}

static int plan_impl(const hstu_attn_desc* desc, const int32_t* offsets,
                     const int32_t* num_targets, int32_t contextual_len, int32_t max_attn_len,
                     void* workspace, size_t workspace_bytes, void* stream, bool cand_only,
                     bool no_split = false, bool transposed = false) {
  int rc = check_desc(desc);
  if (rc != HSTU_OK) return rc;
  rc = check_plan_args(desc, offsets, contextual_len, max_attn_len, workspace, workspace_bytes,
                       no_split);
  if (rc != HSTU_OK) return rc;
  if (desc->num_seqs == 0 || desc->total_tokens == 0) return HSTU_OK;
  const hstu::PlanLayout pl = fwd_layout(desc, no_split);
  const PlanPtrs pp = plan_ptrs(desc, workspace, no_split);
  const int n_wg = persistent_grid(desc, transposed);
  if (n_wg <= 0) return fail(HSTU_ERR_HIP, "cannot query the device for the launch size");
  hstu::PlanArgs a;
  a.offsets = offsets;
  a.num_targets = num_targets;
  a.num_seqs = desc->num_seqs;
  a.num_heads = desc->num_heads;
  a.contextual_len = contextual_len;
  a.max_attn_len = max_attn_len;
  a.items_max = (int32_t)pl.items_max;
  a.n_wg = n_wg;
  a.cand_only = cand_only ? 1 : 0;
  a.no_split = pl.slots_max == 0 ? 1 : 0;
  a.transposed = transposed ? 1 : 0;
  a.hdr = pp.hdr;
  a.units = pp.units;
  a.wg = pp.wg;
  a.counters = pp.counters;
  a.seq_scratch = pp.seq;
  a.item_scratch = pp.items;
  const bool compact = hstu::plan_is_compact(pl.items_max, desc->total_tokens);
  const hipError_t e = hstu::launch_plan(a, compact, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(HSTU_ERR_HIP, "scheduler launch failed: %s", hipGetErrorString(e));
  return HSTU_OK;
}

int hstu_jagged_attn_plan(const hstu_attn_desc* desc, const int32_t* offsets,
                          const int32_t* num_targets, int32_t contextual_len,
                          int32_t max_attn_len, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return plan_impl(desc, offsets, num_targets, contextual_len, max_attn_len, workspace,
                   workspace_bytes, stream, false);
}

int hstu_jagged_attn_plan_candidates(const hstu_attn_desc* desc, const int32_t* offsets,
                                     const int32_t* num_targets, int32_t contextual_len,
                                     int32_t max_attn_len, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return plan_impl(desc, offsets, num_targets, contextual_len, max_attn_len, workspace,
                   workspace_bytes, stream, true);
}

static int run_impl(const hstu_attn_desc* desc, const void* q, const void* k, const void* v,
                    const void* u, const int32_t* offsets, const int64_t* timestamps,
                    const int32_t* num_targets, int32_t contextual_len, int32_t max_attn_len,
                    float alpha, float n_scale, const float* pos_table,
                    const float* time_table, void* out, void* o_raw, void* workspace,
                    size_t workspace_bytes, void* stream, void* t_start = nullptr,
                    void* t_stop = nullptr, bool no_split = false, bool transposed = false) {
  int rc = check_desc(desc);
  if (rc != HSTU_OK) return rc;
  rc = check_plan_args(desc, offsets, contextual_len, max_attn_len, workspace, workspace_bytes,
                       no_split);
  if (rc != HSTU_OK) return rc;
  if (desc->num_seqs == 0 || desc->total_tokens == 0) return HSTU_OK;
  rc = check_run_args(desc, q, k, v, u, timestamps, alpha, n_scale, pos_table, time_table, out);
  if (rc != HSTU_OK) return rc;

  const int n_wg = persistent_grid(desc, transposed);
  if (n_wg <= 0) return fail(HSTU_ERR_HIP, "cannot query the device for the launch size");
  const PlanPtrs pp = plan_ptrs(desc, workspace, no_split);
  hstu::AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  // LayerNorm over all heads: the attention writes O / n_scale, a second pass
  // normalises every token's heads together
  const bool ln_all = desc->epilogue == HSTU_EPILOGUE_LN_ALL_U;
  a.u = (desc->epilogue == HSTU_EPILOGUE_NONE || ln_all) ? nullptr : u;
  a.out = out;
  a.offsets = offsets;
  a.timestamps = time_table ? timestamps : nullptr;
  a.num_targets = num_targets;
  a.pos_table = pos_table;
  a.time_table = time_table;
  a.hdr = pp.hdr;
  a.units = pp.units;
  a.wg = pp.wg;
  a.counters = pp.counters;
  a.partials = pp.partials;
  a.slot_floats = pp.slot_floats;
  a.ld_q = desc->ld_q;
  a.ld_k = desc->ld_k;
  a.ld_v = desc->ld_v;
  a.ld_u = desc->ld_u;
  a.ld_out = desc->ld_out;
  a.num_heads = desc->num_heads;
  a.contextual_len = contextual_len;
  a.max_attn_len = max_attn_len;
  a.pos_len = desc->pos_table_len;
  a.time_len = desc->time_table_len;
  a.epilogue = ln_all ? HSTU_EPILOGUE_NONE : desc->epilogue;
  a.pos_clamp = desc->pos_clamp;
  a.out_raw = o_raw;
  a.ld_raw = (int64_t)desc->num_heads * desc->d_v;
  a.alpha = alpha;
  a.out_scale = (float)(0.69314718055994530942 / (double)n_scale);
  a.ln_eps = desc->ln_eps;
  const int kern = fwd_kernel_choice(desc, transposed);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = static_cast<hipEvent_t>(t_start), e1 = static_cast<hipEvent_t>(t_stop);
  const hipError_t e =
      kern == HSTU_FWD_KERNEL_EIGHT_WAVE    ? hstu::launch_attn_pp(a, n_wg, st, e0, e1)
      : kern == HSTU_FWD_KERNEL_SIXTEEN_ROW
          ? hstu::launch_attn_w16(a, n_wg, st, e0, e1, transposed)
      : kern == HSTU_FWD_KERNEL_THIRTYTWO_ROW ? hstu::launch_attn_w32(a, n_wg, st, e0, e1)
          : hstu::launch_attn(a, desc->dtype, desc->d_qk, desc->d_v, n_wg, st, e0, e1);
  if (e != hipSuccess)
    return fail(HSTU_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  if (ln_all) {
    hstu::LnArgs la;
    la.out = out;
    la.u = u;
    la.ld_out = desc->ld_out;
    la.ld_u = desc->ld_u;
    la.offsets = offsets;
    la.num_targets = num_targets;
    la.hdr = pp.hdr;
    la.num_seqs = desc->num_seqs;
    la.n_tok = desc->total_tokens;
    la.width = desc->num_heads * desc->d_v;
    la.eps = desc->ln_eps;
    const hipError_t e2 = hstu::launch_ln_all_heads(la, desc->dtype,
                                                    static_cast<hipStream_t>(stream));
    if (e2 != hipSuccess)
      return fail(HSTU_ERR_HIP, "LayerNorm launch failed: %s", hipGetErrorString(e2));
  }
  return HSTU_OK;
}

int hstu_jagged_attn_run(const hstu_attn_desc* desc, const void* q, const void* k,
                         const void* v, const void* u, const int32_t* offsets,
                         const int64_t* timestamps, const int32_t* num_targets,
                         int32_t contextual_len, int32_t max_attn_len, float alpha,
                         float n_scale, const float* pos_table, const float* time_table,
                         void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return run_impl(desc, q, k, v, u, offsets, timestamps, num_targets, contextual_len,
                  max_attn_len, alpha, n_scale, pos_table, time_table, out, nullptr, workspace,
                  workspace_bytes, stream);
}

int hstu_jagged_attn_run_timed(const hstu_attn_desc* desc, const void* q, const void* k,
                               const void* v, const void* u, const int32_t* offsets,
                               const int64_t* timestamps, const int32_t* num_targets,
                               int32_t contextual_len, int32_t max_attn_len, float alpha,
                               float n_scale, const float* pos_table, const float* time_table,
                               void* out, void* workspace, size_t workspace_bytes, void* stream,
                               void* start_event, void* stop_event) {
  return run_impl(desc, q, k, v, u, offsets, timestamps, num_targets, contextual_len,
                  max_attn_len, alpha, n_scale, pos_table, time_table, out, nullptr, workspace,
                  workspace_bytes, stream, start_event, stop_event);
}

int hstu_jagged_attn_fwd_train(const hstu_attn_desc* desc, const void* q, const void* k,
                               const void* v, const void* u, const int32_t* offsets,
                               const int64_t* timestamps, const int32_t* num_targets,
                               int32_t contextual_len, int32_t max_attn_len, float alpha,
                               float n_scale, const float* pos_table, const float* time_table,
                               void* out, void* o_raw, void* workspace, size_t workspace_bytes,
                               void* stream) {
  int rc = check_desc(desc);
  if (rc != HSTU_OK) return rc;
  rc = check_plan_args(desc, offsets, contextual_len, max_attn_len, workspace, workspace_bytes);
  if (rc != HSTU_OK) return rc;
  if (desc->num_seqs == 0 || desc->total_tokens == 0) return HSTU_OK;
  rc = check_run_args(desc, q, k, v, u, timestamps, alpha, n_scale, pos_table, time_table, out);
  if (rc != HSTU_OK) return rc;
  if (!o_raw) return fail(HSTU_ERR_INVALID_ARG, "o_raw is NULL");
  if (!aligned16(o_raw)) return fail(HSTU_ERR_INVALID_ARG, "o_raw is not 16-byte aligned");
  rc = hstu_jagged_attn_plan(desc, offsets, num_targets, contextual_len, max_attn_len, workspace,
                             workspace_bytes, stream);
  if (rc != HSTU_OK) return rc;
  return run_impl(desc, q, k, v, u, offsets, timestamps, num_targets, contextual_len,
                  max_attn_len, alpha, n_scale, pos_table, time_table, out, o_raw, workspace,
                  workspace_bytes, stream);
}

int hstu_jagged_attn_fwd(const hstu_attn_desc* desc, const void* q, const void* k,
                         const void* v, const void* u, const int32_t* offsets,
                         const int64_t* timestamps, const int32_t* num_targets,
                         int32_t contextual_len, int32_t max_attn_len, float alpha,
                         float n_scale, const float* pos_table, const float* time_table,
                         void* out, void* workspace, size_t workspace_bytes, void* stream) {
  // Validate everything before the first launch so that a bad call enqueues nothing.
  int rc = check_desc(desc);
  if (rc != HSTU_OK) return rc;
  rc = check_plan_args(desc, offsets, contextual_len, max_attn_len, workspace, workspace_bytes);
  if (rc != HSTU_OK) return rc;
  if (desc->num_seqs == 0 || desc->total_tokens == 0) return HSTU_OK;
  rc = check_run_args(desc, q, k, v, u, timestamps, alpha, n_scale, pos_table, time_table, out);
  if (rc != HSTU_OK) return rc;
  rc = hstu_jagged_attn_plan(desc, offsets, num_targets, contextual_len, max_attn_len, workspace,
                             workspace_bytes, stream);
  if (rc != HSTU_OK) return rc;
  return hstu_jagged_attn_run(desc, q, k, v, u, offsets, timestamps, num_targets, contextual_len,
                              max_attn_len, alpha, n_scale, pos_table, time_table, out,
                              workspace, workspace_bytes, stream);
}

int hstu_jagged_attn_fwd_candidates(const hstu_attn_desc* desc, const void* q, const void* k,
                         const void* v, const void* u, const int32_t* offsets,
                         const int64_t* timestamps, const int32_t* num_targets,
                         int32_t contextual_len, int32_t max_attn_len, float alpha,
                         float n_scale, const float* pos_table, const float* time_table,
                         void* out, void* workspace, size_t workspace_bytes, void* stream) {
  // Validate everything before the first launch so that a bad call enqueues nothing.
  int rc = check_desc(desc);
  if (rc != HSTU_OK) return rc;
  rc = check_plan_args(desc, offsets, contextual_len, max_attn_len, workspace, workspace_bytes);
  if (rc != HSTU_OK) return rc;
  if (desc->num_seqs == 0 || desc->total_tokens == 0) return HSTU_OK;
  rc = check_run_args(desc, q, k, v, u, timestamps, alpha, n_scale, pos_table, time_table, out);
  if (rc != HSTU_OK) return rc;
  rc = hstu_jagged_attn_plan_candidates(desc, offsets, num_targets, contextual_len,
                                        max_attn_len, workspace, workspace_bytes, stream);
  if (rc != HSTU_OK) return rc;
  return hstu_jagged_attn_run(desc, q, k, v, u, offsets, timestamps, num_targets, contextual_len,
                              max_attn_len, alpha, n_scale, pos_table, time_table, out,
                              workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- allocation-free forward ---------------------------------------------
//
// hstu_jagged_attn_fwd_noalloc keeps its work list in `scratch`, an array of
// this file that every GPU the library runs on holds from module load until
// the process ends.  Host code never passes the array's name to a kernel or a
// copy (on the host it is only a stand-in for the symbol): its device address
// is looked up once per device with hipGetSymbolAddress, with that device
// current, and that address is what the scheduler and attention kernels take.
// The call plans without key splits, so the array holds the unit list, the
// per-workgroup shares and, for large batches, the scheduler's per-sequence
// and per-item scratch -- never partial outputs.
namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;   // 8 MiB per device
constexpr int kScratchDevices = 64;

}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call on that device; a negative status (message set) on failure.
int scratch_on_current_device(void** out) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HSTU_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kScratchDevices)
    return fail(HSTU_ERR_UNSUPPORTED, "device %d is beyond the %d the allocation-free call serves",
                dev, kScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t r = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (r != hipSuccess || ptr == nullptr)
      return fail(HSTU_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(r));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return HSTU_OK;
}

}  // namespace

extern "C" {

int hstu_jagged_attn_fwd_noalloc(const hstu_attn_desc* desc, const void* q, const void* k,
                                 const void* v, const void* u, const int32_t* offsets,
                                 const int64_t* timestamps, const int32_t* num_targets,
                                 int32_t contextual_len, int32_t max_attn_len, float alpha,
                                 float n_scale, const float* pos_table,
                                 const float* time_table, void* out, void* stream) {
  int rc = check_desc(desc);
  if (rc != HSTU_OK) return rc;
  if (desc->num_seqs > 0 && !offsets) return fail(HSTU_ERR_INVALID_ARG, "offsets is NULL");
  if (contextual_len < 0) return fail(HSTU_ERR_INVALID_ARG, "contextual_len < 0");
  if (max_attn_len < 0) return fail(HSTU_ERR_INVALID_ARG, "max_attn_len < 0");
  const size_t need = fwd_layout(desc, true).total;
  if (need > kScratchBytes)
    return fail(HSTU_ERR_WORKSPACE,
                "the batch needs %zu bytes of work list; the allocation-free call holds %zu "
                "(use hstu_jagged_attn_fwd with a caller workspace)",
                need, kScratchBytes);
  if (desc->num_seqs == 0 || desc->total_tokens == 0) return HSTU_OK;
  rc = check_run_args(desc, q, k, v, u, timestamps, alpha, n_scale, pos_table, time_table, out);
  if (rc != HSTU_OK) return rc;
  void* ws = nullptr;
  rc = scratch_on_current_device(&ws);
  if (rc != HSTU_OK) return rc;
  rc = plan_impl(desc, offsets, num_targets, contextual_len, max_attn_len, ws, kScratchBytes,
                 stream, false, true);
  if (rc != HSTU_OK) return rc;
  return run_impl(desc, q, k, v, u, offsets, timestamps, num_targets, contextual_len,
                  max_attn_len, alpha, n_scale, pos_table, time_table, out, nullptr, ws,
                  kScratchBytes, stream, nullptr, nullptr, true);
}

int64_t hstu_jagged_attn_valid_pairs(int32_t num_seqs, const int32_t* offsets_host,
                                     const int32_t* num_targets_host, int32_t contextual_len,
                                     int32_t max_attn_len) {
  if (num_seqs < 0) return fail(-1, "num_seqs < 0");
  if (num_seqs > 0 && !offsets_host) return fail(-1, "offsets is NULL");
  if (contextual_len < 0 || max_attn_len < 0) return fail(-1, "negative mask parameter");
  int64_t n = 0;
  for (int b = 0; b < num_seqs; ++b) {
    const int L = offsets_host[b + 1] - offsets_host[b];
    if (L < 0) return fail(-1, "offsets decrease at sequence %d", b);
    const hstu::SeqGeom g = hstu::seq_geom(
        L, num_targets_host ? num_targets_host[b] : 0, contextual_len, max_attn_len);
    for (int i = 0; i < L; ++i) {
      const hstu::RowBounds r = hstu::row_bounds(g, i);
      if (r.lo != hstu::kEmptyLo) n += r.span + 1;
      if (r.self_j >= 0) n += 1;
    }
  }
  return n;
}

int hstu_jagged_attn_set_fwd_kernel(int32_t mode) {
  if (mode != HSTU_FWD_KERNEL_AUTO && mode != HSTU_FWD_KERNEL_FOUR_WAVE &&
      mode != HSTU_FWD_KERNEL_EIGHT_WAVE && mode != HSTU_FWD_KERNEL_SIXTEEN_ROW &&
      mode != HSTU_FWD_KERNEL_THIRTYTWO_ROW)
    return fail(HSTU_ERR_INVALID_ARG, "unknown forward kernel mode %d", mode);
  g_fwd_kernel.store(mode, std::memory_order_relaxed);
  return HSTU_OK;
}

int hstu_jagged_attn_fwd_kernel_of(const hstu_attn_desc* desc) {
  if (check_desc(desc) != HSTU_OK) return -1;
  return fwd_kernel_choice(desc);
}

int hstu_jagged_attn_grid(const hstu_attn_desc* desc) {
  if (check_desc(desc) != HSTU_OK) return -1;
  const int g = persistent_grid(desc);
  if (g <= 0) return fail(-1, "cannot query the device for the launch size");
  return g;
}

const char* hstu_last_error(void) { return g_err; }

}  // extern "C"

// ---- full HSTU layer ------------------------------------------------------

namespace {

struct LayerLayout {
  size_t xn_off, uvqk_off, attn_off, attn_ws_off, total;
  int64_t uvqk_w;   // H * (2 d_v + 2 d_qk)
};

hstu_attn_desc layer_attn_desc(const hstu_layer_desc* d) {
  hstu_attn_desc a;
  a.num_seqs = d->num_seqs;
  a.total_tokens = d->total_tokens;
  a.num_heads = d->num_heads;
  a.d_qk = d->d_qk;
  a.d_v = d->d_v;
  a.dtype = HSTU_DTYPE_BF16;
  const int64_t w = (int64_t)d->num_heads * (2 * d->d_v + 2 * d->d_qk);
  a.ld_q = a.ld_k = a.ld_v = a.ld_u = w;
  a.ld_out = (int64_t)d->num_heads * d->d_v;
  a.pos_table_len = d->pos_table_len;
  a.time_table_len = d->time_table_len;
  a.ln_eps = d->ln_eps;
  a.epilogue = HSTU_EPILOGUE_LN_U;
  a.pos_clamp = 0;
  return a;
}

LayerLayout layer_layout(const hstu_layer_desc* d) {
  LayerLayout l;
  const int64_t N = d->total_tokens, H = d->num_heads;
  l.uvqk_w = H * (2 * d->d_v + 2 * d->d_qk);
  l.xn_off = 0;
  l.uvqk_off = hstu::align256(l.xn_off + (size_t)N * d->hidden * 2);
  l.attn_off = hstu::align256(l.uvqk_off + (size_t)N * l.uvqk_w * 2);
  l.attn_ws_off = hstu::align256(l.attn_off + (size_t)N * H * d->d_v * 2);
  const hstu_attn_desc a_desc = layer_attn_desc(d);
  l.total = l.attn_ws_off + fwd_layout(&a_desc).total;
  return l;
}

int check_layer_desc(const hstu_layer_desc* d) {
  if (!d) return fail(HSTU_ERR_INVALID_ARG, "desc is NULL");
  if (d->hidden <= 0) return fail(HSTU_ERR_INVALID_ARG, "hidden must be positive");
  if (d->hidden % 128 != 0 || d->hidden > hstu::layernorm_rows_max_width())
    return fail(HSTU_ERR_UNSUPPORTED, "hidden must be a multiple of 128 up to %d",
                hstu::layernorm_rows_max_width());
  const hstu_attn_desc a = layer_attn_desc(d);
  int rc = check_desc(&a);
  if (rc != HSTU_OK) return rc;
  const int64_t w = (int64_t)d->num_heads * (2 * d->d_v + 2 * d->d_qk);
  if (w % 128 != 0 || ((int64_t)d->num_heads * d->d_v) % 64 != 0)
    return fail(HSTU_ERR_UNSUPPORTED, "H*(2 d_v + 2 d_qk) must be a multiple of 128 and "
                "H*d_v of 64");
  return HSTU_OK;
}

}  // namespace

extern "C" {

size_t hstu_layer_workspace_bytes(const hstu_layer_desc* desc) {
  if (check_layer_desc(desc) != HSTU_OK) return 0;
  return layer_layout(desc).total;
}

int hstu_layer_fwd(const hstu_layer_desc* desc, const void* x, const void* w_uvqk,
                   const void* b_uvqk, const void* w_o, const int32_t* offsets,
                   const int64_t* timestamps, const int32_t* num_targets, int32_t contextual_len,
                   int32_t max_attn_len, float alpha, float n_scale, const float* pos_table,
                   const float* time_table, void* y, void* workspace, size_t workspace_bytes,
                   void* stream) {
  int rc = check_layer_desc(desc);
  if (rc != HSTU_OK) return rc;
  struct {
    const char* name;
    const void* p;
  } ptrs[] = {{"x", x}, {"w_uvqk", w_uvqk}, {"b_uvqk", b_uvqk}, {"w_o", w_o}, {"y", y}};
  for (auto& e : ptrs) {
    if (!e.p) return fail(HSTU_ERR_INVALID_ARG, "%s is NULL", e.name);
    if (!aligned16(e.p)) return fail(HSTU_ERR_INVALID_ARG, "%s is not 16-byte aligned", e.name);
  }
  const LayerLayout l = layer_layout(desc);
  if (!workspace) return fail(HSTU_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", l.total);
  if (workspace_bytes < l.total)
    return fail(HSTU_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, l.total);
  if (!aligned16(workspace)) return fail(HSTU_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  const hstu_attn_desc ad = layer_attn_desc(desc);
  char* ws = static_cast<char*>(workspace);
  __bf16* xn = reinterpret_cast<__bf16*>(ws + l.xn_off);
  __bf16* uvqk = reinterpret_cast<__bf16*>(ws + l.uvqk_off);
  __bf16* attn = reinterpret_cast<__bf16*>(ws + l.attn_off);
  const size_t attn_ws_bytes = l.total - l.attn_ws_off;
  // the attention's arguments are checked before anything is enqueued
  rc = check_plan_args(&ad, offsets, contextual_len, max_attn_len, ws + l.attn_ws_off,
                       attn_ws_bytes);
  if (rc != HSTU_OK) return rc;
  const int64_t H = desc->num_heads, dv = desc->d_v, dqk = desc->d_qk;
  const __bf16* u_view = uvqk;
  const __bf16* v_view = uvqk + H * dv;
  const __bf16* q_view = uvqk + 2 * H * dv;
  const __bf16* k_view = uvqk + 2 * H * dv + H * dqk;
  rc = check_run_args(&ad, q_view, k_view, v_view, u_view, timestamps, alpha, n_scale,
                      pos_table, time_table, attn);
  if (rc != HSTU_OK) return rc;
  if (desc->num_seqs == 0 || desc->total_tokens == 0) return HSTU_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int N = desc->total_tokens, D = desc->hidden;

  hipError_t e = hstu::launch_layernorm_rows(static_cast<const __bf16*>(x), D, xn, D, N, D,
                                             desc->ln_eps, st);
  if (e != hipSuccess) return fail(HSTU_ERR_HIP, "LayerNorm launch failed: %s", hipGetErrorString(e));
  hstu::GemmArgs g1;
  g1.A = xn;
  g1.B = static_cast<const __bf16*>(w_uvqk);
  g1.bias = static_cast<const __bf16*>(b_uvqk);
  g1.residual = nullptr;
  g1.C = uvqk;
  g1.lda = D;
  g1.ldb = D;
  g1.ldc = l.uvqk_w;
  g1.ldr = 0;
  g1.M = N;
  g1.N = (int32_t)l.uvqk_w;
  g1.K = D;
  g1.act_silu = 1;
  e = hstu::launch_gemm_bt(g1, st);
  if (e != hipSuccess) return fail(HSTU_ERR_HIP, "projection launch failed: %s", hipGetErrorString(e));
  rc = hstu_jagged_attn_fwd(&ad, q_view, k_view, v_view, u_view, offsets, timestamps, num_targets,
                            contextual_len, max_attn_len, alpha, n_scale, pos_table, time_table,
                            attn, ws + l.attn_ws_off, attn_ws_bytes, stream);
  if (rc != HSTU_OK) return rc;
  hstu::GemmArgs g2;
  g2.A = attn;
  g2.B = static_cast<const __bf16*>(w_o);
  g2.bias = nullptr;
  g2.residual = static_cast<const __bf16*>(x);
  g2.C = static_cast<__bf16*>(y);
  g2.lda = H * dv;
  g2.ldb = H * dv;
  g2.ldc = D;
  g2.ldr = D;
  g2.M = N;
  g2.N = D;
  g2.K = (int32_t)(H * dv);
  g2.act_silu = 0;
  e = hstu::launch_gemm_bt(g2, st);
  if (e != hipSuccess) return fail(HSTU_ERR_HIP, "output projection launch failed: %s", hipGetErrorString(e));
  return HSTU_OK;
}

}  // extern "C"


// ---- backward ---------------------------------------------------------------

namespace {

// The backward's value gradient dV_j = sum_i a_ij dO_i is the forward with
// the roles of queries and keys exchanged; for bf16 d = 128 with the plain
// position bias it runs as the sixteen-row forward's transposed walk (k rows
// as the tile, q and dO rows streamed, epilogue none) instead of a pass of
// its own.  `ld_do`: token stride of dO.
bool bwd_tr_dv(const hstu_attn_desc* d) {
  return d->dtype == HSTU_DTYPE_BF16 && d->d_qk == 128 && d->d_v == 128 &&
         !(d->pos_clamp != 0 && d->pos_table_len > 0);
}
hstu_attn_desc tr_dv_desc(const hstu_attn_desc* d, int64_t ld_do) {
  hstu_attn_desc t = *d;
  t.ld_q = d->ld_k;
  t.ld_k = d->ld_q;
  t.ld_v = ld_do;
  t.ld_u = ld_do;   // unused (epilogue none)
  t.ld_out = d->ld_v;
  t.epilogue = HSTU_EPILOGUE_NONE;
  t.pos_clamp = 0;
  return t;
}

struct BwdLayout {
  size_t o_off, do_off, hdr_off, gstart_off, lq_off, lkv_off, part_off, part2_off, total;
  bool gate;    // the LayerNorm * U gate: o recomputed (or saved), dO from the gate kernel
  bool tr_dv;   // dV by the forward's transposed walk
};

BwdLayout bwd_layout(const hstu_attn_desc* d) {
  BwdLayout l;
  l.gate = d->epilogue != HSTU_EPILOGUE_NONE;
  l.tr_dv = bwd_tr_dv(d);
  const int64_t N = d->total_tokens, H = d->num_heads;
  const size_t es = elem_size(d->dtype);
  const size_t rows = (size_t)(N * H * d->d_v) * es;
  const int64_t G = hstu::bwd_groups_max(d->num_seqs, N);
  // the forward's workspace: the recompute of o (gate) and the transposed dV walk
  size_t off = 0;
  if (l.gate) off = fwd_layout(d).total;
  if (l.tr_dv) {
    const hstu_attn_desc t = tr_dv_desc(d, H * d->d_v);
    off = std::max(off, fwd_layout(&t).total);
  }
  l.o_off = hstu::align256(off);
  off = l.o_off + (l.gate ? rows : 0);
  l.do_off = hstu::align256(off);
  off = l.do_off + (l.gate ? rows : 0);
  l.hdr_off = hstu::align256(off);
  off = l.hdr_off + 256;
  l.gstart_off = hstu::align256(off);
  off = l.gstart_off + sizeof(int32_t) * (size_t)(d->num_seqs + 1);
  l.lq_off = hstu::align256(off);
  off = l.lq_off + sizeof(int2) * (size_t)(G > 0 ? G : 1);
  l.lkv_off = hstu::align256(off);
  off = l.lkv_off + sizeof(int2) * (size_t)(G > 0 ? G : 1);
  l.part_off = hstu::align256(off);
  const bool tables = d->pos_table_len > 0 || d->time_table_len > 0;
  const size_t stride = (size_t)(d->pos_table_len + 64);
  l.part2_off = l.part_off;
  if (!hstu::bwd_per_token(d->dtype, d->d_qk, d->d_v) && tables) {
    l.part2_off = hstu::align256(l.part_off + sizeof(float) * (size_t)hstu::kMaxGrid * stride);
    off = l.part2_off + sizeof(float) * (size_t)((hstu::kMaxGrid + 63) / 64) * stride;
  } else if (tables) {   // per-token kernels: the fp64 table sums
    off = l.part_off + sizeof(double) * (size_t)(d->pos_table_len + d->time_table_len);
  }
  l.total = hstu::align256(off);
  return l;
}

// Workgroups of a persistent backward pass (cached per device and variant).
int bwd_pass_grid(const hstu_attn_desc* d, int which) {
  struct Entry {
    int dev, d_qk, d_v, pos_len, has_time, clamp, which, grid;
  };
  static thread_local Entry cache[16];
  static thread_local int cache_n = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const int has_time = d->time_table_len > 0 ? 1 : 0;
  const int clamp = d->pos_clamp != 0 && d->pos_table_len > 0 ? 1 : 0;
  for (int e = 0; e < cache_n && e < 16; ++e) {
    const Entry& c = cache[e];
    if (c.dev == dev && c.d_qk == d->d_qk && c.d_v == d->d_v && c.pos_len == d->pos_table_len &&
        c.has_time == has_time && c.clamp == clamp && c.which == which)
      return c.grid;
  }
  const int g = hstu::bwd_grid(d->dtype, d->d_qk, d->d_v, d->pos_table_len, d->time_table_len,
                               which, clamp != 0);
  if (g >= 0)
    cache[cache_n++ % 16] =
        Entry{dev, d->d_qk, d->d_v, d->pos_table_len, has_time, clamp, which, g};
  return g;
}

}  // namespace

extern "C" {

size_t hstu_jagged_attn_bwd_workspace_bytes(const hstu_attn_desc* desc) {
  if (check_desc(desc) != HSTU_OK) return 0;
  return bwd_layout(desc).total;
}

int hstu_jagged_attn_bwd(const hstu_attn_desc* desc, const void* q, const void* k,
                         const void* v, const void* u, const int32_t* offsets,
                         const int64_t* timestamps, const int32_t* num_targets,
                         int32_t contextual_len, int32_t max_attn_len, float alpha,
                         float n_scale, const float* pos_table, const float* time_table,
                         const void* dout, const void* o_saved, void* dq, void* dk, void* dv,
                         void* du, float* dpos_table, float* dtime_table, void* workspace,
                         size_t workspace_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc != HSTU_OK) return rc;
  if (!hstu::bwd_supported(desc->dtype, desc->d_qk, desc->d_v))
    return fail(HSTU_ERR_UNSUPPORTED,
                "the backward is built for d_qk, d_v in {64, 128} and d_qk = d_v = 256 (bf16) "
                "and d_qk == d_v in {8, 64, 128} (fp32), not (%d, %d)",
                desc->d_qk, desc->d_v);
  if (desc->num_seqs > 0 && !offsets) return fail(HSTU_ERR_INVALID_ARG, "offsets is NULL");
  if (contextual_len < 0) return fail(HSTU_ERR_INVALID_ARG, "contextual_len < 0");
  if (max_attn_len < 0) return fail(HSTU_ERR_INVALID_ARG, "max_attn_len < 0");
  const BwdLayout bl = bwd_layout(desc);
  if (!workspace)
    return fail(HSTU_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", bl.total);
  if (workspace_bytes < bl.total)
    return fail(HSTU_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes,
                bl.total);
  if (!aligned16(workspace)) return fail(HSTU_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  if ((dpos_table == nullptr) != (desc->pos_table_len == 0))
    return fail(HSTU_ERR_INVALID_ARG, "dpos_table and pos_table_len disagree");
  if ((dtime_table == nullptr) != (desc->time_table_len == 0))
    return fail(HSTU_ERR_INVALID_ARG, "dtime_table and time_table_len disagree");
  if (o_saved && !aligned16(o_saved))
    return fail(HSTU_ERR_INVALID_ARG, "o_saved is not 16-byte aligned");
  const bool empty = desc->num_seqs == 0 || desc->total_tokens == 0;
  if (!empty) {
    rc = check_run_args(desc, q, k, v, u, timestamps, alpha, n_scale, pos_table, time_table,
                        dout);
    if (rc != HSTU_OK) return rc;
    struct {
      const char* name;
      const void* p;
    } g[] = {{"dq", dq}, {"dk", dk}, {"dv", dv}, {"du", du}};
    for (auto& x : g) {
      if (x.name[1] == 'u' && desc->epilogue == HSTU_EPILOGUE_NONE) continue;
      if (!x.p) return fail(HSTU_ERR_INVALID_ARG, "%s is NULL", x.name);
      if (!aligned16(x.p)) return fail(HSTU_ERR_INVALID_ARG, "%s is not 16-byte aligned", x.name);
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  // matrix-core passes, or the per-token kernels (fp32; bf16 with d = 256)
  const bool pertok = hstu::bwd_per_token(desc->dtype, desc->d_qk, desc->d_v);
  // the table gradients are sums: zero them where no pass writes them whole
  const bool tables = desc->pos_table_len > 0 || desc->time_table_len > 0;
  double* tab64 = reinterpret_cast<double*>(static_cast<char*>(workspace) + bl.part_off);
  if (!empty && pertok && tables) {
    e = hstu::launch_fill_zero(reinterpret_cast<float*>(tab64),
                               2 * (int64_t)(desc->pos_table_len + desc->time_table_len), s);
    if (e != hipSuccess) return fail(HSTU_ERR_HIP, "fill launch failed: %s", hipGetErrorString(e));
  }
  if (empty) {
    if (dpos_table) e = hstu::launch_fill_zero(dpos_table, desc->pos_table_len, s);
    if (e == hipSuccess && dtime_table)
      e = hstu::launch_fill_zero(dtime_table, desc->time_table_len, s);
    if (e != hipSuccess) return fail(HSTU_ERR_HIP, "fill launch failed: %s", hipGetErrorString(e));
  }
  if (empty) return HSTU_OK;

  int n_q = 0, n_kv = 0, n_v = 0;
  if (!pertok) {
    n_q = bwd_pass_grid(desc, 0);
    n_kv = bwd_pass_grid(desc, 1);
    n_v = bwd_pass_grid(desc, 2);
    if (n_q <= 0 || n_kv <= 0 || n_v < 0)
      return fail(HSTU_ERR_HIP, "cannot query the device for the launch size");
  }
  char* ws = static_cast<char*>(workspace);
  const int64_t H = desc->num_heads;
  const void* d_o = dout;
  int64_t ld_do = desc->ld_out;
  if (bl.gate) {
    // the gate needs the raw aggregation o: the one the training forward kept,
    // or the forward again with epilogue none
    hstu_attn_desc fd = *desc;
    fd.epilogue = HSTU_EPILOGUE_NONE;
    fd.ld_out = H * desc->d_v;
    const void* o = o_saved;
    if (!o) {
      void* orec = ws + bl.o_off;
      rc = hstu_jagged_attn_fwd(&fd, q, k, v, nullptr, offsets, timestamps, num_targets,
                                contextual_len, max_attn_len, alpha, n_scale, pos_table,
                                time_table, orec, ws, bl.o_off, stream);
      if (rc != HSTU_OK) return rc;
      o = orec;
    }
    hstu::GateBwdArgs ga;
    ga.o = o;
    ga.u = u;
    ga.dy = dout;
    ga.du = du;
    ga.d_o = ws + bl.do_off;
    ga.ld_o = H * desc->d_v;
    ga.ld_u = desc->ld_u;
    ga.ld_dy = desc->ld_out;
    ga.n_tok = desc->total_tokens;
    const bool all = desc->epilogue == HSTU_EPILOGUE_LN_ALL_U;
    ga.groups = all ? 1 : desc->num_heads;
    ga.width = all ? desc->num_heads * desc->d_v : desc->d_v;
    ga.eps = desc->ln_eps;
    e = hstu::launch_gate_bwd(ga, desc->dtype, s);
    if (e != hipSuccess)
      return fail(HSTU_ERR_HIP, "gate backward launch failed: %s", hipGetErrorString(e));
    d_o = ws + bl.do_off;
    ld_do = H * desc->d_v;
  }

  hstu::BwdArgs ba;
  ba.q = q;
  ba.k = k;
  ba.v = v;
  ba.dout = d_o;
  ba.dq = dq;
  ba.dk = dk;
  ba.dv = dv;
  ba.offsets = offsets;
  ba.timestamps = time_table ? timestamps : nullptr;
  ba.num_targets = num_targets;
  ba.pos_table = pos_table;
  ba.time_table = time_table;
  ba.tab64 = tab64;
  ba.tab_part = reinterpret_cast<float*>(ws + bl.part_off);
  ba.hdr = reinterpret_cast<int32_t*>(ws + bl.hdr_off);
  ba.list = nullptr;
  ba.ld_q = desc->ld_q;
  ba.ld_k = desc->ld_k;
  ba.ld_v = desc->ld_v;
  ba.ld_do = ld_do;
  ba.num_heads = desc->num_heads;
  ba.contextual_len = contextual_len;
  ba.max_attn_len = max_attn_len;
  ba.pos_len = desc->pos_table_len;
  ba.time_len = desc->time_table_len;
  ba.n_tok = desc->total_tokens;
  ba.alpha = alpha;
  ba.inv_scale = (float)(1.0 / (double)n_scale);
  ba.pos_clamp = desc->pos_clamp != 0 && desc->pos_table_len > 0;
  if (pertok) {
    e = hstu::launch_bwd(ba, desc->dtype, desc->d_qk, desc->d_v, 0, desc->num_seqs, s);
    if (e == hipSuccess) e = hstu::launch_bwd(ba, desc->dtype, desc->d_qk, desc->d_v, 1, desc->num_seqs, s);
    if (e == hipSuccess && tables)
      e = hstu::launch_tab64_finish(tab64, dpos_table, dtime_table, desc->pos_table_len,
                                    desc->time_table_len, s);
    if (e != hipSuccess)
      return fail(HSTU_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
    return HSTU_OK;
  }

  hstu::BwdPlanArgs pa;
  pa.offsets = offsets;
  pa.num_targets = num_targets;
  pa.num_seqs = desc->num_seqs;
  pa.contextual_len = contextual_len;
  pa.max_attn_len = max_attn_len;
  pa.hdr = reinterpret_cast<int32_t*>(ws + bl.hdr_off);
  pa.gstart = reinterpret_cast<int32_t*>(ws + bl.gstart_off);
  pa.list_q = reinterpret_cast<int2*>(ws + bl.lq_off);
  pa.list_kv = reinterpret_cast<int2*>(ws + bl.lkv_off);
  e = hstu::launch_bwd_plan(pa, s);
  if (e != hipSuccess)
    return fail(HSTU_ERR_HIP, "backward scheduler launch failed: %s", hipGetErrorString(e));
  ba.list = pa.list_q;
  e = hstu::launch_bwd(ba, desc->dtype, desc->d_qk, desc->d_v, 0, n_q, s);
  if (e != hipSuccess) return fail(HSTU_ERR_HIP, "dQ launch failed: %s", hipGetErrorString(e));
  ba.list = pa.list_kv;
  e = hstu::launch_bwd(ba, desc->dtype, desc->d_qk, desc->d_v, 1, n_kv, s);
  if (e == hipSuccess && n_v > 0 && !bl.tr_dv)
    e = hstu::launch_bwd(ba, desc->dtype, desc->d_qk, desc->d_v, 2, n_v, s);
  if (e != hipSuccess) return fail(HSTU_ERR_HIP, "dK/dV launch failed: %s", hipGetErrorString(e));
  if (desc->pos_table_len > 0 || desc->time_table_len > 0) {
    hstu::TabReduceArgs ra;
    ra.part = ba.tab_part;
    ra.part2 = reinterpret_cast<float*>(ws + bl.part2_off);
    ra.dpos = dpos_table;
    ra.dtime = dtime_table;
    ra.n_part = n_kv;
    ra.stride = desc->pos_table_len + 64;
    ra.pos_len = desc->pos_table_len;
    ra.time_len = desc->time_table_len;
    ra.scale = ba.inv_scale;
    e = hstu::launch_tab_reduce(ra, s);
    if (e != hipSuccess)
      return fail(HSTU_ERR_HIP, "table reduction launch failed: %s", hipGetErrorString(e));
  }
  if (bl.tr_dv) {   // dV: the forward's transposed walk over key tiles
    const hstu_attn_desc td = tr_dv_desc(desc, ld_do);
    rc = plan_impl(&td, offsets, num_targets, contextual_len, max_attn_len, ws, bl.o_off, stream,
                   false, false, true);
    if (rc != HSTU_OK) return rc;
    rc = run_impl(&td, k, q, d_o, nullptr, offsets, timestamps, num_targets, contextual_len,
                  max_attn_len, alpha, n_scale, pos_table, time_table, dv, nullptr, ws, bl.o_off,
                  stream, nullptr, nullptr, false, true);
    if (rc != HSTU_OK) return rc;
  }
  return HSTU_OK;
}

}  // extern "C"
