/*
 * hstu_attn.h -- C ABI of the MI355X (gfx950) jagged HSTU attention library.
 *
 * Operation (forward; its backward is declared near the end).  Sequences
 * are stored jagged: the tokens of all sequences are concatenated and an
 * int32 offsets array marks where each sequence starts ("Scaling HSTU: ragged execution, candidate amortization and
 * content features", section "Variable length is a central systems issue").
 * For every sequence b, head h and query row i of the sequence:
 *
 *   s_ij  = alpha * <q_i, k_j> + pos_table[min(|i-j|, P-1)]
 *                 + time_table[min(floor(log2(1 + |t_i - t_j|)), Tt-1)]
 *   a_ij  = SiLU(s_ij) / n_scale  if (i, j) is allowed, else exactly 0
 *   o_i   = sum_j a_ij * v_j
 *   out_i = LayerNorm(o_i) * u_i        (HSTU_EPILOGUE_LN_U)
 *         = o_i                         (HSTU_EPILOGUE_NONE)
 *         = LayerNorm over all heads of the token, * u_i   (HSTU_EPILOGUE_LN_ALL_U)
 *
 * This is the pointwise SiLU aggregation with relative position / time bias
 * and the norm-then-U gating of "HSTU tensor by tensor: SiLU aggregation,
 * temporal bias and gating" (sections "SiLU aggregation coefficients are not
 * probabilities", "Relative time adds information content similarity lacks",
 * "Similar shape, different aggregation"); illegal coefficients are zeroed
 * after the nonlinearity (section "Do not copy softmax masking mechanically"),
 * so a masked score that overflows can never turn into NaN.
 *
 * Allowed pairs combine the causal rule with the four rules named on the
 * "HSTU-MUSA" page, section "Mathematical Equivalence".  With L the sequence
 * length, T = clamp(num_targets[b], 0, L) candidates at the end, n_h = L - T
 * history tokens and c = clamp(contextual_len, 0, n_h) prefix tokens:
 *   prefix rows    i <  c        : j < c          (bidirectional)
 *   history rows   c <= i < n_h  : j <= i         (causal)
 *   candidate rows i >= n_h      : j < n_h, or j == i   (target group)
 *   if max_attn_len W > 0, also p_i - j <= W with p_i = min(i, n_h)
 *   (candidate position clamping: every candidate sits at the history end).
 * The bias uses the raw |i-j| and |t_i - t_j|; with desc->pos_clamp = 1 the
 * position bias uses |p_i - p_j| instead, the clamp p = min(position, n_h) of
 * the candidate rule applied to the bias too (so candidates, all at the
 * history end, become interchangeable; "Scaling HSTU", section "Many
 * candidates make reuse valuable"); the backward differentiates either
 * reading.  LayerNorm is taken per (token, head) over d_v, without affine
 * weights, with biased variance and epsilon desc->ln_eps.
 *
 * Memory layout.  q, k: [total_tokens, H, d_qk]; v, u, out: [total_tokens, H,
 * d_v].  Element (t, h, e) of tensor x lives at x + t*ld_x + h*d + e (ld_x in
 * elements, head stride d).  All of q, k, v, u, out share desc->dtype.
 * offsets: int32 [num_seqs+1], offsets[0] = 0, nondecreasing, offsets[num_seqs]
 * = total_tokens.  timestamps: int64 [total_tokens], seconds.  num_targets:
 * int32 [num_seqs].  pos_table, time_table: float32.
 *
 * Ownership and asynchrony.  Every tensor pointer is device memory owned by
 * the caller.  The library allocates no device memory and keeps no pointer
 * after a call returns; scratch space comes from the caller's `workspace`.
 * Calls only enqueue kernels on `stream` (a hipStream_t; NULL = the default
 * stream) and never synchronise: the caller keeps every buffer alive until
 * the stream has passed the call.
 *
 * Errors.  Functions return an hstu_status.  Every condition the host can
 * check (null pointers, sizes, alignment, strides, table lengths, n_scale,
 * workspace size, unsupported shapes) is checked before any HIP call; a
 * failing call enqueues nothing.  A failure sets a thread-local message that
 * hstu_last_error() returns.  Nothing aborts or throws across the ABI.
 * Device data is trusted: non-monotone offsets, offsets[num_seqs] !=
 * total_tokens or non-finite inputs give undefined results (checking them
 * would need a synchronisation).  num_targets[b] and contextual_len are
 * clamped as described above.
 */
#ifndef HSTU_ATTN_H_
#define HSTU_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HSTU_OK = 0,
  HSTU_ERR_INVALID_ARG = -1,  /* null pointer, bad size, stride or alignment     */
  HSTU_ERR_UNSUPPORTED = -2,  /* valid but not built: (dtype, d_qk, d_v) etc.    */
  HSTU_ERR_WORKSPACE = -3,    /* workspace null or smaller than required         */
  HSTU_ERR_HIP = -4           /* a HIP runtime call or kernel launch failed      */
} hstu_status;

typedef enum { HSTU_DTYPE_F32 = 0, HSTU_DTYPE_BF16 = 1 } hstu_dtype;

/*
 * HSTU_EPILOGUE_LN_ALL_U: the same gate with one LayerNorm over all H * d_v
 * values of a token (all heads together) instead of one per (token, head);
 * the attention writes O / n_scale and a second pass normalises each token in
 * place (for bf16 the raw outputs are rounded to bf16 in between).  Requires
 * H * d_v <= 4096 (bf16) or 2048 (fp32).
 */
typedef enum {
  HSTU_EPILOGUE_LN_U = 0,
  HSTU_EPILOGUE_NONE = 1,
  HSTU_EPILOGUE_LN_ALL_U = 2
} hstu_epilogue;

/* Shapes, element type and strides of one call. */
typedef struct {
  int32_t num_seqs;       /* B >= 0                                               */
  int32_t total_tokens;   /* N >= 0, equals offsets[B] on the device              */
  int32_t num_heads;      /* H >= 1                                               */
  int32_t d_qk;           /* head dim of q and k                                  */
  int32_t d_v;            /* head dim of v, u and out                             */
  int32_t dtype;          /* hstu_dtype of q, k, v, u, out                        */
  int64_t ld_q, ld_k, ld_v, ld_u, ld_out;  /* token strides in elements           */
  int32_t pos_table_len;  /* P; 0 iff pos_table is NULL                           */
  int32_t time_table_len; /* Tt; 0 iff time_table is NULL (then no timestamps)    */
  float ln_eps;           /* LayerNorm epsilon (> 0 and finite)                   */
  int32_t epilogue;       /* hstu_epilogue                                        */
  int32_t pos_clamp;      /* 0: position bias of |i-j| (default); 1: of |p_i-p_j|  */
                          /* with p = min(position, n_h) (see above)              */
} hstu_attn_desc;

/*
 * Supported (dtype, d_qk, d_v) of the forward: (BF16,128,128), (BF16,64,64),
 * (BF16,64,128), (BF16,128,64), (BF16,256,256), (F32,128,128), (F32,64,64),
 * (F32,8,8); the backward takes every bf16 shape (d = 256 through its
 * per-token kernels) and the fp32 shapes with d_qk == d_v.  (BF16,256,256)
 * runs one workgroup per CU (its 32 x 256 output tile per wave needs the
 * registers of two).  Alignment: q, k, v, u, out 16-byte aligned and
 * ld_x * sizeof(element) a multiple of 16 bytes with ld_x >= H * d; a token
 * row may span at most 16 MiB (ld_x * sizeof(element) <= 2^24), larger
 * strides are refused with HSTU_ERR_UNSUPPORTED.
 * Returns 1 if supported, 0 if not (no message is set).
 */
int hstu_jagged_attn_supported(int32_t dtype, int32_t d_qk, int32_t d_v);

/*
 * Workspace bytes the call needs for `desc`: the scheduler's work list, the
 * arrival counters and the fp32 partial outputs of items split along keys
 * (2 x 1024 slots of 128 x d_v floats, reserved only when total_tokens >=
 * 481, the shortest sequence in which an item can reach the 16 key tiles the
 * scheduler splits).  Depends on num_seqs, total_tokens, num_heads and d_v
 * only (no device query).  Returns 0 and sets the error message if desc is
 * invalid.
 */
size_t hstu_jagged_attn_workspace_bytes(const hstu_attn_desc* desc);

/*
 * The full forward: hstu_jagged_attn_plan followed by hstu_jagged_attn_run on
 * the same stream.  Arguments are as described for those two calls.
 * B == 0 or total_tokens == 0 returns HSTU_OK and enqueues nothing.
 */
int hstu_jagged_attn_fwd(const hstu_attn_desc* desc,
                         const void* q, const void* k, const void* v, const void* u,
                         const int32_t* offsets, const int64_t* timestamps,
                         const int32_t* num_targets, int32_t contextual_len,
                         int32_t max_attn_len, float alpha, float n_scale,
                         const float* pos_table, const float* time_table, void* out,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Scheduler: enqueues one kernel that reads offsets / num_targets on the
 * device, splits every (sequence, head) into query tiles, estimates each tile's
 * work from the mask geometry (number of key tiles it must visit) and writes a
 * work list sorted by decreasing work into `workspace` ("Scaling HSTU",
 * section "Variable length is a central systems issue": kernels must handle
 * boundaries, grouping and balance).  The plan depends only on offsets,
 * num_targets, contextual_len, max_attn_len and the shapes in desc, so it can
 * be reused by several hstu_jagged_attn_run calls (e.g. every layer of a
 * stack sharing one batch).  num_targets may be NULL (no candidates);
 * contextual_len >= 0; max_attn_len >= 0 (0 = unlimited).
 */
int hstu_jagged_attn_plan(const hstu_attn_desc* desc, const int32_t* offsets,
                          const int32_t* num_targets, int32_t contextual_len,
                          int32_t max_attn_len, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Attention: enqueues the attention kernel, which walks the work list that a
 * previous hstu_jagged_attn_plan call on the same stream wrote into
 * `workspace` with the same offsets, num_targets, contextual_len,
 * max_attn_len and shapes.  Requires n_scale > 0 and finite, alpha finite;
 * timestamps non-NULL iff time_table non-NULL.  Writes every row of `out`
 * exactly once and nothing else.  The workspace also holds counters the run
 * uses and leaves rearmed for the next run of the same plan (the work-queue
 * counter of a batch of short sequences, the arrival counters of items split
 * along keys): runs that share a workspace must be ordered (one stream, or
 * synchronised); two at once on one workspace race.
 */
int hstu_jagged_attn_run(const hstu_attn_desc* desc,
                         const void* q, const void* k, const void* v, const void* u,
                         const int32_t* offsets, const int64_t* timestamps,
                         const int32_t* num_targets, int32_t contextual_len,
                         int32_t max_attn_len, float alpha, float n_scale,
                         const float* pos_table, const float* time_table, void* out,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * hstu_jagged_attn_run with the attention kernel's own start and end times
 * taken into two caller-owned HIP events (hipEvent_t, created with timing
 * enabled, passed as void*; either may be NULL): the launch goes through
 * hipExtLaunchKernelGGL, whose events carry the kernel's start and stop
 * timestamps rather than those of markers around it.  A measurement aid:
 * the work and the result are those of hstu_jagged_attn_run.  With the
 * all-heads LayerNorm epilogue the events cover the attention kernel only.
 */
int hstu_jagged_attn_run_timed(const hstu_attn_desc* desc,
                               const void* q, const void* k, const void* v, const void* u,
                               const int32_t* offsets, const int64_t* timestamps,
                               const int32_t* num_targets, int32_t contextual_len,
                               int32_t max_attn_len, float alpha, float n_scale,
                               const float* pos_table, const float* time_table, void* out,
                               void* workspace, size_t workspace_bytes, void* stream,
                               void* start_event, void* stop_event);

/*
 * Candidate rows only (candidate micro-batching with history reuse, "Scaling
 * HSTU: ragged execution, candidate amortization and content features",
 * section "Many candidates make reuse valuable").  The candidates of a
 * sequence attend to its history keys and to themselves only, and with the
 * candidate position clamped to the history end (the mask rules of
 * hstu_attn_desc's header comment) every candidate sees the same history, so
 * a candidate's output depends on the history and on itself, never on the
 * other candidates.  These calls compute exactly the candidate rows
 * [n_h, L) of every sequence, tiled from n_h (128 candidates of a sequence
 * per work item, all reading the same cached history keys and values), and
 * write only those rows of `out`: history rows are not touched, so a history
 * computed once (its K/V, and its rows' outputs from a previous call) can
 * serve any number of candidate micro-batches laid out after it.  Arguments,
 * layouts, ownership and errors are those of hstu_jagged_attn_plan and
 * hstu_jagged_attn_fwd; a candidates-only plan is run with
 * hstu_jagged_attn_run.  Sequences without candidates contribute no work.
 */
int hstu_jagged_attn_plan_candidates(const hstu_attn_desc* desc, const int32_t* offsets,
                                     const int32_t* num_targets, int32_t contextual_len,
                                     int32_t max_attn_len, void* workspace,
                                     size_t workspace_bytes, void* stream);

int hstu_jagged_attn_fwd_candidates(const hstu_attn_desc* desc,
                                    const void* q, const void* k, const void* v, const void* u,
                                    const int32_t* offsets, const int64_t* timestamps,
                                    const int32_t* num_targets, int32_t contextual_len,
                                    int32_t max_attn_len, float alpha, float n_scale,
                                    const float* pos_table, const float* time_table, void* out,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * hstu_jagged_attn_fwd without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The same forward (scheduler +
 * attention, same arguments, errors and tolerance; items are never split
 * along their keys, so the output may differ from hstu_jagged_attn_fwd's in
 * the last bits), with the work list in an 8 MiB array of the library that
 * each GPU it runs on holds from module load until the process ends.  It
 * calls no allocator: the array's device address is looked up once per
 * device on the first call there.  Batches whose work list exceeds the array
 * (about 250,000 work items) return HSTU_ERR_WORKSPACE with a message naming
 * both sizes.  Every call on one GPU uses the same array and each call
 * rewrites all of it that the call reads: calls that overlap on one GPU
 * (other streams, other threads) race; order them.
 */
int hstu_jagged_attn_fwd_noalloc(const hstu_attn_desc* desc,
                                 const void* q, const void* k, const void* v, const void* u,
                                 const int32_t* offsets, const int64_t* timestamps,
                                 const int32_t* num_targets, int32_t contextual_len,
                                 int32_t max_attn_len, float alpha, float n_scale,
                                 const float* pos_table, const float* time_table, void* out,
                                 void* stream);

/*
 * Host helper for throughput accounting: the exact number of allowed (i, j)
 * pairs of the batch, per head, from HOST copies of offsets and num_targets
 * (num_targets may be NULL).  Returns -1 and sets the message on bad input.
 */
int64_t hstu_jagged_attn_valid_pairs(int32_t num_seqs, const int32_t* offsets_host,
                                     const int32_t* num_targets_host,
                                     int32_t contextual_len, int32_t max_attn_len);

/*
 * Launch configuration of the attention kernel for `desc` on the current
 * device: the number of persistent workgroups (CUs x resident workgroups per
 * CU, capped by the work-item bound).  Returns -1 and sets the message on a
 * bad desc or a HIP error.
 */
int hstu_jagged_attn_grid(const hstu_attn_desc* desc);

/*
 * Forward kernel choice.  Four kernels compute the same forward over the
 * same work list and workspace: a four-wave kernel (32 query rows per wave,
 * two workgroups per CU, every supported dtype and head size) and, for bf16
 * with d_qk = d_v = 128, a sixteen-row kernel (16 query rows per wave, eight
 * waves per workgroup, four waves per SIMD), a thirty-two-row kernel (two
 * 16-row groups per wave sharing every K/V operand read, four waves per
 * workgroup, two waves per SIMD) and an eight-wave kernel (one workgroup per
 * CU whose two waves per SIMD alternate between matrix-core and vector
 * work).  AUTO (the default) takes the sixteen-row kernel where it is built
 * and the four-wave kernel elsewhere; the eight-wave and thirty-two-row
 * kernels run only when chosen.  The setting is process-wide; a plan and the
 * runs that use it must see the same setting (the launch size depends on
 * it).  All kernels meet the same tolerance against the oracle; their
 * outputs differ in the last bits (different summation order).
 * hstu_jagged_attn_set_fwd_kernel returns HSTU_OK, or HSTU_ERR_INVALID_ARG
 * for an unknown mode.  hstu_jagged_attn_fwd_kernel_of returns the kernel
 * `desc` would run (FOUR_WAVE, EIGHT_WAVE, SIXTEEN_ROW or THIRTYTWO_ROW), or
 * -1 on a bad desc.  A mode whose kernel does not support `desc` falls back to the
 * four-wave kernel.
 */
enum {
  HSTU_FWD_KERNEL_AUTO = 0,
  HSTU_FWD_KERNEL_FOUR_WAVE = 1,
  HSTU_FWD_KERNEL_EIGHT_WAVE = 2,
  HSTU_FWD_KERNEL_SIXTEEN_ROW = 3,
  HSTU_FWD_KERNEL_THIRTYTWO_ROW = 4
};
int hstu_jagged_attn_set_fwd_kernel(int32_t mode);
int hstu_jagged_attn_fwd_kernel_of(const hstu_attn_desc* desc);

/*
 * Full HSTU layer forward, bf16 (the block of "HSTU tensor by tensor: SiLU
 * aggregation, temporal bias and gating": sections "Follow the U, V, Q and K
 * branches", "Trace four projections" and the teaching equation of "Similar
 * shape, different aggregation", o_i = W_o[U_i * Norm(sum_j A_ij V_j)] + x_i):
 *
 *   xn   = LayerNorm(x)                       per token over `hidden`, no affine
 *   uvqk = SiLU(xn W_uvqk^T + b_uvqk)         one fused projection
 *   U, V, Q, K = column blocks of uvqk        widths H d_v, H d_v, H d_qk, H d_qk
 *   a    = jagged attention with the per-(token, head) LayerNorm * U gate
 *   y    = a W_o^T + x                        output projection, residual
 *
 * x, y: [total_tokens, hidden]; w_uvqk: [H (2 d_v + 2 d_qk), hidden] and
 * b_uvqk: [H (2 d_v + 2 d_qk)]; w_o: [hidden, H d_v] (weights in the [out, in]
 * layout), all bf16, rows contiguous, 16-byte aligned.  The intermediates (xn,
 * uvqk, a) are bf16 in the workspace (hstu_layer_workspace_bytes, which also
 * holds the attention's work list).  Requires hidden % 128 == 0 and <= 4096,
 * H (2 d_v + 2 d_qk) % 128 == 0, H d_v % 64 == 0 and a supported bf16
 * attention shape.  The attention arguments and errors are those of
 * hstu_jagged_attn_fwd; ln_eps serves both LayerNorms.  Enqueues five kernels
 * on `stream` (LayerNorm, projection GEMM, scheduler, attention, output GEMM).
 */
typedef struct {
  int32_t num_seqs;
  int32_t total_tokens;
  int32_t num_heads;
  int32_t d_qk;
  int32_t d_v;
  int32_t hidden;          /* width of x and y                                    */
  int32_t pos_table_len;
  int32_t time_table_len;
  float ln_eps;
} hstu_layer_desc;

size_t hstu_layer_workspace_bytes(const hstu_layer_desc* desc);

int hstu_layer_fwd(const hstu_layer_desc* desc, const void* x, const void* w_uvqk,
                   const void* b_uvqk, const void* w_o, const int32_t* offsets,
                   const int64_t* timestamps, const int32_t* num_targets,
                   int32_t contextual_len, int32_t max_attn_len, float alpha, float n_scale,
                   const float* pos_table, const float* time_table, void* y, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * Backward of the attention (dtype, shapes, strides, rules and epilogue of
 * `desc`, the same inputs as the forward).  Given dout = dLoss/d(out) it
 * writes the gradients of the loss with respect to q, k, v, u and both bias
 * tables, by the chain rule through the forward's steps (the pages give the
 * forward only; training the model end to end, "Scaling HSTU: ragged
 * execution, candidate amortization and content features", needs these):
 *
 *   gate   xhat_i = (o_i - mean) * rstd,  out_i = xhat_i * u_i:
 *          du_i = dout_i * xhat_i,  g = dout_i * u_i,
 *          do_i = rstd * (g - mean(g) - xhat_i * mean(g * xhat_i))
 *          (per (token, head) over d_v, or over all H * d_v values of the
 *          token for LN_ALL_U; epilogue NONE: do_i = dout_i)
 *   da_ij = <do_i, v_j>,  ds_ij = da_ij * SiLU'(s_ij) / n_scale on allowed
 *          pairs (0 elsewhere), SiLU'(x) = sig(x) (1 + x (1 - sig(x)))
 *   dq_i = alpha sum_j ds_ij k_j,  dk_j = alpha sum_i ds_ij q_i,
 *   dv_j = sum_i a_ij do_i,
 *   dpos_table[min(|i-j|, P-1)] += ds_ij,  dtime_table[bucket_ij] += ds_ij.
 *
 * Layouts: dq, dk, dv, du have the layouts (token strides ld_q, ld_k, ld_v,
 * ld_u) and dtype of q, k, v, u; dout has those of out (ld_out).
 * dpos_table / dtime_table: float32 [P] / [Tt], NULL exactly when the table
 * is.  Every token row of dq, dk, dv (and du unless the epilogue is NONE, in
 * which case du may be NULL and is not touched) and both tables are
 * overwritten.  The raw aggregation o that the gate needs is o_saved when
 * given, else recomputed (one forward pass with epilogue NONE, rounded to
 * dtype) inside the call.
 *
 * Shapes: d_qk, d_v in {64, 128} for bf16 (equal or not), d_qk = d_v = 256
 * for bf16, and d_qk == d_v in {8, 64, 128} for fp32; other head sizes
 * return HSTU_ERR_UNSUPPORTED before any HIP call.
 *
 * Execution: for bf16 with d = 64, 128 a scheduler kernel, then a dQ pass
 * over query tiles and a dK/dV pass over key tiles (bf16 MFMA, fp32
 * accumulation; each token gradient written by one workgroup, so those are
 * deterministic) and a reduction of the table gradients (fp32 sums whose
 * order depends on the schedule only through LDS atomics within a
 * workgroup); for d_qk = d_v = 128 without the clamped-position bias, dV is
 * the forward's sixteen-row kernel walking key tiles (dV_j = sum_i a_ij dO_i
 * is the forward with queries and keys exchanged), planned by the forward's
 * scheduler in the same workspace.  For fp32, and for bf16 with d = 256, two per-token kernels
 * (one wave per token and head, fp32 arithmetic, bf16 or fp32 loads and
 * stores) with fp64 atomics on the table sums, rounded to fp32 at the end:
 * a correctness path, far slower than the matrix-core passes.  Ownership, streams, error
 * behaviour and trusted device data as for the forward.  Workspace:
 * hstu_jagged_attn_bwd_workspace_bytes(desc) bytes, 16-byte aligned; B == 0
 * or total_tokens == 0 only zeroes the tables.
 */
size_t hstu_jagged_attn_bwd_workspace_bytes(const hstu_attn_desc* desc);

/*
 * o_saved: NULL, or the raw aggregation o / n_scale ([total_tokens, H, d_v],
 * token stride H * d_v, dtype of desc) that hstu_jagged_attn_fwd_train wrote
 * for these inputs; then the backward skips its forward recompute.
 */
int hstu_jagged_attn_bwd(const hstu_attn_desc* desc,
                         const void* q, const void* k, const void* v, const void* u,
                         const int32_t* offsets, const int64_t* timestamps,
                         const int32_t* num_targets, int32_t contextual_len,
                         int32_t max_attn_len, float alpha, float n_scale,
                         const float* pos_table, const float* time_table,
                         const void* dout, const void* o_saved,
                         void* dq, void* dk, void* dv, void* du,
                         float* dpos_table, float* dtime_table,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * The forward for training: hstu_jagged_attn_fwd (same arguments, same `out`)
 * that also writes o_raw = o / n_scale, the aggregation before the gate
 * ([total_tokens, H, d_v], token stride H * d_v, dtype of desc; 16-byte
 * aligned, caller-owned), which hstu_jagged_attn_bwd can take as o_saved
 * instead of recomputing it.  Costs one more write of that tensor.
 */
int hstu_jagged_attn_fwd_train(const hstu_attn_desc* desc,
                               const void* q, const void* k, const void* v, const void* u,
                               const int32_t* offsets, const int64_t* timestamps,
                               const int32_t* num_targets, int32_t contextual_len,
                               int32_t max_attn_len, float alpha, float n_scale,
                               const float* pos_table, const float* time_table, void* out,
                               void* o_raw, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Thread-local message for the last failing call of this thread ("" if none). */
const char* hstu_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_ATTN_H_ */
