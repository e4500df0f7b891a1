/*
 * hstu_oracle.c -- plain fp64 CPU oracle for jagged HSTU attention (forward,
 * and its backward further down).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; it exists so that the tests,
 * the smoke check and the benchmark's CPU-baseline leg can compare the HIP
 * path against an obviously correct definition.  It shares no code, header,
 * table or helper with the HIP sources.
 *
 * What it computes, per sequence b, head h and row i of the sequence
 * (definitions from the pages; citations name page title and section):
 *
 *   s_ij = alpha * <q_i, k_j> + pos[min(|i-j|, P-1)]
 *                 + time[min(floor(log2(1 + |t_i - t_j|)), Tt-1)]
 *       The biased score: relative-position and relative-time bias
 *       ("HSTU tensor by tensor: SiLU aggregation, temporal bias and gating",
 *       sections "Relative time adds information content similarity lacks"
 *       and "Similar shape, different aggregation").
 *   a_ij = SiLU(s_ij) / n_scale   for allowed (i,j), and exactly 0 otherwise.
 *       Pointwise SiLU aggregation with no row normalisation (same page,
 *       "SiLU aggregation coefficients are not probabilities" and "Similar
 *       shape, different aggregation"); illegal pairs are zeroed after the
 *       nonlinearity ("Do not copy softmax masking mechanically") -- here they
 *       are simply never evaluated, which is the same value and cannot make NaN.
 *   o_i  = sum_j a_ij v_j
 *   out_i = LayerNorm(o_i) * u_i   (or o_i itself with epilogue NONE)
 * With epilogue LN_ALL_U the LayerNorm runs over the concatenation of all
 * heads' o_i of a token (H * d_v values) instead of each head's d_v values;
 * the gate by u_i is the same.
 *       The norm-then-gate step U_i (.) Norm(sum_j A_ij V_j) of the teaching
 *       equation ("Similar shape, different aggregation"; "Follow the U, V, Q
 *       and K branches").
 *
 * The allowed set combines the four rules the "HSTU-MUSA" page names in
 * "Mathematical Equivalence" (contextual bidirectional prefix, candidate
 * position clamping, target-group masking, max attention length) with the
 * causal indicator 1_{j<=i} of the teaching equation.  Readings taken where the
 * pages are silent:
 *   - L = seq length, T = clamp(num_targets[b], 0, L), n_h = L - T history
 *     tokens, c = clamp(contextual_len, 0, n_h) prefix tokens.
 *   - prefix rows i < c see j < c (bidirectional);
 *     history rows c <= i < n_h see j <= i;
 *     candidate rows i >= n_h see every history token j < n_h, plus j == i.
 *   - window W > 0: additionally p_i - j <= W, where p_i = min(i, n_h) is the
 *     clamped candidate position (candidates all sit at the history end).
 *   - the bias uses the raw |i-j| and |t_i - t_j| (symmetric inside the prefix);
 *     with pos_clamp != 0 the position bias uses |p_i - p_j| instead, p = min(
 *     position, n_h): the candidate clamp of the mask applied to the bias too
 *     (the alternative reading; the backward takes the raw reading only).
 *   - floor(log2(1+dt)) is taken in exact integer arithmetic.
 *   - LayerNorm per (token, head) over d_v, no affine weights, biased
 *     variance, epsilon given by the caller.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_EPILOGUE_LN_U 0
#define ORACLE_EPILOGUE_NONE 1
#define ORACLE_EPILOGUE_LN_ALL_U 2

static int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

/* Geometry of one sequence: length, history length, prefix length. */
typedef struct {
  int64_t L, n_h, c, W;
} seq_geom;

static seq_geom geometry(const int32_t* offsets, const int32_t* num_targets, int b,
                         int contextual_len, int max_attn_len) {
  seq_geom g;
  g.L = (int64_t)offsets[b + 1] - (int64_t)offsets[b];
  int64_t T = num_targets ? clamp64(num_targets[b], 0, g.L) : 0;
  g.n_h = g.L - T;
  g.c = clamp64(contextual_len, 0, g.n_h);
  g.W = max_attn_len;
  return g;
}

/* Whether query row i may aggregate key j (both local to the sequence). */
static int allowed(const seq_geom* g, int64_t i, int64_t j) {
  int ok;
  if (i < g->c) {
    ok = j < g->c;                              /* bidirectional prefix     */
  } else if (i < g->n_h) {
    ok = j <= i;                                /* causal history           */
  } else {
    ok = (j < g->n_h) || (j == i);              /* target group: history+self */
  }
  if (ok && g->W > 0) {
    int64_t p = i < g->n_h ? i : g->n_h;        /* candidate position clamp */
    ok = (p - j) <= g->W;
  }
  return ok;
}

/* floor(log2(x)) for x >= 1 by repeated halving: plain integer arithmetic. */
static int floor_log2_u64(uint64_t x) {
  int b = 0;
  while (x > 1) {
    x >>= 1;
    ++b;
  }
  return b;
}

int hstu_oracle_time_bucket(int64_t t_i, int64_t t_j) {
  uint64_t dt = t_i >= t_j ? (uint64_t)t_i - (uint64_t)t_j : (uint64_t)t_j - (uint64_t)t_i;
  return floor_log2_u64(1u + dt);
}

double hstu_oracle_silu(double x) { return x / (1.0 + exp(-x)); }

int hstu_oracle_allowed(int64_t L, int64_t num_targets, int64_t contextual_len,
                        int64_t max_attn_len, int64_t i, int64_t j) {
  seq_geom g;
  g.L = L;
  g.n_h = L - clamp64(num_targets, 0, L);
  g.c = clamp64(contextual_len, 0, g.n_h);
  g.W = max_attn_len;
  if (i < 0 || j < 0 || i >= L || j >= L) return 0;
  return allowed(&g, i, j);
}

/* Number of allowed (i, j) pairs over the batch, counted one pair at a time. */
int64_t hstu_oracle_count_allowed(int num_seqs, const int32_t* offsets,
                                  const int32_t* num_targets, int contextual_len,
                                  int max_attn_len) {
  int64_t n = 0;
  for (int b = 0; b < num_seqs; ++b) {
    seq_geom g = geometry(offsets, num_targets, b, contextual_len, max_attn_len);
    for (int64_t i = 0; i < g.L; ++i)
      for (int64_t j = 0; j < g.L; ++j) n += allowed(&g, i, j);
  }
  return n;
}

typedef struct {
  int b, h;
  int64_t work;
} oracle_item;

static int cmp_item_desc(const void* a, const void* b) {
  const oracle_item* x = (const oracle_item*)a;
  const oracle_item* y = (const oracle_item*)b;
  if (x->work != y->work) return x->work < y->work ? 1 : -1;
  if (x->b != y->b) return x->b - y->b;
  return x->h - y->h;
}

/*
 * Full forward.  Tensors are [total_tokens, H, d] with a token stride `ld_*`
 * (in elements) and head stride d.  All floating inputs are fp64 copies of the
 * exact values the device sees.  If row_select is not NULL, only tokens t with
 * row_select[t] != 0 are computed (other output rows are left untouched).
 * Returns 0, or -1 on a bad argument.
 */
int hstu_oracle_fwd(int num_seqs, const int32_t* offsets, int num_heads, int d_qk, int d_v,
                    const double* q, int64_t ld_q, const double* k, int64_t ld_k,
                    const double* v, int64_t ld_v, const double* u, int64_t ld_u,
                    const int64_t* timestamps, const int32_t* num_targets,
                    int contextual_len, int max_attn_len, double alpha, double n_scale,
                    const double* pos_table, int pos_len, const double* time_table,
                    int time_len, double eps, int epilogue, double* out, int64_t ld_out,
                    const unsigned char* row_select, int nthreads, int pos_clamp) {
  if (num_seqs < 0 || num_heads <= 0 || d_qk <= 0 || d_v <= 0) return -1;
  if ((pos_table == NULL) != (pos_len == 0) || (time_table == NULL) != (time_len == 0)) return -1;
  if (time_table && !timestamps) return -1;
  if (!(n_scale > 0.0)) return -1;
  int n_items = num_seqs * num_heads;
  oracle_item* items = (oracle_item*)malloc(sizeof(oracle_item) * (size_t)(n_items > 0 ? n_items : 1));
  if (!items) return -1;
  for (int b = 0; b < num_seqs; ++b) {
    int64_t L = (int64_t)offsets[b + 1] - (int64_t)offsets[b];
    for (int h = 0; h < num_heads; ++h) {
      items[b * num_heads + h].b = b;
      items[b * num_heads + h].h = h;
      items[b * num_heads + h].work = L * L;
    }
  }
  qsort(items, (size_t)n_items, sizeof(oracle_item), cmp_item_desc);
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif

#pragma omp parallel
  {
    double* o = (double*)malloc(sizeof(double) * (size_t)d_v);
#pragma omp for schedule(dynamic, 1)
    for (int it = 0; it < n_items; ++it) {
      int b = items[it].b, h = items[it].h;
      seq_geom g = geometry(offsets, num_targets, b, contextual_len, max_attn_len);
      int64_t base = offsets[b];
      for (int64_t i = 0; i < g.L; ++i) {
        if (row_select && !row_select[base + i]) continue;
        const double* qi = q + (base + i) * ld_q + (int64_t)h * d_qk;
        for (int e = 0; e < d_v; ++e) o[e] = 0.0;
        for (int64_t j = 0; j < g.L; ++j) {
          if (!allowed(&g, i, j)) continue;
          const double* kj = k + (base + j) * ld_k + (int64_t)h * d_qk;
          double dot = 0.0;
          for (int e = 0; e < d_qk; ++e) dot += qi[e] * kj[e];
          double s = alpha * dot;
          if (pos_table) {
            /* pos_clamp: positions taken as p = min(position, n_h), the
               candidate clamp applied to the bias as well */
            int64_t pi = pos_clamp && i > g.n_h ? g.n_h : i;
            int64_t pj = pos_clamp && j > g.n_h ? g.n_h : j;
            int64_t rel = pi >= pj ? pi - pj : pj - pi;
            s += pos_table[rel < pos_len - 1 ? rel : pos_len - 1];
          }
          if (time_table) {
            int bucket = hstu_oracle_time_bucket(timestamps[base + i], timestamps[base + j]);
            s += time_table[bucket < time_len - 1 ? bucket : time_len - 1];
          }
          double a = hstu_oracle_silu(s) / n_scale;
          const double* vj = v + (base + j) * ld_v + (int64_t)h * d_v;
          for (int e = 0; e < d_v; ++e) o[e] += a * vj[e];
        }
        double* dst = out + (base + i) * ld_out + (int64_t)h * d_v;
        if (epilogue == ORACLE_EPILOGUE_NONE || epilogue == ORACLE_EPILOGUE_LN_ALL_U) {
          for (int e = 0; e < d_v; ++e) dst[e] = o[e];
        } else {
          double mean = 0.0;
          for (int e = 0; e < d_v; ++e) mean += o[e];
          mean /= d_v;
          double var = 0.0;
          for (int e = 0; e < d_v; ++e) var += (o[e] - mean) * (o[e] - mean);
          var /= d_v;
          double rstd = 1.0 / sqrt(var + eps);
          const double* ui = u + (base + i) * ld_u + (int64_t)h * d_v;
          for (int e = 0; e < d_v; ++e) dst[e] = (o[e] - mean) * rstd * ui[e];
        }
      }
    }
    free(o);
  }
  free(items);
  if (epilogue == ORACLE_EPILOGUE_LN_ALL_U) {
    /* second pass: each token's H * d_v raw outputs, normalised together */
    int64_t n_tok = num_seqs > 0 ? (int64_t)offsets[num_seqs] : 0;
    int64_t width = (int64_t)num_heads * d_v;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_tok; ++t) {
      if (row_select && !row_select[t]) continue;
      double* row = out + t * ld_out;   /* heads are consecutive d_v blocks */
      double mean = 0.0;
      for (int64_t e = 0; e < width; ++e) mean += row[e];
      mean /= (double)width;
      double var = 0.0;
      for (int64_t e = 0; e < width; ++e) var += (row[e] - mean) * (row[e] - mean);
      var /= (double)width;
      double rstd = 1.0 / sqrt(var + eps);
      for (int h = 0; h < num_heads; ++h) {
        const double* ui = u + t * ld_u + (int64_t)h * d_v;
        for (int e = 0; e < d_v; ++e) {
          double* x = row + (int64_t)h * d_v + e;
          *x = (*x - mean) * rstd * ui[e];
        }
      }
    }
  }
  return 0;
}

/*
 * Backward of hstu_oracle_fwd (the same arguments, plus dout = dLoss/dout):
 * the gradients of a scalar loss with respect to q, k, v, u and both bias
 * tables, by the chain rule taken through the forward's steps in reverse.
 * Training needs them ("Scaling HSTU: ragged execution, candidate
 * amortization and content features", where the model is trained end to
 * end); the pages give no backward, so every step below is the derivative of
 * the forward step named beside it.
 *
 *   gate  out_i = xhat_i * u_i, xhat_i = (o_i - mean) * rstd  (no affine):
 *         du_i = dout_i * xhat_i;  g = dout_i * u_i;
 *         do_i = rstd * (g - mean(g) - xhat_i * mean(g * xhat_i))
 *         (means over the d_v values of the head, or over all H * d_v values
 *         of the token for LN_ALL_U; epilogue NONE: do_i = dout_i, du_i = 0)
 *   sum   o_i = sum_j a_ij v_j:      dv_j += a_ij do_i;  da_ij = <do_i, v_j>
 *   gate  a_ij = SiLU(s_ij)/n_scale on allowed pairs (0 elsewhere):
 *         ds_ij = da_ij * SiLU'(s_ij) / n_scale,
 *         SiLU'(s) = sig(s) * (1 + s * (1 - sig(s))), sig(s) = 1/(1 + e^-s)
 *   score s_ij = alpha <q_i, k_j> + pos[..] + time[..]:
 *         dq_i += alpha ds_ij k_j;  dk_j += alpha ds_ij q_i;
 *         dpos[min(|i-j|, P-1)] += ds_ij;  dtime[bucket_ij] += ds_ij
 *
 * dq, dk, dv, du use the token strides of q, k, v, u; dout uses ld_out.  All
 * outputs are overwritten (every token row, whole tables).  dpos / dtime may
 * be NULL only when the matching table is.  Returns 0, or -1 on a bad
 * argument or allocation failure.
 */
int hstu_oracle_bwd(int num_seqs, const int32_t* offsets, int num_heads, int d_qk, int d_v,
                    const double* q, int64_t ld_q, const double* k, int64_t ld_k,
                    const double* v, int64_t ld_v, const double* u, int64_t ld_u,
                    const int64_t* timestamps, const int32_t* num_targets,
                    int contextual_len, int max_attn_len, double alpha, double n_scale,
                    const double* pos_table, int pos_len, const double* time_table,
                    int time_len, double eps, int epilogue, const double* dout,
                    int64_t ld_out, double* dq, double* dk, double* dv, double* du,
                    double* dpos, double* dtime, int nthreads, int pos_clamp) {
  if (num_seqs < 0 || num_heads <= 0 || d_qk <= 0 || d_v <= 0) return -1;
  if ((pos_table != NULL && dpos == NULL) || (time_table != NULL && dtime == NULL)) return -1;
  int64_t n_tok = num_seqs > 0 ? (int64_t)offsets[num_seqs] : 0;
  int64_t width = (int64_t)num_heads * d_v;
  for (int64_t t = 0; t < n_tok; ++t) {
    for (int64_t e = 0; e < (int64_t)num_heads * d_qk; ++e) {
      dq[t * ld_q + e] = 0.0;
      dk[t * ld_k + e] = 0.0;
    }
    for (int64_t e = 0; e < width; ++e) {
      dv[t * ld_v + e] = 0.0;
      du[t * ld_u + e] = 0.0;
    }
  }
  if (dpos) memset(dpos, 0, sizeof(double) * (size_t)pos_len);
  if (dtime) memset(dtime, 0, sizeof(double) * (size_t)time_len);
  if (n_tok == 0) return 0;

  /* forward again, stopping before the gate: o_i for every token and head */
  double* o = (double*)malloc(sizeof(double) * (size_t)(n_tok * width));
  double* dO = (double*)malloc(sizeof(double) * (size_t)(n_tok * width));
  if (!o || !dO) {
    free(o);
    free(dO);
    return -1;
  }
  int rc = hstu_oracle_fwd(num_seqs, offsets, num_heads, d_qk, d_v, q, ld_q, k, ld_k, v, ld_v,
                           u, ld_u, timestamps, num_targets, contextual_len, max_attn_len,
                           alpha, n_scale, pos_table, pos_len, time_table, time_len, eps,
                           ORACLE_EPILOGUE_NONE, o, width, NULL, nthreads, pos_clamp);
  if (rc != 0) {
    free(o);
    free(dO);
    return rc;
  }

  /* gate backward: groups of `gw` consecutive values normalised together */
  int64_t gw = epilogue == ORACLE_EPILOGUE_LN_ALL_U ? width : d_v;
  int64_t groups_per_tok = width / gw;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n_tok; ++t) {
    for (int64_t gi = 0; gi < groups_per_tok; ++gi) {
      const double* x = o + t * width + gi * gw;
      const double* dy = dout + t * ld_out + gi * gw;
      const double* ug = u + t * ld_u + gi * gw;
      double* dx = dO + t * width + gi * gw;
      double* dug = du + t * ld_u + gi * gw;
      if (epilogue == ORACLE_EPILOGUE_NONE) {
        for (int64_t e = 0; e < gw; ++e) dx[e] = dy[e];
        continue;
      }
      double mean = 0.0, var = 0.0;
      for (int64_t e = 0; e < gw; ++e) mean += x[e];
      mean /= (double)gw;
      for (int64_t e = 0; e < gw; ++e) var += (x[e] - mean) * (x[e] - mean);
      var /= (double)gw;
      double rstd = 1.0 / sqrt(var + eps);
      double mg = 0.0, mgx = 0.0;
      for (int64_t e = 0; e < gw; ++e) {
        double xh = (x[e] - mean) * rstd;
        double g = dy[e] * ug[e];
        dug[e] = dy[e] * xh;
        mg += g;
        mgx += g * xh;
      }
      mg /= (double)gw;
      mgx /= (double)gw;
      for (int64_t e = 0; e < gw; ++e) {
        double xh = (x[e] - mean) * rstd;
        dx[e] = rstd * (dy[e] * ug[e] - mg - xh * mgx);
      }
    }
  }

  /* pair pass: one (sequence, head) at a time; table gradients per thread */
  int n_items = num_seqs * num_heads;
  int nt = 1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
  nt = omp_get_max_threads();
#else
  (void)nthreads;
#endif
  size_t tab = (size_t)pos_len + (size_t)time_len;
  double* part = (double*)calloc((size_t)nt * (tab > 0 ? tab : 1), sizeof(double));
  if (!part) {
    free(o);
    free(dO);
    return -1;
  }
#pragma omp parallel
  {
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
    double* tp = part + (size_t)tid * (tab > 0 ? tab : 1);
#pragma omp for schedule(dynamic, 1)
    for (int it = 0; it < n_items; ++it) {
      int b = it / num_heads, h = it % num_heads;
      seq_geom g = geometry(offsets, num_targets, b, contextual_len, max_attn_len);
      int64_t base = offsets[b];
      for (int64_t i = 0; i < g.L; ++i) {
        const double* qi = q + (base + i) * ld_q + (int64_t)h * d_qk;
        const double* doi = dO + (base + i) * width + (int64_t)h * d_v;
        double* dqi = dq + (base + i) * ld_q + (int64_t)h * d_qk;
        for (int64_t j = 0; j < g.L; ++j) {
          if (!allowed(&g, i, j)) continue;
          const double* kj = k + (base + j) * ld_k + (int64_t)h * d_qk;
          const double* vj = v + (base + j) * ld_v + (int64_t)h * d_v;
          double dot = 0.0;
          for (int e = 0; e < d_qk; ++e) dot += qi[e] * kj[e];
          double s = alpha * dot;
          int64_t pidx = 0;
          int bidx = 0;
          if (pos_table) {
            /* the forward's position index: |i - j|, or with pos_clamp the
               distance of the clamped positions min(position, n_h) */
            int64_t pi = pos_clamp && i > g.n_h ? g.n_h : i;
            int64_t pj = pos_clamp && j > g.n_h ? g.n_h : j;
            int64_t rel = pi >= pj ? pi - pj : pj - pi;
            pidx = rel < pos_len - 1 ? rel : pos_len - 1;
            s += pos_table[pidx];
          }
          if (time_table) {
            int bucket = hstu_oracle_time_bucket(timestamps[base + i], timestamps[base + j]);
            bidx = bucket < time_len - 1 ? bucket : time_len - 1;
            s += time_table[bidx];
          }
          double sig = 1.0 / (1.0 + exp(-s));
          double a = s * sig / n_scale;
          double da = 0.0;
          for (int e = 0; e < d_v; ++e) da += doi[e] * vj[e];
          double ds = da * sig * (1.0 + s * (1.0 - sig)) / n_scale;
          double* dvj = dv + (base + j) * ld_v + (int64_t)h * d_v;
          for (int e = 0; e < d_v; ++e) dvj[e] += a * doi[e];
          double* dkj = dk + (base + j) * ld_k + (int64_t)h * d_qk;
          for (int e = 0; e < d_qk; ++e) {
            dqi[e] += alpha * ds * kj[e];
            dkj[e] += alpha * ds * qi[e];
          }
          if (pos_table) tp[pidx] += ds;
          if (time_table) tp[pos_len + bidx] += ds;
        }
      }
    }
  }
  for (int t = 0; t < nt; ++t) {
    const double* tp = part + (size_t)t * (tab > 0 ? tab : 1);
    for (int e = 0; e < pos_len; ++e) dpos[e] += tp[e];
    for (int e = 0; e < time_len; ++e) dtime[e] += tp[pos_len + e];
  }
  free(part);
  free(o);
  free(dO);
  return 0;
}

int hstu_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
