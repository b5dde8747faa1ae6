/*
 * gdn_oracle.c -- plain, slow, fp64 CPU oracle for the Gated DeltaNet mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file: only tests/, the smoke check in __graft_entry__ and the
 * cpu_baseline leg of bench.py use it.  It shares no code, header, table or
 * helper with the HIP library (libgdn); the two meet only through buffers of
 * inputs drawn by the seeded generators.
 *
 * Sources (the pages this follows):
 *   [HYB]  "L'attention hybride" (Qwen3.8-27B architecture chapter):
 *          section "La recurrence" -- per value head a 128x128 fp32 state,
 *          alpha_t fades the whole state, beta_t rewrites the association of
 *          k_t, I is the 128x128 identity (the update formula itself is lost
 *          from the page text; the standard gated delta rule is taken, see
 *          below); section "La dissymetrie 16 / 48" -- one key head serves
 *          several value heads; section "Le float32 n'est pas un detail" --
 *          the state is float32 while the rest is BF16; table "Le decompte"
 *          -- causal conv with kernel 4 over the q,k,v channels, no bias,
 *          and a 128-weight output normalisation; config block "Les 48
 *          couches Gated DeltaNet" -- output_gate_type swish.
 *   [BRI]  "Les briques d'un reseau de neurones" (Kimi K3 foundations):
 *          section 2 table (sigmoid, Swish/SiLU = x*sigmoid(x), softplus) and
 *          section 4 (RMSNorm with a small epsilon against division by zero
 *          and a learned per-coordinate gain).
 *
 * Everything is computed in double precision, token by token, exactly as the
 * definitions read, with no blocking, chunking or reordering.  Inputs may be
 * given as fp64, fp32 or bf16 bit patterns; they are widened exactly.
 *
 * Recurrence (per batch b and value head h, key head h / (Hv/Hk)):
 *     S_t = a_t * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t                         (read after the update)
 * with a_t = exp(log_alpha_t).  The state is stored as M = S^T, a
 * [Dk][Dv] row-major matrix (the pages give the state as d_k x d_v).  With
 * M the update is the rank-one form
 *     u = M^T k ;  M <- a M + k (beta (v - a u))^T ;  o = M^T q
 * which is algebraically the same expression (expand S(I - b k k^T)).
 * Each column j of M (value coordinate j) evolves on its own, so the work
 * is split across threads by (head, column block) -- a partition of the
 * arithmetic, not a change of it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F64 = 0, OR_F32 = 1, OR_BF16 = 2 };

static double ld(const void* p, int dt, int64_t i) {
  if (dt == OR_F64) return ((const double*)p)[i];
  if (dt == OR_F32) return (double)((const float*)p)[i];
  uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Shapes and options of one recurrence call.  Strides are in elements
 * between consecutive tokens; heads are packed inside a token; the batch
 * stride is T * stride.  Gates are [B][T][Hv] contiguous.  The state is
 * [B][Hv][Dk][Dv] contiguous. */
typedef struct {
  int64_t B, T, Hk, Hv, Dk, Dv;
  int64_t stride_q, stride_k, stride_v;
  int32_t q_dtype, k_dtype, v_dtype, gate_dtype, state_dtype;
  int32_t l2norm; /* 1: q and k are divided by sqrt(sum of squares + l2_eps) */
  double q_scale, l2_eps;
} gdn_oracle_dims;

int gdn_oracle_abi_version(void) { return 2; }

/* Per-token L2 normalisation of one head vector: x / sqrt(sum x^2 + eps). */
static void l2_normalise(double* x, int64_t n, double eps) {
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s += x[i] * x[i];
  double r = 1.0 / sqrt(s + eps);
  for (int64_t i = 0; i < n; ++i) x[i] *= r;
}

/*
 * Runs the recurrence for the selected (b, h) pairs (sel[i] = b*Hv + h; NULL
 * means every pair) over all T tokens.
 *   o_out     : [n_sel][T][Dv] doubles, or NULL
 *   state_out : [n_sel][Dk][Dv] doubles, or NULL
 * Returns 0, or -1 on a bad argument.
 */
int gdn_oracle_recurrence(const gdn_oracle_dims* d, const void* q, const void* k,
                          const void* v, const void* log_alpha, const void* beta,
                          const void* state_in, int64_t n_sel, const int64_t* sel,
                          double* o_out, double* state_out, int32_t n_threads) {
  if (!d || !q || !k || !v || !log_alpha || !beta) return -1;
  if (d->Hk <= 0 || d->Hv <= 0 || d->Hv % d->Hk != 0 || d->Dk <= 0 || d->Dv <= 0 ||
      d->T < 0 || d->B <= 0)
    return -1;
  const int64_t B = d->B, T = d->T, Hv = d->Hv, Dk = d->Dk, Dv = d->Dv;
  const int64_t G = d->Hv / d->Hk;
  if (!sel) n_sel = B * Hv;
  const int64_t CB = 16; /* value columns per task */
  const int64_t nblk = (Dv + CB - 1) / CB;
  const int64_t ntask = n_sel * nblk;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t task = 0; task < ntask; ++task) {
    const int64_t si = task / nblk, blk = task % nblk;
    const int64_t bh = sel ? sel[si] : si;
    const int64_t b = bh / Hv, h = bh % Hv, hk = h / G;
    const int64_t j0 = blk * CB, nj = (Dv - j0 < CB) ? (Dv - j0) : CB;
    double* M = (double*)calloc((size_t)(Dk * nj), sizeof(double)); /* M[i][jj] */
    double* qv = (double*)malloc(sizeof(double) * (size_t)Dk);
    double* kv = (double*)malloc(sizeof(double) * (size_t)Dk);
    double u[16], vv[16];
    if (state_in) {
      for (int64_t i = 0; i < Dk; ++i)
        for (int64_t jj = 0; jj < nj; ++jj)
          M[i * nj + jj] = ld(state_in, d->state_dtype, ((b * Hv + h) * Dk + i) * Dv + j0 + jj);
    }
    for (int64_t t = 0; t < T; ++t) {
      const int64_t tok = b * T + t;
      for (int64_t i = 0; i < Dk; ++i) {
        qv[i] = ld(q, d->q_dtype, tok * d->stride_q + hk * Dk + i);
        kv[i] = ld(k, d->k_dtype, tok * d->stride_k + hk * Dk + i);
      }
      if (d->l2norm) {
        l2_normalise(qv, Dk, d->l2_eps);
        l2_normalise(kv, Dk, d->l2_eps);
      }
      for (int64_t i = 0; i < Dk; ++i) qv[i] *= d->q_scale;
      const double a = exp(ld(log_alpha, d->gate_dtype, tok * Hv + h));
      const double bt = ld(beta, d->gate_dtype, tok * Hv + h);
      for (int64_t jj = 0; jj < nj; ++jj) {
        vv[jj] = ld(v, d->v_dtype, tok * d->stride_v + h * Dv + j0 + jj);
        u[jj] = 0.0;
      }
      /* u = M^T k */
      for (int64_t i = 0; i < Dk; ++i)
        for (int64_t jj = 0; jj < nj; ++jj) u[jj] += M[i * nj + jj] * kv[i];
      /* M <- a M + k (beta (v - a u))^T */
      for (int64_t jj = 0; jj < nj; ++jj) u[jj] = bt * (vv[jj] - a * u[jj]);
      for (int64_t i = 0; i < Dk; ++i)
        for (int64_t jj = 0; jj < nj; ++jj) M[i * nj + jj] = a * M[i * nj + jj] + kv[i] * u[jj];
      /* o = M^T q, read after the update */
      if (o_out) {
        double* orow = o_out + (si * T + t) * Dv + j0;
        for (int64_t jj = 0; jj < nj; ++jj) orow[jj] = 0.0;
        for (int64_t i = 0; i < Dk; ++i)
          for (int64_t jj = 0; jj < nj; ++jj) orow[jj] += M[i * nj + jj] * qv[i];
      }
    }
    if (state_out) {
      for (int64_t i = 0; i < Dk; ++i)
        for (int64_t jj = 0; jj < nj; ++jj) state_out[(si * Dk + i) * Dv + j0 + jj] = M[i * nj + jj];
    }
    free(M);
    free(qv);
    free(kv);
  }
  return 0;
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/*
 * Depthwise causal convolution with K taps followed by SiLU ([HYB] table
 * "Le decompte": kernel 4 over the q|k|v channels, K weights per channel and
 * no bias; [BRI] section 2: SiLU(x) = x sigmoid(x)).
 *     y[b,t,c] = silu( sum_{j=0}^{K-1} w[c][j] * x[b, t-(K-1)+j, c] )
 * Inputs before t = 0 come from conv_state_in[b][c][K-1+t'] (t' = -(K-1)..-1)
 * or are zero when conv_state_in is NULL.  w is [C][K]; x is [B][T][C] with
 * token stride x_stride (elements).  Computes y for batch b, tokens [t0,t1)
 * and channels [c0,c1) into y_out[t1-t0][c1-c0].  When conv_state_out is
 * given it receives, for every (b, c), the last K-1 inputs of the sequence
 * (oldest first), taken from conv_state_in where T < K-1.
 */
int gdn_oracle_conv1d_silu(int64_t B, int64_t T, int64_t C, int64_t K, int64_t x_stride,
                           int32_t x_dtype, const void* x, int32_t w_dtype, const void* w,
                           int32_t cs_dtype, const void* conv_state_in, int64_t b, int64_t t0,
                           int64_t t1, int64_t c0, int64_t c1, double* y_out,
                           double* conv_state_out, int32_t n_threads) {
  if (!x || !w || K < 1 || C < 1 || T < 0 || B < 1) return -1;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
  if (y_out) {
    if (b < 0 || b >= B || t0 < 0 || t1 > T || t0 > t1 || c0 < 0 || c1 > C || c0 > c1) return -1;
    const int64_t nc = c1 - c0;
#pragma omp parallel for schedule(static)
    for (int64_t t = t0; t < t1; ++t) {
      for (int64_t c = c0; c < c1; ++c) {
        double acc = 0.0;
        for (int64_t j = 0; j < K; ++j) {
          const int64_t ts = t - (K - 1) + j;
          double xv = 0.0;
          if (ts >= 0)
            xv = ld(x, x_dtype, (b * T + ts) * x_stride + c);
          else if (conv_state_in)
            xv = ld(conv_state_in, cs_dtype, (b * C + c) * (K - 1) + (K - 1) + ts);
          acc += ld(w, w_dtype, c * K + j) * xv;
        }
        y_out[(t - t0) * nc + (c - c0)] = acc * sigmoid(acc);
      }
    }
  }
  if (conv_state_out && K > 1) {
    for (int64_t bb = 0; bb < B; ++bb)
      for (int64_t c = 0; c < C; ++c)
        for (int64_t j = 0; j < K - 1; ++j) {
          const int64_t ts = T - (K - 1) + j;
          double xv = 0.0;
          if (ts >= 0)
            xv = ld(x, x_dtype, (bb * T + ts) * x_stride + c);
          else if (conv_state_in)
            xv = ld(conv_state_in, cs_dtype, (bb * C + c) * (K - 1) + (K - 1) + ts);
          conv_state_out[(bb * C + c) * (K - 1) + j] = xv;
        }
  }
  return 0;
}

/*
 * Gate activation from the raw per-value-head outputs of the in_proj_ba
 * projection ([HYB] table "Le decompte": in_proj_ba gives beta and alpha, one
 * each per value head, 2 x Hv outputs per token, beta first; [HYB] section
 * "La recurrence": alpha and beta lie in ]0,1[; [BRI] section 2 table: the
 * sigmoid as the gate that squashes into ]0,1[ and softplus(x) = log(1+e^x)).
 * The pages do not give alpha's activation; the layer recipe used for the
 * inputs fixes log alpha = -exp(A_h) * softplus(a + dt_bias_h):
 *     beta_t[h]      = sigmoid(ba[t][h])
 *     log_alpha_t[h] = -exp(A_log[h]) * log(1 + exp(ba[t][Hv + h] + dt_bias[h]))
 * ba is [n_tok][stride] (element stride between tokens); A_log and dt_bias
 * are [Hv]; outputs are [n_tok][Hv].
 */
int gdn_oracle_gates(int64_t n_tok, int64_t Hv, int64_t stride, int32_t ba_dtype, const void* ba,
                     int32_t p_dtype, const void* A_log, const void* dt_bias, double* log_alpha,
                     double* beta) {
  if (n_tok < 0 || Hv < 1 || stride < 2 * Hv || !A_log || !dt_bias || (n_tok > 0 && (!ba || !log_alpha || !beta)))
    return -1;
  for (int64_t t = 0; t < n_tok; ++t)
    for (int64_t h = 0; h < Hv; ++h) {
      const double b = ld(ba, ba_dtype, t * stride + h);
      const double a = ld(ba, ba_dtype, t * stride + Hv + h);
      beta[t * Hv + h] = sigmoid(b);
      /* log1p(e^x) is log(1 + e^x) without rounding 1 + e^x (exact enough down to x ~ -745) */
      log_alpha[t * Hv + h] = -exp(ld(A_log, p_dtype, h)) * log1p(exp(a + ld(dt_bias, p_dtype, h)));
    }
  return 0;
}

/*
 * Swish-gated RMSNorm over rows of D ([BRI] section 4: RMSNorm divides by the
 * root mean square with epsilon inside the root, then multiplies a learned
 * per-coordinate gain; [HYB] config block: output gate of type swish; [HYB]
 * table "Le decompte": one 128-weight vector for the layer, applied per head):
 *     y = x / sqrt(mean(x^2) + eps) * w * z * sigmoid(z)
 * x, z are [rows][D] with row stride D; w is [D].  Computes the selected rows
 * (sel_rows NULL = all) into y_out[n_sel][D].
 */
int gdn_oracle_gated_rmsnorm(int64_t rows, int64_t D, int32_t x_dtype, const void* x,
                             int32_t z_dtype, const void* z, int32_t w_dtype, const void* w,
                             double eps, int64_t n_sel, const int64_t* sel_rows, double* y_out,
                             int32_t n_threads) {
  if (!x || !z || !w || !y_out || D < 1 || rows < 0) return -1;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
  if (!sel_rows) n_sel = rows;
#pragma omp parallel for schedule(static)
  for (int64_t si = 0; si < n_sel; ++si) {
    const int64_t r = sel_rows ? sel_rows[si] : si;
    double ss = 0.0;
    for (int64_t i = 0; i < D; ++i) {
      const double xv = ld(x, x_dtype, r * D + i);
      ss += xv * xv;
    }
    const double inv = 1.0 / sqrt(ss / (double)D + eps);
    for (int64_t i = 0; i < D; ++i) {
      const double zv = ld(z, z_dtype, r * D + i);
      y_out[si * D + i] = ld(x, x_dtype, r * D + i) * inv * ld(w, w_dtype, i) * zv * sigmoid(zv);
    }
  }
  return 0;
}

/*
 * Round doubles to the nearest bf16 (ties to even), returning bit patterns.
 * Used only where an API boundary fixes a bf16 tensor (the conv output fed
 * to the recurrence, the recurrence output fed to the gated norm).  The
 * value is rounded once, directly from double: bf16 keeps 8 significant
 * bits, with subnormal spacing 2^-133 below 2^-126.
 */
void gdn_oracle_round_bf16(const double* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    const double xv = in[i];
    float f;
    if (xv == 0.0 || !isfinite(xv)) {
      f = (float)xv;
    } else {
      int e;
      (void)frexp(xv, &e);          /* xv = m 2^e, 0.5 <= |m| < 1 */
      int se = e - 8;               /* unit of the 8th significant bit */
      if (se < -133) se = -133;
      const double unit = ldexp(1.0, se);
      const double r = nearbyint(xv / unit) * unit; /* exact scaling, ties-to-even */
      f = (fabs(r) > 3.3895313892515355e38) ? (float)copysign(INFINITY, r) : (float)r;
    }
    uint32_t u;
    memcpy(&u, &f, 4);
    out[i] = (uint16_t)(u >> 16);
  }
}
