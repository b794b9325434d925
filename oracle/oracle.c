/*
 * oracle.c -- plain, slow, fp64 CPU oracle for sink-aware grouped-query
 * attention with per-head RMSNorm and NeoX RoPE on Q and K.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file.  Only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or table with the HIP path.
 *
 * Sources (NeMo AutoModel API reference pages):
 *   [L]  "nemo_automodel.components.models.flint.layers" -- FlintAttention
 *        (class summary: separate Q/K/V, per-head RMSNorm, selective NeoX RoPE,
 *        learned sinks; _apply_rope: rotate corresponding channels in the two
 *        halves of each head; forward: full-sequence causal attention with a
 *        zero-value sink category, document-local zero-based THD positions),
 *        _FlintSinkParameters (FP32 denominator logits, returned unscaled,
 *        one per query head).
 *   [C]  "nemo_automodel.components.models.flint.config" -- FlintConfig
 *        (docstring: full layers have no RoPE, sliding layers rotate all head
 *        channels with NeoX RoPE, the window counts the current token;
 *        fields rms_norm_eps = 1e-6, head_dim = 128, 32 / 4 heads).
 *   [U]  "nemo_automodel.components.attention.utils" --
 *        preprocess_args_and_kwargs_for_attn (THD tensors [tokens, heads,
 *        head_dim]; cu_seqlens int32 [documents + 1]; a positive left window
 *        counts visible keys including the current token, negative means
 *        unbounded).
 *
 * Every step is the plain definition, evaluated in double precision from the
 * exactly widened inputs, one (token, head) row at a time:
 *   1. per-head RMSNorm      y = w * x / sqrt(mean(x^2) + eps)              [L],[C]
 *   2. NeoX RoPE (optional)  pair channel i with i + d/2, angle p*theta^(-2i/d) [L],[C]
 *   3. visible set J(t)      same document, p(u) <= p(t), and p(t) - p(u) < W  [L],[C],[U]
 *   4. scores               s_u = scale * <q_hat, k_hat_u>                    [L]
 *   5. softmax with the sink as one extra category of value zero:
 *        M = max(sink, max_J s),  Z = exp(sink - M) + sum_J exp(s_u - M),
 *        out = sum_J exp(s_u - M) v_u / Z,   lse = M + log Z                  [L]
 * Readings where the pages leave a step open (scale 1/sqrt(d), weight shape
 * [d] shared by all heads, norm before RoPE, inv_freq = theta^(-2i/d),
 * kv head = h / (Hq/Hkv), lse including the sink, an empty row giving
 * out = 0 and lse = sink) are listed with the tests that pin them.
 *
 * Parity pinned by tests/test_oracle_pins.py except where noted there.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL -1

/* Document of each token and the token's position inside its document.
 * [L] forward(): THD position_ids are document-local, contiguous and
 * zero-based by default.  cu has num_docs + 1 entries, cu[0] = 0,
 * non-decreasing, cu[num_docs] = T ([U] cu_seqlens). */
static int doc_layout(int T, int num_docs, const int32_t* cu, int32_t* doc_of,
                      int32_t* pos_of) {
  if (cu[0] != 0 || cu[num_docs] != T) return ORACLE_EINVAL;
  for (int n = 0; n < num_docs; ++n) {
    if (cu[n + 1] < cu[n]) return ORACLE_EINVAL;
    for (int t = cu[n]; t < cu[n + 1]; ++t) {
      doc_of[t] = n;
      pos_of[t] = t - cu[n];
    }
  }
  return ORACLE_OK;
}

/* Step 1: per-head RMSNorm of one head vector ([L] FlintAttention q_norm /
 * k_norm; [C] rms_norm_eps).  The weight has head_dim entries shared by all
 * heads of the projection. */
static void rmsnorm_vec(int d, const double* x, const double* w, double eps,
                        double* y) {
  double ss = 0.0;
  for (int i = 0; i < d; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss / (double)d + eps);
  for (int i = 0; i < d; ++i) y[i] = w[i] * x[i] * inv;
}

/* Step 2: NeoX rotary embedding at integer position p ([L] _apply_rope:
 * corresponding channels of the two halves are rotated together; [C] all
 * channels are rotated).  Channel i (i < d/2) and channel i + d/2 form one
 * pair turned by the angle p * theta^(-2i/d). */
static void rope_neox_vec(int d, double p, double theta, double* y) {
  int half = d / 2;
  for (int i = 0; i < half; ++i) {
    double inv_freq = pow(theta, -2.0 * (double)i / (double)d);
    double ang = p * inv_freq;
    double c = cos(ang), s = sin(ang);
    double a = y[i], b = y[i + half];
    y[i] = a * c - b * s;
    y[i + half] = b * c + a * s;
  }
}

/* Steps 1-2 for a whole [rows, H, d] tensor.  x and y may not alias.
 * pos[r] is the document-local position of row r.  Rows are independent, so
 * they are spread over threads with no effect on the values. */
static void prologue_rows(int rows, const int32_t* pos, int H, int d,
                          const double* x, const double* w, double eps,
                          double theta, int use_rope, double* y) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int r = 0; r < rows; ++r)
    for (int h = 0; h < H; ++h) {
      const double* xi = x + ((size_t)r * H + h) * d;
      double* yi = y + ((size_t)r * H + h) * d;
      rmsnorm_vec(d, xi, w, eps, yi);
      if (use_rope) rope_neox_vec(d, (double)pos[r], theta, yi);
    }
}

/* Public: steps 1-2 on every token of a packed THD tensor x [T, H, d]. */
int oracle_rmsnorm_rope(int T, int num_docs, const int32_t* cu, int H, int d,
                        const double* x, const double* w, double eps,
                        double theta, int use_rope, double* y) {
  if (T < 0 || num_docs < 0 || H <= 0 || d <= 0 || (d & 1)) return ORACLE_EINVAL;
  int32_t* doc_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  int32_t* pos_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  int rc = doc_layout(T, num_docs, cu, doc_of, pos_of);
  if (rc == ORACLE_OK)
    prologue_rows(T, pos_of, H, d, x, w, eps, theta, use_rope, y);
  free(doc_of);
  free(pos_of);
  return rc;
}

/* Step 3: is key u visible to query t?  Same document, not in the future
 * ([L] forward: causal), and inside the window when one is set: the window
 * counts the current token, so W = 1 sees only the query itself ([C]
 * docstring; [U] window_size).  window < 0 means unbounded. */
static int visible(int t, int u, const int32_t* doc_of, const int32_t* pos_of,
                   int window) {
  if (doc_of[u] != doc_of[t]) return 0;
  int dp = pos_of[t] - pos_of[u];
  if (dp < 0) return 0;
  if (window > 0 && dp >= window) return 0;
  return 1;
}

/* Steps 3-5 for one (token t, query head) row.  qh: the row's normalised and
 * rotated query [d]; kh, v: [T, Hkv, d]; g: the kv head of this query head.
 * The sink is one more softmax category whose value vector is zero and whose
 * logit is used as given, without the softmax scale ([L]
 * _FlintSinkParameters.forward returns unscaled logits; FlintAttention.forward
 * names the zero-value sink category).  scores is scratch of T doubles. */
static void attend_row(int t, int T, int Hkv, int g, int d, const double* qh,
                       const double* kh, const double* v, double sink,
                       double scale, int window, const int32_t* doc_of,
                       const int32_t* pos_of, double* scores, double* out_row,
                       double* lse_out) {
  /* scores over the visible set */
  int n_vis = 0;
  double M = sink;
  for (int u = 0; u < T; ++u) {
    scores[u] = -INFINITY;
    if (!visible(t, u, doc_of, pos_of, window)) continue;
    const double* ku = kh + ((size_t)u * Hkv + g) * d;
    double dot = 0.0;
    for (int i = 0; i < d; ++i) dot += qh[i] * ku[i];
    scores[u] = scale * dot;
    if (scores[u] > M) M = scores[u];
    ++n_vis;
  }
  for (int i = 0; i < d; ++i) out_row[i] = 0.0;
  if (n_vis == 0) {
    /* No visible key: only the zero-value sink category remains. */
    *lse_out = sink;
    return;
  }
  /* denominator Z includes the sink category; the numerator does not */
  double Z = exp(sink - M);
  for (int u = 0; u < T; ++u) {
    if (scores[u] == -INFINITY) continue;
    double e = exp(scores[u] - M);
    Z += e;
    const double* vu = v + ((size_t)u * Hkv + g) * d;
    for (int i = 0; i < d; ++i) out_row[i] += e * vu[i];
  }
  for (int i = 0; i < d; ++i) out_row[i] /= Z;
  *lse_out = M + log(Z);
}

/* Public: steps 3-5 given already normalised/rotated queries and keys.
 *   qh   [n_rows, Hq, d]   query rows for the tokens listed in rows
 *   kh,v [T, Hkv, d]       every key / value token
 *   rows token index of each query row, or NULL for all T tokens in order
 *   out  [n_rows, Hq, d];  lse [Hq, n_rows] (may be NULL)
 * Query head h reads kv head h / (Hq / Hkv).  nthreads <= 0 uses every
 * OpenMP thread.  Returns 0, or -1 on an invalid argument. */
int oracle_attention(int T, int num_docs, const int32_t* cu, int Hq, int Hkv,
                     int d, const double* qh, const double* kh,
                     const double* v, const double* sinks, double scale,
                     int window, const int32_t* rows, int n_rows, double* out,
                     double* lse, int nthreads) {
  if (T < 0 || num_docs < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv)
    return ORACLE_EINVAL;
  if (window == 0) return ORACLE_EINVAL;
  if (rows == NULL) n_rows = T;
  if (n_rows < 0) return ORACLE_EINVAL;
  int32_t* doc_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  int32_t* pos_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  int rc = doc_layout(T, num_docs, cu, doc_of, pos_of);
  if (rc == ORACLE_OK && rows)
    for (int r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= T) rc = ORACLE_EINVAL;
  if (rc != ORACLE_OK) {
    free(doc_of);
    free(pos_of);
    return rc;
  }
  int group = Hq / Hkv;
#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#endif
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    double lse_val;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (long item = 0; item < (long)n_rows * Hq; ++item) {
      int r = (int)(item / Hq), h = (int)(item % Hq);
      int t = rows ? rows[r] : r;
      attend_row(t, T, Hkv, h / group, d, qh + ((size_t)r * Hq + h) * d, kh, v,
                 sinks[h], scale, window, doc_of, pos_of, scores,
                 out + ((size_t)r * Hq + h) * d, &lse_val);
      if (lse) lse[(size_t)h * n_rows + r] = lse_val;
    }
    free(scores);
  }
  free(doc_of);
  free(pos_of);
  return ORACLE_OK;
}

/* Public: the whole forward pass, steps 1-5.
 *   q [n_rows, Hq, d] raw (projected) queries of the tokens in rows (all T
 *   tokens when rows is NULL); k, v [T, Hkv, d] raw keys and values;
 *   qnorm_w, knorm_w [d]; sinks [Hq]; scale <= 0 selects 1/sqrt(d).
 * V passes through untouched ([L]: only Q and K are normalised and rotated). */
int oracle_sink_attn_fwd(int T, int num_docs, const int32_t* cu, int Hq,
                         int Hkv, int d, const double* q, const double* k,
                         const double* v, const double* sinks,
                         const double* qnorm_w, const double* knorm_w,
                         double eps, double theta, double scale, int window,
                         int use_rope, const int32_t* rows, int n_rows,
                         double* out, double* lse, int nthreads) {
  if (T < 0 || num_docs < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || (d & 1) ||
      Hq % Hkv || window == 0)
    return ORACLE_EINVAL;
  if (rows == NULL) n_rows = T;
  if (n_rows < 0) return ORACLE_EINVAL;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
  int32_t* doc_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  int32_t* pos_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  int32_t* qpos = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_rows > 0 ? n_rows : 1));
  int rc = doc_layout(T, num_docs, cu, doc_of, pos_of);
  for (int r = 0; rc == ORACLE_OK && r < n_rows; ++r) {
    int t = rows ? rows[r] : r;
    if (t < 0 || t >= T) rc = ORACLE_EINVAL;
    else qpos[r] = pos_of[t];
  }
  double* qh = NULL;
  double* kh = NULL;
  if (rc == ORACLE_OK) {
    qh = (double*)malloc(sizeof(double) * ((size_t)n_rows * Hq * d + 1));
    kh = (double*)malloc(sizeof(double) * ((size_t)T * Hkv * d + 1));
    prologue_rows(n_rows, qpos, Hq, d, q, qnorm_w, eps, theta, use_rope, qh);
    prologue_rows(T, pos_of, Hkv, d, k, knorm_w, eps, theta, use_rope, kh);
    rc = oracle_attention(T, num_docs, cu, Hq, Hkv, d, qh, kh, v, sinks, scale,
                          window, rows, n_rows, out, lse, nthreads);
  }
  free(qh);
  free(kh);
  free(qpos);
  free(doc_of);
  free(pos_of);
  return rc;
}

/* ------------------------------------------------------------------------
 * Backward pass: gradients of L = sum(dout * out) with respect to q, k, v,
 * the sinks and the two norm weights, for the forward above.  Each is the
 * derivative of steps 1-5 by the chain rule, evaluated in double precision:
 *   step 5, per (token t, query head h) with weights P_u = exp(s_u - lse) over
 *   the visible set and p_sink = exp(sink - lse):
 *     D       = dout_t . out_t
 *     dv_u   += P_u dout_t                       (summed over the heads of u's group)
 *     dS_u    = P_u (dout_t . v_u - D)
 *     dsink_h -= p_sink D                        (the sink's value is zero)
 *   step 4:  dq_hat_t += scale sum_u dS_u k_hat_u,  dk_hat_u += scale dS_u q_hat_t
 *   step 2:  the transpose of the rotation: rotate each pair back by -angle
 *   step 1:  y = w x r with r = (mean(x^2) + eps)^(-1/2):
 *            dw += dy x r,  dx = w dy r - x r^3 (sum_c w_c dy_c x_c) / d
 * The sinks are trainable fp32 logits ([L] _FlintSinkParameters) and the norm
 * weights are the RMSNorm parameters ([L] q_norm / k_norm).
 * ------------------------------------------------------------------------ */

static int all_zero(int d, const double* x) {
  for (int i = 0; i < d; ++i)
    if (x[i] != 0.0) return 0;
  return 1;
}

/* Transpose of step 2 for one head vector: turn each pair by -angle. */
static void rope_neox_vec_t(int d, double p, double theta, double* y) {
  int half = d / 2;
  for (int i = 0; i < half; ++i) {
    double inv_freq = pow(theta, -2.0 * (double)i / (double)d);
    double ang = p * inv_freq;
    double c = cos(ang), s = sin(ang);
    double a = y[i], b = y[i + half];
    y[i] = a * c + b * s;
    y[i + half] = b * c - a * s;
  }
}

/* Backward of step 1 for one head vector: dy -> dx, and dy * x * r added
 * into dw. */
static void rmsnorm_vec_bwd(int d, const double* x, const double* w, double eps,
                            const double* dy, double* dx, double* dw) {
  double ss = 0.0;
  for (int i = 0; i < d; ++i) ss += x[i] * x[i];
  double r = 1.0 / sqrt(ss / (double)d + eps);
  double dot = 0.0;
  for (int i = 0; i < d; ++i) dot += w[i] * dy[i] * x[i];
  for (int i = 0; i < d; ++i) {
    dx[i] = w[i] * dy[i] * r - x[i] * r * r * r * dot / (double)d;
    dw[i] += dy[i] * x[i] * r;
  }
}

/* Public: gradients of sum(dout * out) for the whole forward pass.
 *   q, dout, dq [T, Hq, d]; k, v, dk, dv [T, Hkv, d]; dsinks [Hq];
 *   dqnorm_w, dknorm_w [d].  Every output is overwritten.  Two passes, each
 *   split over independent outputs: pass 1 over (token, query head) rows
 *   (the forward row, D, the row's sink term and dq_hat), pass 2 over (key,
 *   kv head) pairs (dk_hat and dv, from the rows' stored lse and D).  Every
 *   sum is added in a fixed order -- dq_hat over keys in token order; dk_hat
 *   and dv over queries in token order, then head order; dsink and the norm
 *   weights over tokens in order -- so the result does not depend on the
 *   thread count.  A row whose dout is zero contributes exactly nothing: its
 *   D is 0, so dS = P (0 - 0) = 0 for every key it sees and its dv terms are
 *   P * 0 (its lse is finite, since a query always sees its own key).  Both
 *   passes skip such rows; that changes no value (adding a signed zero to a
 *   sum leaves it as it is) and makes a backward whose dout is non-zero on a
 *   sample of rows cost time in proportion to the sample. */
int oracle_sink_attn_bwd(int T, int num_docs, const int32_t* cu, int Hq, int Hkv,
                         int d, const double* q, const double* k, const double* v,
                         const double* sinks, const double* qnorm_w,
                         const double* knorm_w, double eps, double theta,
                         double scale, int window, int use_rope, const double* dout,
                         double* dq, double* dk, double* dv, double* dsinks,
                         double* dqnorm_w, double* dknorm_w, int nthreads) {
  if (T < 0 || num_docs < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || (d & 1) ||
      Hq % Hkv || window == 0)
    return ORACLE_EINVAL;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
  int32_t* doc_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  int32_t* pos_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  int rc = doc_layout(T, num_docs, cu, doc_of, pos_of);
  if (rc != ORACLE_OK) {
    free(doc_of);
    free(pos_of);
    return rc;
  }
  const int group = Hq / Hkv;
  const size_t nq = (size_t)T * Hq * d, nk = (size_t)T * Hkv * d;
  const size_t nrow = (size_t)T * Hq;
  double* qh = (double*)malloc(sizeof(double) * (nq + 1));
  double* kh = (double*)malloc(sizeof(double) * (nk + 1));
  double* dqh = (double*)calloc(nq + 1, sizeof(double));
  double* dkh = (double*)calloc(nk + 1, sizeof(double));
  double* row_lse = (double*)malloc(sizeof(double) * (nrow + 1));
  double* row_D = (double*)malloc(sizeof(double) * (nrow + 1));
  double* row_sink = (double*)malloc(sizeof(double) * (nrow + 1));
  /* rows with a non-zero dout, and per (token, kv head) whether any row of
   * the group has one */
  unsigned char* row_live = (unsigned char*)malloc(nrow + 1);
  unsigned char* grp_live = (unsigned char*)malloc((size_t)T * Hkv + 1);
  for (size_t r = 0; r < nrow; ++r) {
    int live = 0;
    for (int i = 0; i < d && !live; ++i) live = dout[r * d + i] != 0.0;
    row_live[r] = (unsigned char)live;
  }
  for (size_t c = 0; c < (size_t)T * Hkv; ++c) {
    int live = 0;
    for (int j = 0; j < group; ++j) live |= row_live[c * group + j];
    grp_live[c] = (unsigned char)live;
  }
  prologue_rows(T, pos_of, Hq, d, q, qnorm_w, eps, theta, use_rope, qh);
  prologue_rows(T, pos_of, Hkv, d, k, knorm_w, eps, theta, use_rope, kh);
  for (size_t i = 0; i < nk; ++i) dv[i] = 0.0;

#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#endif
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    double* out_row = (double*)malloc(sizeof(double) * (size_t)d);
    /* pass 1: per (token t, query head h) row -- steps 3-5 forward, then
     * D = dout . out, the row's term of dsink, and dq_hat over the visible keys
     * in token order */
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (long r = 0; r < (long)nrow; ++r) {
      const int t = (int)(r / Hq), h = (int)(r % Hq), g = h / group;
      const int n = doc_of[t];
      const double* qrow = qh + (size_t)r * d;
      const double* dorow = dout + (size_t)r * d;
      if (!row_live[r]) {  /* zero dout: D = 0, no dsink term, dq_hat stays 0 */
        row_lse[r] = 0.0;
        row_D[r] = 0.0;
        row_sink[r] = 0.0;
        continue;
      }
      double lse;
      attend_row(t, T, Hkv, g, d, qrow, kh, v, sinks[h], scale, window, doc_of, pos_of,
                 scores, out_row, &lse);
      double D = 0.0;
      for (int i = 0; i < d; ++i) D += dorow[i] * out_row[i];
      row_lse[r] = lse;
      row_D[r] = D;
      row_sink[r] = exp(sinks[h] - lse) * D;
      double* dqrow = dqh + (size_t)r * d;
      for (int u = cu[n]; u <= t; ++u) {
        if (scores[u] == -INFINITY) continue;
        const double P = exp(scores[u] - lse);
        const double* vu = v + ((size_t)u * Hkv + g) * d;
        const double* ku = kh + ((size_t)u * Hkv + g) * d;
        double dP = 0.0;
        for (int i = 0; i < d; ++i) dP += dorow[i] * vu[i];
        const double dS = P * (dP - D);
        for (int i = 0; i < d; ++i) dqrow[i] += scale * dS * ku[i];
      }
    }
    /* pass 2: per (key u, kv head g) -- dk_hat and dv over the queries that
     * see u, in token order, then head order (the scores, weights and dS are
     * the same expressions as in pass 1 and attend_row) */
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (long c = 0; c < (long)T * Hkv; ++c) {
      const int u = (int)(c / Hkv), g = (int)(c % Hkv);
      const int n = doc_of[u];
      const double* vu = v + (size_t)c * d;
      const double* ku = kh + (size_t)c * d;
      double* dku = dkh + (size_t)c * d;
      double* dvu = dv + (size_t)c * d;
      /* the queries that can see u: [u, end of its document), and under a
       * window only the first `window` of them (visible() is 0 past that) */
      const int t_end = window > 0 && window < cu[n + 1] - u ? u + window : cu[n + 1];
      for (int t = u; t < t_end; ++t) {
        if (!grp_live[(size_t)t * Hkv + g] || !visible(t, u, doc_of, pos_of, window)) continue;
        for (int h = g * group; h < (g + 1) * group; ++h) {
          const size_t r = (size_t)t * Hq + h;
          if (!row_live[r]) continue;
          const double* qrow = qh + r * d;
          const double* dorow = dout + r * d;
          double dot = 0.0;
          for (int i = 0; i < d; ++i) dot += qrow[i] * ku[i];
          const double s = scale * dot;
          const double P = exp(s - row_lse[r]);
          double dP = 0.0;
          for (int i = 0; i < d; ++i) dP += dorow[i] * vu[i];
          const double dS = P * (dP - row_D[r]);
          for (int i = 0; i < d; ++i) {
            dku[i] += scale * dS * qrow[i];
            dvu[i] += P * dorow[i];
          }
        }
      }
    }
    free(scores);
    free(out_row);
  }
  /* dsink_h = -sum over the tokens of each document, in token order, then
   * over documents in order */
  for (int h = 0; h < Hq; ++h) {
    dsinks[h] = 0.0;
    for (int n = 0; n < num_docs; ++n) {
      double part = 0.0;
      for (int t = cu[n]; t < cu[n + 1]; ++t) part -= row_sink[(size_t)t * Hq + h];
      dsinks[h] += part;
    }
  }
  /* steps 2 and 1 backwards, token by token in order (fixed summation order
   * for the norm weights) */
  /* (a row whose dy is all zero has dx = 0 and adds nothing to dw, so it is
   * written as zeros without the rotation and norm steps) */
  for (int i = 0; i < d; ++i) dqnorm_w[i] = dknorm_w[i] = 0.0;
  for (int t = 0; t < T; ++t) {
    for (int h = 0; h < Hq; ++h) {
      double* dy = dqh + ((size_t)t * Hq + h) * d;
      double* dx = dq + ((size_t)t * Hq + h) * d;
      if (all_zero(d, dy)) {
        for (int i = 0; i < d; ++i) dx[i] = 0.0;
        continue;
      }
      if (use_rope) rope_neox_vec_t(d, (double)pos_of[t], theta, dy);
      rmsnorm_vec_bwd(d, q + ((size_t)t * Hq + h) * d, qnorm_w, eps, dy, dx, dqnorm_w);
    }
    for (int g = 0; g < Hkv; ++g) {
      double* dy = dkh + ((size_t)t * Hkv + g) * d;
      double* dx = dk + ((size_t)t * Hkv + g) * d;
      if (all_zero(d, dy)) {
        for (int i = 0; i < d; ++i) dx[i] = 0.0;
        continue;
      }
      if (use_rope) rope_neox_vec_t(d, (double)pos_of[t], theta, dy);
      rmsnorm_vec_bwd(d, k + ((size_t)t * Hkv + g) * d, knorm_w, eps, dy, dx, dknorm_w);
    }
  }
  free(qh);
  free(kh);
  free(dqh);
  free(dkh);
  free(row_lse);
  free(row_D);
  free(row_sink);
  free(row_live);
  free(grp_live);
  free(doc_of);
  free(pos_of);
  return ORACLE_OK;
}

/* Number of OpenMP threads a call with nthreads <= 0 would use. */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
