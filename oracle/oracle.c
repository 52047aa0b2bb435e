/*
 * oracle.c -- plain, slow, fp64 CPU oracle for exact blockwise / ring attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant with the HIP
 * path.
 *
 * Sources (cited by page title and section):
 *  [LVX]  "LV-XAttn: Distributed Cross-Attention for Long Visual Inputs in
 *         Multimodal Large Language Models" (Pith review page):
 *         - "What carries the argument": KV blocks stay on their worker, the
 *           query block Q_i, partial output O_i and softmax statistics L_i
 *           rotate, and partial outputs are rescaled as in FlashAttention;
 *           recompute of K, V from the one shared copy of the visual tokens y.
 *         - Figure 3 caption (start of Algorithm 1): per-worker blocks
 *           Q_i, K_i, V_i; O_i, L_i initialised; one loop of n rounds.
 *         - "Assumptions": online-softmax rescaling computes exact attention.
 *         - Referee report, major comment 1: the backward must be the exact
 *           gradient of the attention formula (checked against autograd).
 *  [RING] "Ring Attention with Blockwise Transformers for Near-Infinite
 *         Context", abstract (Pith citation hub page): blockwise attention,
 *         KV blocks passed around a ring, no approximation.
 *
 * Readings where the pages are silent (each is also listed in the design notes):
 *  - L_i is the log-sum-exp m + ln(l) of the (scaled) logits of a row,
 *    natural log, scale included; the identity element of the merge is
 *    (O = 0, L = -inf), not (0, 0).
 *  - scale tau = 1/sqrt(D) with D the per-head dimension (the caller passes it).
 *  - causal (self-attention only, S_Q == S_KV): key j is allowed for query i
 *    iff j <= i.
 *  - shard k of a length-S sequence split n ways is [floor(kS/n), floor((k+1)S/n)).
 *  - round r pairs for virtual worker w:
 *      KV-stationary (LV-XAttn): query block (w - r) mod n with KV shard w;
 *      Q-stationary  (Ring):     query block w with KV shard (w - r) mod n.
 *  - backward: the exact gradient of O = softmax(tau Q K^T) V.
 *
 * Inputs are read through ld(), which widens f64 / f32 / bf16 (raw bits)
 * element i to double.  All arithmetic is fp64.  Tensors are contiguous:
 * q [B,H,SQ,D], k and v [B,H,SKV,D], o [B,H,SQ,D], lse [B,H,SQ].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F64 = 0, ORC_F32 = 1, ORC_BF16 = 2 };

static double ld(const void* p, int dt, int64_t i) {
  if (dt == ORC_F64) return ((const double*)p)[i];
  if (dt == ORC_F32) return (double)((const float*)p)[i];
  /* bf16: the 16 stored bits are the upper half of an IEEE binary32. */
  uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sequence position held by row i of a striped layout of S rows over n
 * shards (the token assignment of "Striped attention: Faster ring attention
 * for causal transformers", named in the LV-XAttn review's references; the
 * pages give only the title, read as round-robin): shard w = rows
 * [w*S/n, (w+1)*S/n) holds positions w, w+n, w+2n, ... in order. */
static int64_t stripe_pos(int64_t i, int64_t S, int64_t n) {
  int64_t blk = S / n;
  return (i % blk) * n + i / blk;
}

/* Is key j visible to query i?  causal: 0 none; 1 key position <= query
 * position with rows in sequence order; -n the same with rows in the striped
 * order over n shards (S = sequence length). */
static int allowed(int causal, int64_t S, int64_t i, int64_t j) {
  if (causal == 0) return 1;
  if (causal > 0) return j <= i;
  return stripe_pos(j, S, -causal) <= stripe_pos(i, S, -causal);
}

/*
 * Attention of one query row against the keys j in [k0, k1) that it may see:
 *   s_j = tau * sum_d q_d k_jd,  m = max_j s_j,  l = sum_j exp(s_j - m),
 *   o   = (1/l) sum_j exp(s_j - m) v_j,  LSE = m + ln l.
 * No visible key gives o = 0, LSE = -inf.  s is scratch of k1 - k0 doubles.
 * Returns LSE and writes o[0..D).
 */
static double attn_row(const void* q, const void* k, const void* v, int dt,
                       int64_t qrow, int64_t kvbase, int64_t D, int64_t i,
                       int64_t k0, int64_t k1, double tau, int causal, int64_t S,
                       double* s, double* o) {
  double m = -INFINITY;
  for (int64_t j = k0; j < k1; ++j) {
    if (!allowed(causal, S, i, j)) { s[j - k0] = -INFINITY; continue; }
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d)
      dot += ld(q, dt, qrow * D + d) * ld(k, dt, (kvbase + j) * D + d);
    s[j - k0] = tau * dot;
    if (s[j - k0] > m) m = s[j - k0];
  }
  for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
  if (m == -INFINITY) return -INFINITY;
  double l = 0.0;
  for (int64_t j = k0; j < k1; ++j) {
    if (s[j - k0] == -INFINITY) continue;
    double p = exp(s[j - k0] - m);
    l += p;
    for (int64_t d = 0; d < D; ++d) o[d] += p * ld(v, dt, (kvbase + j) * D + d);
  }
  for (int64_t d = 0; d < D; ++d) o[d] /= l;
  return m + log(l);
}

/*
 * Unblocked attention (the plain definition) for the listed rows.
 * rows[r] is a flat row index (b*H + h)*SQ + i; o_out is [nrows, D],
 * lse_out is [nrows].  rows == NULL means every row in order.
 */
void orc_attn_fwd_rows(const void* q, const void* k, const void* v, int dt,
                       int64_t B, int64_t H, int64_t SQ, int64_t SKV, int64_t D,
                       double tau, int causal, const int64_t* rows, int64_t nrows,
                       double* o_out, double* lse_out) {
  (void)B; (void)H;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(SKV > 0 ? SKV : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
      int64_t row = rows ? rows[r] : r;
      int64_t bh = row / SQ, i = row % SQ;
      lse_out[r] = attn_row(q, k, v, dt, row, bh * SKV, D, i, 0, SKV, tau, causal, SKV,
                            s, o_out + r * D);
    }
    free(s);
  }
}

/*
 * Partial of every query row in [q0, q1) against keys [k0, k1): the same
 * definition restricted to a key subset (one block pair of the ring).
 * Writes o_out [B,H,SQ,D] and lse_out [B,H,SQ] only for rows in [q0, q1).
 */
void orc_attn_partial(const void* q, const void* k, const void* v, int dt,
                      int64_t B, int64_t H, int64_t SQ, int64_t SKV, int64_t D,
                      double tau, int causal, int64_t q0, int64_t q1,
                      int64_t k0, int64_t k1, double* o_out, double* lse_out) {
  int64_t nq = q1 - q0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(k1 - k0 > 0 ? k1 - k0 : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < B * H * nq; ++t) {
      int64_t bh = t / nq, i = q0 + t % nq;
      int64_t row = bh * SQ + i;
      lse_out[row] = attn_row(q, k, v, dt, row, bh * SKV, D, i, k0, k1, tau, causal, SKV,
                              s, o_out + row * D);
    }
    free(s);
  }
}

/*
 * Rescale-merge of two partials of the same rows over disjoint key sets:
 *   M = max(La, Lb),  L = M + ln(exp(La - M) + exp(Lb - M)),
 *   O = exp(La - L) Oa + exp(Lb - L) Ob.
 * (0, -inf) is the identity; two empty partials stay (0, -inf).
 * The output may alias either input.
 */
void orc_merge(int64_t rows, int64_t D, const double* oa, const double* la,
               const double* ob, const double* lb, double* o_out, double* l_out) {
  for (int64_t r = 0; r < rows; ++r) {
    double M = la[r] > lb[r] ? la[r] : lb[r];
    if (M == -INFINITY) {
      for (int64_t d = 0; d < D; ++d) o_out[r * D + d] = 0.0;
      l_out[r] = -INFINITY;
      continue;
    }
    double L = M + log(exp(la[r] - M) + exp(lb[r] - M));
    double wa = exp(la[r] - L), wb = exp(lb[r] - L);
    for (int64_t d = 0; d < D; ++d)
      o_out[r * D + d] = wa * oa[r * D + d] + wb * ob[r * D + d];
    l_out[r] = L;
  }
}

/* Shard k of a length-S sequence split n ways: [floor(kS/n), floor((k+1)S/n)). */
int64_t orc_shard_start(int64_t S, int64_t n, int64_t k) { return (k * S) / n; }

/*
 * The pair virtual worker w works on in round r (0 <= r, w < n):
 *   sched 0, KV-stationary (LV-XAttn): KV shard w stays, the query block
 *            that arrives in round r is (w - r) mod n;
 *   sched 1, Q-stationary (Ring):      query block w stays, the KV shard that
 *            arrives in round r is (w - r) mod n.
 */
void orc_ring_pair(int sched, int64_t n, int64_t r, int64_t w, int64_t* qblk, int64_t* kblk) {
  int64_t moved = ((w - r) % n + n) % n;
  if (sched == 0) { *qblk = moved; *kblk = w; }
  else            { *qblk = w;     *kblk = moved; }
}

/*
 * The ring forward as the pages describe it, with the transfers replaced by
 * indexing: O, L start at the identity (0, -inf); in each of the n rounds
 * every worker attends the query block it holds to the KV shard it holds and
 * rescale-merges the partial into that query block's running (O, L).
 * Query blocks and KV shards use the same n-way split of SQ and SKV.
 * o_out [B,H,SQ,D], lse_out [B,H,SQ].
 */
void orc_ring_fwd(const void* q, const void* k, const void* v, int dt,
                  int64_t B, int64_t H, int64_t SQ, int64_t SKV, int64_t D,
                  double tau, int causal, int64_t n, int sched,
                  double* o_out, double* lse_out) {
  int64_t rows = B * H * SQ;
  double* po = (double*)calloc((size_t)(rows * D), sizeof(double));
  double* pl = (double*)malloc(sizeof(double) * (size_t)rows);
  for (int64_t r = 0; r < rows; ++r) {
    lse_out[r] = -INFINITY;
    for (int64_t d = 0; d < D; ++d) o_out[r * D + d] = 0.0;
  }
  for (int64_t round = 0; round < n; ++round) {
    for (int64_t w = 0; w < n; ++w) {
      int64_t qb, kb;
      orc_ring_pair(sched, n, round, w, &qb, &kb);
      int64_t q0 = orc_shard_start(SQ, n, qb), q1 = orc_shard_start(SQ, n, qb + 1);
      int64_t k0 = orc_shard_start(SKV, n, kb), k1 = orc_shard_start(SKV, n, kb + 1);
      if (q1 == q0) continue;
      orc_attn_partial(q, k, v, dt, B, H, SQ, SKV, D, tau, causal, q0, q1, k0, k1, po, pl);
      for (int64_t bh = 0; bh < B * H; ++bh) {
        int64_t base = bh * SQ + q0;
        orc_merge(q1 - q0, D, o_out + base * D, lse_out + base, po + base * D, pl + base,
                  o_out + base * D, lse_out + base);
      }
    }
  }
  free(po);
  free(pl);
}

/*
 * Exact gradient of O = softmax(tau Q K^T) V for the listed (b, h) heads
 * (heads[t] = b*H + h), given dO.  With s_ij = tau q_i . k_j over visible j:
 *   LSE_i = ln sum_j exp(s_ij),  P_ij = exp(s_ij - LSE_i)  (0 where masked),
 *   dP_ij = dO_i . v_j,  Dlt_i = sum_j P_ij dP_ij,  dS_ij = P_ij (dP_ij - Dlt_i),
 *   dQ_i = tau sum_j dS_ij k_j,  dK_j = tau sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i.
 * Outputs are per listed head: dq [nh,SQ,D], lse_out and delta_out [nh,SQ],
 * dk and dv [nh,nkeys,D] for the listed keys (keys == NULL: all SKV keys).
 * Pass 1 runs over query rows (LSE, Dlt, dQ); pass 2 runs over keys
 * (dK, dV) and recomputes s and dP.
 */
void orc_attn_bwd_heads(const void* q, const void* k, const void* v, const void* dout,
                        int dt, int dt_do, int64_t B, int64_t H, int64_t SQ, int64_t SKV,
                        int64_t D, double tau, int causal, const int64_t* heads, int64_t nh,
                        const int64_t* keys, int64_t nkeys,
                        double* dq, double* dk, double* dv, double* lse_out, double* delta_out) {
  (void)B; (void)H;
  for (int64_t t = 0; t < nh; ++t) {
    int64_t bh = heads[t];
    const int64_t qb = bh * SQ, kb = bh * SKV;
    double* lse = lse_out + t * SQ;
    double* dlt = delta_out + t * SQ;
#pragma omp parallel
    {
      double* s = (double*)malloc(sizeof(double) * (size_t)(SKV > 0 ? SKV : 1));
      double* dp = (double*)malloc(sizeof(double) * (size_t)(SKV > 0 ? SKV : 1));
#pragma omp for schedule(dynamic, 1)
      for (int64_t i = 0; i < SQ; ++i) {
        double m = -INFINITY;
        for (int64_t j = 0; j < SKV; ++j) {
          if (!allowed(causal, SKV, i, j)) { s[j] = -INFINITY; dp[j] = 0.0; continue; }
          double dot = 0.0, dpo = 0.0;
          for (int64_t d = 0; d < D; ++d) {
            dot += ld(q, dt, (qb + i) * D + d) * ld(k, dt, (kb + j) * D + d);
            dpo += ld(dout, dt_do, (qb + i) * D + d) * ld(v, dt, (kb + j) * D + d);
          }
          s[j] = tau * dot;
          dp[j] = dpo;
          if (s[j] > m) m = s[j];
        }
        double* g = dq + (t * SQ + i) * D;
        for (int64_t d = 0; d < D; ++d) g[d] = 0.0;
        if (m == -INFINITY) { lse[i] = -INFINITY; dlt[i] = 0.0; continue; }
        double l = 0.0;
        for (int64_t j = 0; j < SKV; ++j)
          if (s[j] != -INFINITY) l += exp(s[j] - m);
        lse[i] = m + log(l);
        double delta = 0.0;
        for (int64_t j = 0; j < SKV; ++j)
          if (s[j] != -INFINITY) delta += exp(s[j] - lse[i]) * dp[j];
        dlt[i] = delta;
        for (int64_t j = 0; j < SKV; ++j) {
          if (s[j] == -INFINITY) continue;
          double P = exp(s[j] - lse[i]);
          double dS = P * (dp[j] - delta);
          for (int64_t d = 0; d < D; ++d) g[d] += tau * dS * ld(k, dt, (kb + j) * D + d);
        }
      }
      free(s);
      free(dp);
    }
    int64_t nk = keys ? nkeys : SKV;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t jj = 0; jj < nk; ++jj) {
      int64_t j = keys ? keys[jj] : jj;
      double* gk = dk + (t * nk + jj) * D;
      double* gv = dv + (t * nk + jj) * D;
      for (int64_t d = 0; d < D; ++d) { gk[d] = 0.0; gv[d] = 0.0; }
      for (int64_t i = 0; i < SQ; ++i) {
        if (!allowed(causal, SKV, i, j) || lse[i] == -INFINITY) continue;
        double dot = 0.0, dpo = 0.0;
        for (int64_t d = 0; d < D; ++d) {
          dot += ld(q, dt, (qb + i) * D + d) * ld(k, dt, (kb + j) * D + d);
          dpo += ld(dout, dt_do, (qb + i) * D + d) * ld(v, dt, (kb + j) * D + d);
        }
        double P = exp(tau * dot - lse[i]);
        double dS = P * (dpo - dlt[i]);
        for (int64_t d = 0; d < D; ++d) {
          gk[d] += tau * dS * ld(q, dt, (qb + i) * D + d);
          gv[d] += P * ld(dout, dt_do, (qb + i) * D + d);
        }
      }
    }
  }
}

/*
 * Recompute of keys (or values) from the shared visual features:
 *   out[b, h, s, d] = sum_e y[b, s, e] * W[e, h*D + d]
 * where W (E x H*D) is stored transposed, as w_t[n, e] = W[e, n]
 * (row n = h*D + d holds column n of W).  Only the listed (b, s) rows
 * (rows[t] = b*S + s) are computed; out is [nrows, H*D] in (h, d) order.
 */
void orc_kv_proj_rows(const void* y, const void* w_t, int dt, int64_t B, int64_t S,
                      int64_t E, int64_t HD, const int64_t* rows, int64_t nrows, double* out) {
  (void)B; (void)S;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < nrows; ++t) {
    int64_t row = rows ? rows[t] : t;
    for (int64_t nn = 0; nn < HD; ++nn) {
      double acc = 0.0;
      for (int64_t e = 0; e < E; ++e) acc += ld(y, dt, row * E + e) * ld(w_t, dt, nn * E + e);
      out[t * HD + nn] = acc;
    }
  }
}

/* ------------------------------------------------------------------------
 * Gradients through the recompute ([LVX] "What carries the argument": K, V
 * are recomputed from the one shared y, so the backward also yields the
 * gradients of W_k, W_v and y).  Plain definitions of the derivatives of
 * K[b,h,s,d] = sum_e y[b,s,e] * w_t[h*D+d, e]:
 *   dW_t[n, e] = sum_{b,s} g[b, h, s, d] * y[b, s, e]       (n = h*D + d)
 *   dy[b, s, e] = sum_n gk[b, h, s, d] * wk_t[n, e] + gv[b, h, s, d] * wv_t[n, e]
 * g, gk, gv are [B, H, S, D] contiguous. */
static double g_at(const void* g, int dt, int64_t H, int64_t S, int64_t D, int64_t b, int64_t s,
                   int64_t n) {
  int64_t h = n / D, d = n % D;
  return ld(g, dt, ((b * H + h) * S + s) * D + d);
}

/* rows n of dW_t (nrows of them, or all H*D when nrows < 0), out [nrows, E] */
void orc_kv_grad_w_rows(const void* y, const void* g, int dt, int64_t B, int64_t S, int64_t E,
                        int64_t H, int64_t D, const int64_t* rows, int64_t nrows, double* out) {
  int64_t cnt = nrows < 0 ? H * D : nrows;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < cnt; ++t) {
    int64_t n = nrows < 0 ? t : rows[t];
    for (int64_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t b = 0; b < B; ++b)
        for (int64_t s = 0; s < S; ++s)
          acc += g_at(g, dt, H, S, D, b, s, n) * ld(y, dt, (b * S + s) * E + e);
      out[t * E + e] = acc;
    }
  }
}

/* rows (b*S + s) of dy (nrows of them, or all B*S when nrows < 0), out [nrows, E] */
void orc_kv_grad_y_rows(const void* gk, const void* gv, const void* wk_t, const void* wv_t,
                        int dt, int64_t B, int64_t S, int64_t E, int64_t H, int64_t D,
                        const int64_t* rows, int64_t nrows, double* out) {
  int64_t cnt = nrows < 0 ? B * S : nrows;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < cnt; ++t) {
    int64_t row = nrows < 0 ? t : rows[t];
    int64_t b = row / S, s = row % S;
    for (int64_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t n = 0; n < H * D; ++n)
        acc += g_at(gk, dt, H, S, D, b, s, n) * ld(wk_t, dt, n * E + e) +
               g_at(gv, dt, H, S, D, b, s, n) * ld(wv_t, dt, n * E + e);
      out[t * E + e] = acc;
    }
  }
}

/* ------------------------------------------------------------------------
 * Per-round cost model of the two ring schedules ([LVX] "What carries the
 * argument": a round lasts max(f(S_Q d/n, S_KV d/n), comm(message)), with
 * message 2 S_Q d/n + S_Q/n elements for LV-XAttn (Q_i, O_i, L_i) and
 * 2 S_KV d/n elements for Ring Attention (K_i, V_i)).
 * Reading: f is the FLOP count of one block pair, two contractions of a
 * (S_Q/n x d) block with a (S_KV/n x d) block, a multiply-add counted as 2;
 * comm(x) = x * elem_bytes / bytes_per_s.  out = {compute, comm_lv,
 * comm_ring, round_lv, round_ring} seconds; returns 0 (LV-XAttn) when its
 * round is not longer, else 1 (Ring). */
int orc_schedule_model(double S_Q, double S_KV, double d, double n, double flops_per_s,
                       double bytes_per_s, double elem_bytes, double* out) {
  double q_block = S_Q / n, kv_block = S_KV / n;
  double f = 2.0 * (2.0 * q_block * kv_block * d); /* S = Q K^T, then P V */
  double lv_elems = 2.0 * S_Q * d / n + S_Q / n;
  double ring_elems = 2.0 * S_KV * d / n;
  double t_f = f / flops_per_s;
  double t_lv = lv_elems * elem_bytes / bytes_per_s;
  double t_ring = ring_elems * elem_bytes / bytes_per_s;
  out[0] = t_f;
  out[1] = t_lv;
  out[2] = t_ring;
  out[3] = t_f > t_lv ? t_f : t_lv;
  out[4] = t_f > t_ring ? t_f : t_ring;
  return out[3] <= out[4] ? 0 : 1;
}
