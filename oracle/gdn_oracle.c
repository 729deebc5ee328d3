/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the Gated DeltaNet token-mixer
 * hot path.  TEST INFRASTRUCTURE ONLY: it is loaded by the tests, by the
 * smoke check and by the CPU-baseline leg of the benchmark, never by the
 * product path.  It shares no code, header or constant with the HIP library.
 *
 * Every routine is the plain definition of the step it covers, written out
 * token by token, with no blocking or fusion:
 *
 *   oracle_localize        -- flash-linear-attention "fla/ops/cp/context.py",
 *                             get_cp_cu_seqlens (steps 2-5 of its comments).
 *   oracle_conv1d_silu     -- hyper-parallel "linear_attention_context_parallel.py",
 *                             _causal_conv1d_with_cp_halo: causal depthwise
 *                             conv1d (cross-correlation, padding K-1 on the
 *                             left, or the previous shard's K-1 pre-conv
 *                             tokens) followed by SiLU.
 *   oracle_gdn_fwd         -- same page, _l2norm_torch + the gated delta rule
 *                             that _prepare_gdn_chunks_for_summary /
 *                             _run_prepared_gdn_chunks evaluate chunk-wise,
 *                             here as the token recurrence it is equal to:
 *                               S <- exp(g_t) S
 *                               u  = beta_t (v_t - S^T k_t)
 *                               S <- S + k_t u^T
 *                               o_t = S^T q_t
 *                             with the state laid out [dk, dv] as in the
 *                             page's recurrent_state.
 *   oracle_gdn_bwd         -- hand-written reverse mode of oracle_gdn_fwd,
 *                             l2norm included (the P2P send/recv autograd
 *                             functions on the same page fix the state
 *                             gradient contract: dh0 flows back, dht in).
 *   oracle_conv1d_silu_bwd -- reverse mode of oracle_conv1d_silu, with the
 *                             halo gradient the differentiable halo
 *                             all-to-all returns to the previous shard.
 *   oracle_gating_fwd      -- the gating lines of the same page's CP
 *                             wrappers (LinearAttentionP2PCPWrapper.forward
 *                             and its siblings): per token and value head
 *                               beta = sigmoid(b)
 *                               g    = -exp(A_log) * softplus(a + dt_bias)
 *   oracle_gating_bwd      -- its reverse mode (da, db, dA_log, ddt_bias).
 *
 * Layouts (row-major): x,y [T,C]; w [C,K]; halo [K-1,C]; q,k [T,Hk,dk];
 * v,o [T,Hv,dv]; g,beta [T,Hv]; states [N,Hv,dk,dv].  Varlen batches are
 * described by cu_seqlens[N+1]; sequences never mix.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define L2NORM_EPS 1e-6

/* ---------------------------------------------------------------------- */
/* Localisation: fla "context.py", get_cp_cu_seqlens.                      */
/* ---------------------------------------------------------------------- */

/* First index i in a[0..n) with a[i] > v (torch.searchsorted side='right'). */
static int64_t search_right(const int64_t *a, int64_t n, int64_t v) {
  int64_t i = 0;
  while (i < n && a[i] <= v) i++;
  return i;
}

/* First index i in a[0..n) with a[i] >= v (torch.searchsorted side='left'). */
static int64_t search_left(const int64_t *a, int64_t n, int64_t v) {
  int64_t i = 0;
  while (i < n && a[i] < v) i++;
  return i;
}

/* floor division for the non-negative operands the algorithm produces, and
 * Python's floor for a negative numerator (last_seq_global_end - 1 can be -1
 * only when total is 0, which is rejected before). */
static int64_t floordiv(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) q -= 1;
  return q;
}

/*
 * meta[0..9] = rank_start, rank_end, num_local_seqs, first_seq_global_idx,
 *              is_first_rank, is_last_rank, pre_num_ranks, post_num_ranks,
 *              pre_num_conv_tokens, n_halo
 * local_cu receives num_local_seqs+1 entries (capacity num_seqs+1).
 * Returns 0, or -1 when the split is undefined (world_size < 1, rank out of
 * range, total not divisible by world_size, or an empty part).
 */
int oracle_localize(const int64_t *cu, int64_t num_seqs, int64_t world_size, int64_t rank,
                    int64_t conv_k, int64_t *local_cu, int64_t *meta) {
  if (world_size < 1 || rank < 0 || rank >= world_size || num_seqs < 1) return -1;
  int64_t total = cu[num_seqs];
  if (total % world_size != 0) return -1;
  int64_t part_len = total / world_size;
  if (part_len <= 0) return -1;
  int64_t rank_start = part_len * rank;
  int64_t rank_end = rank_start + part_len;

  /* the ends are cu[1..num_seqs], the starts cu[0..num_seqs-1] */
  int64_t start_seq_idx = search_right(cu + 1, num_seqs, rank_start);
  int64_t end_seq_idx = search_left(cu, num_seqs, rank_end);

  /* slice [start_seq_idx, end_seq_idx], clamp, rebase, drop repeats */
  int64_t n_out = 0;
  for (int64_t i = start_seq_idx; i <= end_seq_idx; i++) {
    int64_t c = cu[i];
    if (c < rank_start) c = rank_start;
    if (c > rank_end) c = rank_end;
    c -= rank_start;
    if (n_out == 0 || local_cu[n_out - 1] != c) local_cu[n_out++] = c;
  }

  int64_t first_seq_global_start = cu[start_seq_idx];
  int64_t last_seq_global_end = cu[end_seq_idx];
  int64_t pre_num_conv_tokens = rank_start - first_seq_global_start;
  if (pre_num_conv_tokens < 0) pre_num_conv_tokens = 0;
  int64_t first_rank = floordiv(first_seq_global_start, part_len);
  int64_t last_rank = floordiv(last_seq_global_end - 1, part_len);

  int64_t halo_rows = conv_k > 1 ? conv_k - 1 : 0;
  meta[0] = rank_start;
  meta[1] = rank_end;
  meta[2] = n_out - 1;
  meta[3] = start_seq_idx;
  meta[4] = (rank == first_rank);
  meta[5] = (rank == last_rank);
  meta[6] = rank - first_rank;
  meta[7] = last_rank - rank;
  meta[8] = pre_num_conv_tokens;
  meta[9] = pre_num_conv_tokens < halo_rows ? pre_num_conv_tokens : halo_rows;
  return 0;
}

/* ---------------------------------------------------------------------- */
/* Causal depthwise conv1d + SiLU with a carried-in halo.                  */
/* ---------------------------------------------------------------------- */

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* The padded input x~ seen by token tau of sequence n (which starts at s):
 * its own tokens; for n == 0 the last n_halo halo rows; zero otherwise. */
static double xtilde(const double *x, const double *halo, int64_t n_halo, int64_t n, int64_t s,
                     int64_t tau, int64_t c, int64_t C, int64_t K) {
  if (tau >= s) return x[tau * C + c];
  int64_t back = s - tau; /* 1 = the token just before the sequence start */
  if (n == 0 && halo != NULL && back <= n_halo) return halo[(K - 1 - back) * C + c];
  return 0.0;
}

void oracle_conv1d_silu(const double *x, const double *w, const double *bias, const double *halo,
                        int64_t n_halo, const int64_t *cu, int64_t N, int64_t T, int64_t C, int64_t K,
                        double *y, double *z_out) {
  (void)T;
  /* every output element is independent: the tokens of a sequence are shared
   * among the threads (rows stay contiguous in memory) */
  for (int64_t n = 0; n < N; n++) {
    int64_t s = cu[n], e = cu[n + 1];
#pragma omp parallel for schedule(static)
    for (int64_t t = s; t < e; t++) {
      for (int64_t c = 0; c < C; c++) {
        double z = bias ? bias[c] : 0.0;
        for (int64_t j = 0; j < K; j++)
          z += w[c * K + j] * xtilde(x, halo, n_halo, n, s, t - (K - 1) + j, c, C, K);
        if (z_out) z_out[t * C + c] = z;
        y[t * C + c] = z * sigmoid(z);
      }
    }
  }
}

/* dw [C,K], dbias [C] (nullable), dhalo [K-1,C] (nullable) are overwritten;
 * dx [T,C] is overwritten. */
void oracle_conv1d_silu_bwd(const double *x, const double *w, const double *bias, const double *halo,
                            int64_t n_halo, const int64_t *cu, int64_t N, int64_t T, int64_t C,
                            int64_t K, const double *dy, double *dx, double *dw, double *dbias,
                            double *dhalo) {
  memset(dx, 0, sizeof(double) * (size_t)(T * C));
  memset(dw, 0, sizeof(double) * (size_t)(C * K));
  if (dbias) memset(dbias, 0, sizeof(double) * (size_t)C);
  if (dhalo && K > 1) memset(dhalo, 0, sizeof(double) * (size_t)((K - 1) * C));
  /* channels are independent (each writes its own column of dx, dhalo and
   * its own dw row): they are shared among the threads */
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < C; c++) {
  for (int64_t n = 0; n < N; n++) {
    int64_t s = cu[n], e = cu[n + 1];
    for (int64_t t = s; t < e; t++) {
      {
        double z = bias ? bias[c] : 0.0;
        for (int64_t j = 0; j < K; j++)
          z += w[c * K + j] * xtilde(x, halo, n_halo, n, s, t - (K - 1) + j, c, C, K);
        double sg = sigmoid(z);
        double dz = dy[t * C + c] * sg * (1.0 + z * (1.0 - sg));
        if (dbias) dbias[c] += dz;
        for (int64_t j = 0; j < K; j++) {
          int64_t tau = t - (K - 1) + j;
          dw[c * K + j] += dz * xtilde(x, halo, n_halo, n, s, tau, c, C, K);
          if (tau >= s) {
            dx[tau * C + c] += w[c * K + j] * dz;
          } else {
            int64_t back = s - tau;
            if (n == 0 && halo != NULL && back <= n_halo && dhalo)
              dhalo[(K - 1 - back) * C + c] += w[c * K + j] * dz;
          }
        }
      }
    }
  }
  }
}

/* ---------------------------------------------------------------------- */
/* l2norm (hyper-parallel page, _l2norm_torch): x * rsqrt(sum x^2 + eps).  */
/* ---------------------------------------------------------------------- */

static void l2norm_fwd(const double *x, int64_t d, double mult, int use, double *out, double *r_out) {
  double r = 1.0;
  if (use) {
    double ss = 0.0;
    for (int64_t i = 0; i < d; i++) ss += x[i] * x[i];
    r = 1.0 / sqrt(ss + L2NORM_EPS);
  }
  for (int64_t i = 0; i < d; i++) out[i] = mult * x[i] * r;
  if (r_out) *r_out = r;
}

/* out = mult * x * r(x) ; returns dx given dout. */
static void l2norm_bwd(const double *x, int64_t d, double mult, int use, const double *dout, double *dx) {
  if (!use) {
    for (int64_t i = 0; i < d; i++) dx[i] = mult * dout[i];
    return;
  }
  double ss = 0.0, xd = 0.0;
  for (int64_t i = 0; i < d; i++) {
    ss += x[i] * x[i];
    xd += x[i] * dout[i];
  }
  double r = 1.0 / sqrt(ss + L2NORM_EPS);
  for (int64_t i = 0; i < d; i++) dx[i] = mult * r * (dout[i] - x[i] * r * r * xd);
}

/* ---------------------------------------------------------------------- */
/* Gated delta rule, token recurrence.                                     */
/* ---------------------------------------------------------------------- */

/* One token step on S [dk,dv]: decay, delta update, readout.
 * qh, kh are the normalised (and for q, scaled) vectors. */
static void token_step(double *S, const double *qh, const double *kh, const double *v, double g,
                       double beta, int64_t dk, int64_t dv, double *u, double *o) {
  double a = exp(g);
  for (int64_t i = 0; i < dk * dv; i++) S[i] *= a;
  for (int64_t j = 0; j < dv; j++) {
    double p = 0.0;
    for (int64_t i = 0; i < dk; i++) p += S[i * dv + j] * kh[i];
    u[j] = beta * (v[j] - p);
  }
  for (int64_t i = 0; i < dk; i++)
    for (int64_t j = 0; j < dv; j++) S[i * dv + j] += kh[i] * u[j];
  if (o) {
    for (int64_t j = 0; j < dv; j++) {
      double acc = 0.0;
      for (int64_t i = 0; i < dk; i++) acc += S[i * dv + j] * qh[i];
      o[j] = acc;
    }
  }
}

/* Runs every (sequence, v-head) pair; v-head h reads q/k head h / (Hv/Hk),
 * the repeat_interleave mapping of the page's GQA expansion.  h0 may be
 * NULL (zero initial state); ht may be NULL. */
void oracle_gdn_fwd(const double *q, const double *k, const double *v, const double *g,
                    const double *beta, const double *h0, const int64_t *cu, int64_t N, int64_t T,
                    int64_t Hk, int64_t Hv, int64_t dk, int64_t dv, double scale, int use_l2norm,
                    double *o, double *ht, int nthreads) {
  (void)T;
  int64_t grp = Hv / Hk;
  int64_t units = N * Hv;
#ifdef _OPENMP
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t unit = 0; unit < units; unit++) {
    int64_t n = unit / Hv, h = unit % Hv, a = h / grp;
    double *S = (double *)malloc(sizeof(double) * (size_t)(dk * dv));
    double *qh = (double *)malloc(sizeof(double) * (size_t)dk);
    double *kh = (double *)malloc(sizeof(double) * (size_t)dk);
    double *u = (double *)malloc(sizeof(double) * (size_t)dv);
    if (h0)
      memcpy(S, h0 + (n * Hv + h) * dk * dv, sizeof(double) * (size_t)(dk * dv));
    else
      memset(S, 0, sizeof(double) * (size_t)(dk * dv));
    for (int64_t t = cu[n]; t < cu[n + 1]; t++) {
      l2norm_fwd(q + (t * Hk + a) * dk, dk, scale, use_l2norm, qh, NULL);
      l2norm_fwd(k + (t * Hk + a) * dk, dk, 1.0, use_l2norm, kh, NULL);
      token_step(S, qh, kh, v + (t * Hv + h) * dv, g[t * Hv + h], beta[t * Hv + h], dk, dv, u,
                 o + (t * Hv + h) * dv);
    }
    if (ht) memcpy(ht + (n * Hv + h) * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
    free(S);
    free(qh);
    free(kh);
    free(u);
  }
}

/*
 * Reverse mode of oracle_gdn_fwd.  Outputs (overwritten):
 *   dq, dk_ [T,Hk,d]  gradients w.r.t. the raw q, k (before l2norm/scale),
 *                     summed over the v-heads that share a q/k head;
 *   dv_ [T,Hv,dv], dg, dbeta [T,Hv], dh0 [N,Hv,dk,dv] (nullable).
 * do_ [T,Hv,dv]; dht [N,Hv,dk,dv] nullable (zero).
 * States S_{t-1} are recovered from checkpoints every CKPT tokens and a
 * forward re-run inside each block, so memory stays bounded.
 */
#define CKPT 64
void oracle_gdn_bwd(const double *q, const double *k, const double *v, const double *g,
                    const double *beta, const double *h0, const int64_t *cu, int64_t N, int64_t T,
                    int64_t Hk, int64_t Hv, int64_t dk, int64_t dv, double scale, int use_l2norm,
                    const double *do_, const double *dht, double *dq, double *dk_, double *dv_,
                    double *dg, double *dbeta, double *dh0, int nthreads) {
  int64_t grp = Hv / Hk;
  int64_t dd = dk * dv;
  memset(dq, 0, sizeof(double) * (size_t)(T * Hk * dk));
  memset(dk_, 0, sizeof(double) * (size_t)(T * Hk * dk));
  memset(dv_, 0, sizeof(double) * (size_t)(T * Hv * dv));
  memset(dg, 0, sizeof(double) * (size_t)(T * Hv));
  memset(dbeta, 0, sizeof(double) * (size_t)(T * Hv));
  int64_t units = N * Hk; /* one unit owns a q/k head and all its v-heads */
#ifdef _OPENMP
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t unit = 0; unit < units; unit++) {
    int64_t n = unit / Hk, a = unit % Hk;
    int64_t s = cu[n], e = cu[n + 1], len = e - s;
    int64_t nblk = (len + CKPT - 1) / CKPT;
    double *ck = (double *)malloc(sizeof(double) * (size_t)((nblk + 1) * dd));
    double *st = (double *)malloc(sizeof(double) * (size_t)((CKPT + 1) * dd));
    double *dS = (double *)malloc(sizeof(double) * (size_t)dd);
    double *dSt = (double *)malloc(sizeof(double) * (size_t)dd);
    double *qh = (double *)malloc(sizeof(double) * (size_t)dk);
    double *kh = (double *)malloc(sizeof(double) * (size_t)dk);
    double *u = (double *)malloc(sizeof(double) * (size_t)dv);
    double *p = (double *)malloc(sizeof(double) * (size_t)dv);
    double *du = (double *)malloc(sizeof(double) * (size_t)dv);
    double *dqh = (double *)malloc(sizeof(double) * (size_t)(len * dk + 1));
    double *dkh = (double *)malloc(sizeof(double) * (size_t)(len * dk + 1));
    double *tmp = (double *)malloc(sizeof(double) * (size_t)dk);
    memset(dqh, 0, sizeof(double) * (size_t)(len * dk + 1));
    memset(dkh, 0, sizeof(double) * (size_t)(len * dk + 1));
    for (int64_t h = a * grp; h < (a + 1) * grp; h++) {
      /* forward pass storing a checkpoint before every block */
      double *S = st;
      if (h0)
        memcpy(S, h0 + (n * Hv + h) * dd, sizeof(double) * (size_t)dd);
      else
        memset(S, 0, sizeof(double) * (size_t)dd);
      for (int64_t b = 0; b < nblk; b++) {
        memcpy(ck + b * dd, S, sizeof(double) * (size_t)dd);
        for (int64_t t = s + b * CKPT; t < s + (b + 1) * CKPT && t < e; t++) {
          l2norm_fwd(k + (t * Hk + a) * dk, dk, 1.0, use_l2norm, kh, NULL);
          token_step(S, NULL, kh, v + (t * Hv + h) * dv, g[t * Hv + h], beta[t * Hv + h], dk, dv,
                     u, NULL);
        }
      }
      /* reverse pass */
      if (dht)
        memcpy(dS, dht + (n * Hv + h) * dd, sizeof(double) * (size_t)dd);
      else
        memset(dS, 0, sizeof(double) * (size_t)dd);
      for (int64_t b = nblk - 1; b >= 0; b--) {
        int64_t t0 = s + b * CKPT, t1 = t0 + CKPT < e ? t0 + CKPT : e;
        /* st[i] = state before token t0+i ; st[t1-t0] = after the block */
        memcpy(st, ck + b * dd, sizeof(double) * (size_t)dd);
        for (int64_t t = t0; t < t1; t++) {
          double *Sn = st + (t - t0 + 1) * dd;
          memcpy(Sn, st + (t - t0) * dd, sizeof(double) * (size_t)dd);
          l2norm_fwd(k + (t * Hk + a) * dk, dk, 1.0, use_l2norm, kh, NULL);
          token_step(Sn, NULL, kh, v + (t * Hv + h) * dv, g[t * Hv + h], beta[t * Hv + h], dk,
                     dv, u, NULL);
        }
        for (int64_t t = t1 - 1; t >= t0; t--) {
          const double *Sprev = st + (t - t0) * dd; /* S_{t-1} */
          const double *Scur = st + (t - t0 + 1) * dd; /* S_t */
          const double *vt = v + (t * Hv + h) * dv;
          const double *dot = do_ + (t * Hv + h) * dv;
          double gt = g[t * Hv + h], bt = beta[t * Hv + h], ea = exp(gt);
          l2norm_fwd(q + (t * Hk + a) * dk, dk, scale, use_l2norm, qh, NULL);
          l2norm_fwd(k + (t * Hk + a) * dk, dk, 1.0, use_l2norm, kh, NULL);
          /* o_t = S_t^T qh */
          for (int64_t i = 0; i < dk; i++) {
            double acc = 0.0;
            for (int64_t j = 0; j < dv; j++) {
              dS[i * dv + j] += qh[i] * dot[j];
              acc += Scur[i * dv + j] * dot[j];
            }
            dqh[(t - s) * dk + i] += acc;
          }
          /* p = (e^g S_{t-1})^T kh ; u = beta (v - p) */
          for (int64_t j = 0; j < dv; j++) {
            double acc = 0.0;
            for (int64_t i = 0; i < dk; i++) acc += ea * Sprev[i * dv + j] * kh[i];
            p[j] = acc;
            u[j] = bt * (vt[j] - acc);
          }
          /* S_t = St~ + kh u^T */
          for (int64_t j = 0; j < dv; j++) {
            double acc = 0.0;
            for (int64_t i = 0; i < dk; i++) acc += dS[i * dv + j] * kh[i];
            du[j] = acc;
          }
          for (int64_t i = 0; i < dk; i++) {
            double acc = 0.0;
            for (int64_t j = 0; j < dv; j++) acc += dS[i * dv + j] * u[j];
            tmp[i] = acc;
          }
          double db = 0.0;
          for (int64_t j = 0; j < dv; j++) {
            dv_[(t * Hv + h) * dv + j] = bt * du[j];
            db += du[j] * (vt[j] - p[j]);
          }
          dbeta[t * Hv + h] = db;
          /* dp = -beta du ; dSt~ = dS + kh dp^T ; dkh += St~ dp */
          for (int64_t i = 0; i < dk; i++) {
            double acc = 0.0;
            for (int64_t j = 0; j < dv; j++) {
              double dp = -bt * du[j];
              dSt[i * dv + j] = dS[i * dv + j] + kh[i] * dp;
              acc += ea * Sprev[i * dv + j] * dp;
            }
            dkh[(t - s) * dk + i] += tmp[i] + acc;
          }
          /* St~ = e^g S_{t-1}: dg = <dSt~, St~>, dS_{t-1} = e^g dSt~ */
          double dgt = 0.0;
          for (int64_t i = 0; i < dd; i++) {
            dgt += dSt[i] * ea * Sprev[i];
            dS[i] = ea * dSt[i];
          }
          dg[t * Hv + h] = dgt;
        }
      }
      if (dh0) memcpy(dh0 + (n * Hv + h) * dd, dS, sizeof(double) * (size_t)dd);
    }
    /* back through l2norm and the q scale, once per q/k head */
    for (int64_t t = s; t < e; t++) {
      l2norm_bwd(q + (t * Hk + a) * dk, dk, scale, use_l2norm, dqh + (t - s) * dk,
                 dq + (t * Hk + a) * dk);
      l2norm_bwd(k + (t * Hk + a) * dk, dk, 1.0, use_l2norm, dkh + (t - s) * dk,
                 dk_ + (t * Hk + a) * dk);
    }
    free(ck);
    free(st);
    free(dS);
    free(dSt);
    free(qh);
    free(kh);
    free(u);
    free(p);
    free(du);
    free(dqh);
    free(dkh);
    free(tmp);
  }
}

/* ---------------------------------------------------------------------- */
/* Gating (hyper-parallel page, the CP wrappers' forward):                 */
/*   beta = sigmoid(b),  g = -exp(A_log) * softplus(a + dt_bias)           */
/* a, b [T, Hv] with token stride ld; A_log, dt_bias [Hv]; g, beta [T, Hv]. */
/* ---------------------------------------------------------------------- */

/* log(1 + e^x) without overflow: for x > 0 it is x + log(1 + e^-x). */
static double softplus(double x) { return x > 0 ? x + log1p(exp(-x)) : log1p(exp(x)); }

void oracle_gating_fwd(const double *a, const double *b, int64_t ld, const double *A_log,
                       const double *dt_bias, int64_t T, int64_t Hv, double *g, double *beta) {
  for (int64_t t = 0; t < T; t++)
    for (int64_t h = 0; h < Hv; h++) {
      beta[t * Hv + h] = sigmoid(b[t * ld + h]);
      g[t * Hv + h] = -exp(A_log[h]) * softplus(a[t * ld + h] + dt_bias[h]);
    }
}

/* d softplus(x) / dx = sigmoid(x); d g / d A_log = g.  da, db [T, Hv] (token
 * stride ld_d) and dA_log, ddt_bias [Hv] are overwritten; the per-head sums
 * run over the tokens in order. */
void oracle_gating_bwd(const double *a, const double *b, int64_t ld, const double *A_log,
                       const double *dt_bias, const double *dg, const double *dbeta, int64_t T,
                       int64_t Hv, double *da, double *db, int64_t ld_d, double *dA_log,
                       double *ddt_bias) {
  for (int64_t h = 0; h < Hv; h++) {
    dA_log[h] = 0.0;
    ddt_bias[h] = 0.0;
  }
  for (int64_t t = 0; t < T; t++)
    for (int64_t h = 0; h < Hv; h++) {
      double sb = sigmoid(b[t * ld + h]);
      double x = a[t * ld + h] + dt_bias[h];
      double e = exp(A_log[h]);
      double gv = -e * softplus(x);
      double dgv = dg[t * Hv + h];
      db[t * ld_d + h] = dbeta[t * Hv + h] * sb * (1.0 - sb);
      double dx = dgv * (-e) * sigmoid(x);
      da[t * ld_d + h] = dx;
      ddt_bias[h] += dx;
      dA_log[h] += dgv * gv;
    }
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
