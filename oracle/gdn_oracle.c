/*
 * gdn_oracle.c -- CPU oracle for the varlen chunked Gated Delta Rule prefill.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or helper with the
 * HIP path.
 *
 * Everything is plain fp64 C, written from the pages' definitions:
 *
 *  - Token recurrence (weigao.cc "GDN 与 Chunked Prefill", sections
 *    "GDN 是什么" and "64-token chunk 里的计算形态变化": the gate multiplies the
 *    whole previous state, the output reads the state after the update;
 *    gitcode "FlashInfer GDN Prefill 完全指南", section "API 全参数解析": g is
 *    the forget gate alpha, beta the update gate, both default to ones, scale
 *    defaults to 1/sqrt(head_size), state layout [N, H, V, K], optional
 *    in-kernel q/k L2 normalisation with epsilon 1e-6, cu_seqlens with
 *    repeated offsets meaning empty sequences, state_indices pool,
 *    checkpoints every n tokens):
 *
 *        S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *        o_t = scale * S_t^T q_t
 *
 *    with S a dk x dv matrix.  0539edu "GDN与线性注意力GPU并行实现" section 1.2
 *    prints a variant with alpha inside the rank-one term; the pages' other
 *    two sources (and the forget-gate meaning of g) settle on the form above.
 *
 *  - Chunk table (weigao.cc, section "chunked prefill 有两层含义"): every
 *    sequence is cut into ceil(len/64) chunks, listed sequence-major,
 *    chunk-minor.
 *
 *  - Checkpoint starts (gitcode, section "中间状态检查点"): the exclusive
 *    prefix sum of floor(len_i / n).
 *
 *  - Chunked form, any chunk size C (weigao.cc sections "递推公式如何展开成块内
 *    计算" and "块内 state 和块间 final state"; 0539edu sections 2.2 and 3.3):
 *    the recurrence rewritten per chunk as a unit-lower-triangular solve
 *    followed by matrix products; only the chunk's last state crosses to the
 *    next chunk.  Its derivation from the token recurrence is spelled out at
 *    oracle_gdn_chunked() below.  It is a second, independent form of the same
 *    definition: the tests check the two against each other and against exact
 *    rational arithmetic.
 *
 * Readings of the pages that this file takes (all listed with their reasons in
 * the design notes): the recurrence form above; outputs read the updated
 * state; g is alpha itself (not its log); stored state element [v][k] is
 * S[k][v]; q/k head for sab head h is h / (H / h_src); L2 norm is
 * x / sqrt(sum x^2 + 1e-6); checkpoint j of a sequence is the state after j*n
 * of its tokens, stored at row cu_starts[i] + j - 1; an empty sequence's final
 * state is its initial state.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int64_t T;          /* total tokens */
  int32_t N;          /* sequences */
  int32_t hq, hk, hv; /* head counts of q, k, v */
  int32_t D;          /* head size (dk = dv = D) */
  const double *q, *k, *v;  /* [T][hq][D], [T][hk][D], [T][hv][D] */
  const double *g, *beta;   /* [T][H] or NULL (all ones) */
  int32_t has_scale;
  double scale;
  const int64_t *cu;        /* [N+1] */
  int32_t l2norm;
  const double *init_state; /* [rows][H][D][D], element [v][k]; NULL = zero */
  const int64_t *state_indices; /* [N] or NULL */
  int64_t state_rows;       /* rows of init_state (pool size) */
  int64_t ckpt_every;       /* 0 = off */
  const int64_t *ckpt_cu_starts; /* [N+1] or NULL */
  const int32_t *heads;     /* subset of sab heads to compute, or NULL = all */
  int32_t n_heads;
} oracle_problem;

static int32_t sab_heads(const oracle_problem *p) {
  return p->hq > p->hv ? p->hq : p->hv;
}

/* Chunk table: returns the number of chunks, or -1 if cap is too small. */
int64_t oracle_chunk_table(const int64_t *cu, int32_t n_seqs, int32_t chunk,
                           int32_t *table, int64_t cap, int32_t *cu_chunks) {
  int64_t f = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    int64_t len = cu[i + 1] - cu[i];
    int64_t nc = len > 0 ? (len + chunk - 1) / chunk : 0;
    if (cu_chunks) cu_chunks[i] = (int32_t)f;
    for (int64_t c = 0; c < nc; ++c, ++f) {
      if (f >= cap) return -1;
      table[2 * f] = i;
      table[2 * f + 1] = (int32_t)c;
    }
  }
  if (cu_chunks) cu_chunks[n_seqs] = (int32_t)f;
  return f;
}

void oracle_checkpoint_starts(const int64_t *cu, int32_t n_seqs, int64_t every,
                              int64_t *out) {
  int64_t acc = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    out[i] = acc;
    int64_t len = cu[i + 1] - cu[i];
    if (every > 0 && len > 0) acc += len / every;
  }
  out[n_seqs] = acc;
}

/* Load one token's vector for sab head h from x[T][hx][D], optionally
 * L2-normalised. */
static void load_vec(const double *x, int64_t t, int32_t hx, int32_t H,
                     int32_t h, int32_t D, int32_t norm, double *dst) {
  int32_t src = h / (H / hx);
  const double *row = x + ((size_t)t * hx + src) * D;
  if (!norm) {
    memcpy(dst, row, sizeof(double) * D);
    return;
  }
  double ss = 0.0;
  for (int32_t a = 0; a < D; ++a) ss += row[a] * row[a];
  double inv = 1.0 / sqrt(ss + 1e-6);
  for (int32_t a = 0; a < D; ++a) dst[a] = row[a] * inv;
}

static int64_t state_row_of(const oracle_problem *p, int32_t i) {
  if (p->state_indices) return p->state_indices[i];
  return i;
}

/* S[a][b] (a over keys, b over values) from the stored [v][k] layout. */
static void load_state(const oracle_problem *p, int32_t i, int32_t h,
                       double *S) {
  int32_t H = sab_heads(p), D = p->D;
  memset(S, 0, sizeof(double) * D * D);
  if (!p->init_state) return;
  int64_t row = state_row_of(p, i);
  if (row < 0 || row >= p->state_rows) return;
  const double *src = p->init_state + ((size_t)row * H + h) * D * D;
  for (int32_t b = 0; b < D; ++b)
    for (int32_t a = 0; a < D; ++a) S[a * D + b] = src[b * D + a];
}

static void store_state(const double *S, int32_t D, double *dst) {
  for (int32_t b = 0; b < D; ++b)
    for (int32_t a = 0; a < D; ++a) dst[b * D + a] = S[a * D + b];
}

static double scale_of(const oracle_problem *p) {
  return p->has_scale ? p->scale : 1.0 / sqrt((double)p->D);
}

/*
 * Token recurrence.  out: [T][H][D]; final_state: [N][H][D][D] ([v][k]),
 * per sequence (the caller maps it onto a pool); checkpoints: [rows][H][D][D].
 * Only heads in p->heads (or all) are written.
 */
int oracle_gdn_token(const oracle_problem *p, double *out, double *final_state,
                     double *checkpoints) {
  const int32_t H = sab_heads(p), D = p->D;
  const int32_t nh = p->heads ? p->n_heads : H;
  const double sc = scale_of(p);
  const int64_t items = (int64_t)p->N * nh;
#pragma omp parallel
  {
    double *S = (double *)malloc(sizeof(double) * D * D);
    double *qv = (double *)malloc(sizeof(double) * D);
    double *kv = (double *)malloc(sizeof(double) * D);
    double *vv = (double *)malloc(sizeof(double) * D);
    double *kS = (double *)malloc(sizeof(double) * D);
#pragma omp for schedule(dynamic, 1)
    for (int64_t it = 0; it < items; ++it) {
      int32_t i = (int32_t)(it / nh);
      int32_t h = p->heads ? p->heads[it % nh] : (int32_t)(it % nh);
      load_state(p, i, h, S);
      int64_t bos = p->cu[i], eos = p->cu[i + 1];
      for (int64_t t = bos; t < eos; ++t) {
        double alpha = p->g ? p->g[t * H + h] : 1.0;
        double beta = p->beta ? p->beta[t * H + h] : 1.0;
        load_vec(p->q, t, p->hq, H, h, D, p->l2norm, qv);
        load_vec(p->k, t, p->hk, H, h, D, p->l2norm, kv);
        load_vec(p->v, t, p->hv, H, h, D, 0, vv);
        /* kS = k^T S (a row vector over values) */
        for (int32_t b = 0; b < D; ++b) {
          double s = 0.0;
          for (int32_t a = 0; a < D; ++a) s += kv[a] * S[a * D + b];
          kS[b] = s;
        }
        /* S <- alpha (S - beta k (k^T S)) + beta k v^T */
        for (int32_t a = 0; a < D; ++a)
          for (int32_t b = 0; b < D; ++b)
            S[a * D + b] = alpha * (S[a * D + b] - beta * kv[a] * kS[b]) +
                           beta * kv[a] * vv[b];
        /* o_t = scale S^T q */
        if (out) {
          double *o = out + ((size_t)t * H + h) * D;
          for (int32_t b = 0; b < D; ++b) {
            double s = 0.0;
            for (int32_t a = 0; a < D; ++a) s += S[a * D + b] * qv[a];
            o[b] = sc * s;
          }
        }
        int64_t done = t - bos + 1;
        if (checkpoints && p->ckpt_every > 0 && done % p->ckpt_every == 0) {
          int64_t row = p->ckpt_cu_starts[i] + done / p->ckpt_every - 1;
          store_state(S, D, checkpoints + ((size_t)row * H + h) * D * D);
        }
      }
      if (final_state)
        store_state(S, D, final_state + ((size_t)i * H + h) * D * D);
    }
    free(S); free(qv); free(kv); free(vv); free(kS);
  }
  return 0;
}

/*
 * Chunked form with chunk size C >= 1.  Derivation, for one chunk with rows
 * t = 1..n (n <= C), start state S0, gamma_t = alpha_1 ... alpha_t:
 *
 *   Write nu_t = beta_t (v_t - alpha_t S_{t-1}^T k_t).  Then the recurrence is
 *   S_t = alpha_t S_{t-1} + k_t nu_t^T, which unrolls (the weigao.cc 4-token
 *   table with u_j = k_j nu_j^T) to
 *       S_t = gamma_t S0 + sum_{j<=t} (gamma_t/gamma_j) k_j nu_j^T.
 *   Putting this S_{t-1} into nu_t gives, for the matrix N with rows nu_t,
 *       (I + A) N = diag(beta) V - diag(beta*gamma) K S0,
 *       A[t][j] = beta_t (gamma_t/gamma_j) (k_t . k_j)  for j < t, else 0,
 *   so with T = (I + A)^{-1} (unit lower triangular, by forward substitution)
 *       W = T diag(beta*gamma) K,  U = T diag(beta) V,  N = U - W S0,
 *       O = scale (diag(gamma) Q S0 + (Q K^T .* M) N),
 *           M[t][j] = gamma_t/gamma_j for j <= t, else 0,
 *       S_end = gamma_n S0 + (diag(gamma_n/gamma) K)^T N.
 *   Ratios gamma_t/gamma_j are formed as exp(G_t - G_j), G = cumulative sum
 *   of log alpha.
 *
 * chunk_states (optional): [n_chunks][H][D][D] ([v][k]) state at the start of
 * every chunk, flat chunks in oracle_chunk_table() order.  vnew (optional):
 * [T][H][D], the rows nu_t.
 */
int oracle_gdn_chunked(const oracle_problem *p, int32_t C, double *out,
                       double *final_state, double *checkpoints,
                       double *chunk_states, double *vnew) {
  const int32_t H = sab_heads(p), D = p->D;
  const int32_t nh = p->heads ? p->n_heads : H;
  const double sc = scale_of(p);
  const int64_t items = (int64_t)p->N * nh;
  if (C < 1) return -1;
  if (checkpoints && p->ckpt_every > 0 && p->ckpt_every % C != 0) return -2;
  /* flat chunk offsets per sequence */
  int64_t *cstart = (int64_t *)malloc(sizeof(int64_t) * (p->N + 1));
  cstart[0] = 0;
  for (int32_t i = 0; i < p->N; ++i) {
    int64_t len = p->cu[i + 1] - p->cu[i];
    cstart[i + 1] = cstart[i] + (len > 0 ? (len + C - 1) / C : 0);
  }
#pragma omp parallel
  {
    double *S = (double *)malloc(sizeof(double) * D * D);
    double *Q = (double *)malloc(sizeof(double) * C * D);
    double *K = (double *)malloc(sizeof(double) * C * D);
    double *V = (double *)malloc(sizeof(double) * C * D);
    double *G = (double *)malloc(sizeof(double) * C);
    double *B = (double *)malloc(sizeof(double) * C);
    double *A = (double *)malloc(sizeof(double) * C * C);
    double *Tm = (double *)malloc(sizeof(double) * C * C);
    double *W = (double *)malloc(sizeof(double) * C * D);
    double *U = (double *)malloc(sizeof(double) * C * D);
    double *Nm = (double *)malloc(sizeof(double) * C * D);
    double *P = (double *)malloc(sizeof(double) * C * C);
    double *S2 = (double *)malloc(sizeof(double) * D * D);
#pragma omp for schedule(dynamic, 1)
    for (int64_t it = 0; it < items; ++it) {
      int32_t i = (int32_t)(it / nh);
      int32_t h = p->heads ? p->heads[it % nh] : (int32_t)(it % nh);
      load_state(p, i, h, S);
      int64_t bos = p->cu[i], eos = p->cu[i + 1];
      int64_t ci = 0;
      for (int64_t c0 = bos; c0 < eos; c0 += C, ++ci) {
        int32_t n = (int32_t)((eos - c0) < C ? (eos - c0) : C);
        if (chunk_states)
          store_state(S, D,
                      chunk_states + ((size_t)(cstart[i] + ci) * H + h) * D * D);
        double run = 0.0;
        for (int32_t t = 0; t < n; ++t) {
          int64_t tok = c0 + t;
          load_vec(p->q, tok, p->hq, H, h, D, p->l2norm, Q + t * D);
          load_vec(p->k, tok, p->hk, H, h, D, p->l2norm, K + t * D);
          load_vec(p->v, tok, p->hv, H, h, D, 0, V + t * D);
          double alpha = p->g ? p->g[tok * H + h] : 1.0;
          run += log(alpha);
          G[t] = run;
          B[t] = p->beta ? p->beta[tok * H + h] : 1.0;
        }
        /* A (strictly lower) */
        for (int32_t t = 0; t < n; ++t)
          for (int32_t j = 0; j < n; ++j) {
            double a = 0.0;
            if (j < t) {
              double kk = 0.0;
              for (int32_t x = 0; x < D; ++x) kk += K[t * D + x] * K[j * D + x];
              a = B[t] * exp(G[t] - G[j]) * kk;
            }
            A[t * C + j] = a;
          }
        /* T = (I + A)^{-1} by forward substitution, column by column:
         * T[t][j] = delta_tj - sum_{m<t} A[t][m] T[m][j]. */
        for (int32_t j = 0; j < n; ++j)
          for (int32_t t = 0; t < n; ++t) {
            double s = (t == j) ? 1.0 : 0.0;
            for (int32_t m = 0; m < t; ++m) s -= A[t * C + m] * Tm[m * C + j];
            Tm[t * C + j] = s;
          }
        /* W = T diag(beta*gamma) K, U = T diag(beta) V */
        for (int32_t t = 0; t < n; ++t)
          for (int32_t x = 0; x < D; ++x) {
            double w = 0.0, u = 0.0;
            for (int32_t j = 0; j < n; ++j) {
              w += Tm[t * C + j] * B[j] * exp(G[j]) * K[j * D + x];
              u += Tm[t * C + j] * B[j] * V[j * D + x];
            }
            W[t * D + x] = w;
            U[t * D + x] = u;
          }
        /* N = U - W S0 */
        for (int32_t t = 0; t < n; ++t)
          for (int32_t b = 0; b < D; ++b) {
            double s = 0.0;
            for (int32_t a = 0; a < D; ++a) s += W[t * D + a] * S[a * D + b];
            Nm[t * D + b] = U[t * D + b] - s;
          }
        if (vnew)
          for (int32_t t = 0; t < n; ++t)
            memcpy(vnew + ((size_t)(c0 + t) * H + h) * D, Nm + t * D,
                   sizeof(double) * D);
        /* P = (Q K^T) .* M */
        for (int32_t t = 0; t < n; ++t)
          for (int32_t j = 0; j < n; ++j) {
            double s = 0.0;
            if (j <= t) {
              for (int32_t x = 0; x < D; ++x) s += Q[t * D + x] * K[j * D + x];
              s *= exp(G[t] - G[j]);
            }
            P[t * C + j] = s;
          }
        /* O = scale (diag(gamma) Q S0 + P N) */
        if (out)
          for (int32_t t = 0; t < n; ++t) {
            double *o = out + ((size_t)(c0 + t) * H + h) * D;
            double gt = exp(G[t]);
            for (int32_t b = 0; b < D; ++b) {
              double s1 = 0.0, s2 = 0.0;
              for (int32_t a = 0; a < D; ++a) s1 += Q[t * D + a] * S[a * D + b];
              for (int32_t j = 0; j <= t; ++j) s2 += P[t * C + j] * Nm[j * D + b];
              o[b] = sc * (gt * s1 + s2);
            }
          }
        /* S_end = gamma_n S0 + (diag(gamma_n/gamma) K)^T N */
        double gn = exp(G[n - 1]);
        for (int32_t a = 0; a < D; ++a)
          for (int32_t b = 0; b < D; ++b) {
            double s = 0.0;
            for (int32_t j = 0; j < n; ++j)
              s += exp(G[n - 1] - G[j]) * K[j * D + a] * Nm[j * D + b];
            S2[a * D + b] = gn * S[a * D + b] + s;
          }
        memcpy(S, S2, sizeof(double) * D * D);
        int64_t done = c0 + n - bos;
        /* a checkpoint falls inside this chunk only at its end when C divides
         * the checkpoint interval; other positions are handled by the token
         * form, so the chunked form requires ckpt_every % C == 0. */
        if (checkpoints && p->ckpt_every > 0 && done % p->ckpt_every == 0) {
          int64_t row = p->ckpt_cu_starts[i] + done / p->ckpt_every - 1;
          store_state(S, D, checkpoints + ((size_t)row * H + h) * D * D);
        }
      }
      if (final_state)
        store_state(S, D, final_state + ((size_t)i * H + h) * D * D);
    }
    free(S); free(Q); free(K); free(V); free(G); free(B); free(A); free(Tm);
    free(W); free(U); free(Nm); free(P); free(S2);
  }
  free(cstart);
  return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

int oracle_abi_version(void) { return 1; }
