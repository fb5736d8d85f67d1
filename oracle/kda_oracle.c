/*
 * Plain CPU oracle for the Kimi Delta Attention (KDA) forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code with the HIP library.
 *
 * Everything is computed token by token, in fp64.  q, k and v are taken as
 * fp64 (an exact upcast of fp32 or bf16 values, or the fp64 output of the
 * short convolution below); the gate inputs are fp32.  No chunking, no
 * blocking, no fusion.
 *
 * Sources (the pages give the interface; the recurrence is the KDA definition):
 *  - call contract of chunk_kda (q, k, v, gate, beta, a_log, dt_bias, scale,
 *    lower_bound, initial_state, output_final_state, in-kernel q/k L2 norm,
 *    in-kernel gate, in-kernel beta sigmoid): hyper_parallel coverage page for
 *    context_parallel/kimi_delta_attention.py, `_run_local_kda` and the
 *    `chunk_kda` call inside `_eager_kda_state_p2p`;
 *  - tensor shapes q,k [B,T,H,K], v [B,T,HV,V], gate [B,T,HV,K], beta [B,T,HV],
 *    a_log HV values, dt_bias HV*K values: same page, `_validate_projected_inputs`;
 *  - fp32 recurrent state of shape (B, HV, K, V): same page,
 *    `_RecvKDAInitialState.forward` and the state_shape built in
 *    `_eager_kda_state_p2p`;
 *  - affine state summary (state_ext, transition) and its application to an
 *    optional initial state: same page, `_eager_kda_state_p2p`
 *    (torch_kda_state_summary / torch_apply_kda_state_summary);
 *  - document resets through cu_seqlens: NeMo AutoModel page
 *    "nemo_automodel.components.models.kimi_k3.cp", module introduction and
 *    `doc_ids_from_cu_seqlens` / `segment_cu_seqlens`;
 *  - two gate activations (unbounded and lower-bounded): torchtitan PR #4025
 *    "[kimi k3] add eager reference model with FSDP2", the follow-up commit
 *    note on chunk_kda with the gate activation fused into the kernel.
 *
 * Definition (per sequence n and head h, state S of shape K x V, row = key
 * channel, column = value channel):
 *     q^ = q / sqrt(sum q^2 + 1e-6),  k^ likewise
 *     g_c = -exp(a_log[h]) * softplus(gate_c + dt_bias[h,c])          (no bound)
 *     g_c = lb * sigmoid(exp(a_log[h]) * (gate_c + dt_bias[h,c]))     (bound lb<0)
 *     beta = sigmoid(beta_logit)
 *     S_t  = (I - beta k^ k^T) Diag(exp g) S_{t-1} + beta k^ v^T
 *     o_t  = scale * S_t^T q^
 * The gate formula is not printed on the pages; the two forms above are the
 * reading this oracle takes.  A third, alternative reading of the bound (a hard
 * clamp max(lb, -exp(a_log) softplus(.))) is available as gate mode 2.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_EPS 1e-6

enum { GATE_SOFTPLUS = 0, GATE_SIGMOID_BOUND = 1, GATE_CLAMP_BOUND = 2 };

static double softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* L2 normalisation of one head vector (in-kernel q/k norm). */
static void l2norm(const double* x, int n, double* out) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double r = 1.0 / sqrt(ss + ORACLE_EPS);
  for (int i = 0; i < n; ++i) out[i] = x[i] * r;
}

/* Per-key-channel log-decay built from the raw gate logits (in-kernel gate). */
static void gate_row(const double* gate, const double* dt_bias_h, double a_log_h, int K, int mode,
                     double lb, double* g) {
  double A = exp(a_log_h);
  for (int c = 0; c < K; ++c) {
    double x = (double)gate[c] + (double)dt_bias_h[c];
    if (mode == GATE_SOFTPLUS) {
      g[c] = -A * softplus(x);
    } else if (mode == GATE_SIGMOID_BOUND) {
      g[c] = lb * sigmoid(A * x);
    } else {
      g[c] = fmax(lb, -A * softplus(x));
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Public: prologue only (q^, k^, g, beta) for every token and head.         */
/* ------------------------------------------------------------------------ */
int oracle_prologue(int B, int T, int H, int K, const double* q, const double* k, const double* gate,
                    const double* beta, const double* a_log, const double* dt_bias, int gate_mode,
                    double lower_bound, double* qn, double* kn, double* g, double* b) {
  if (B < 0 || T < 0 || H <= 0 || K <= 0) return 1;
  for (long bt = 0; bt < (long)B * T; ++bt) {
    for (int h = 0; h < H; ++h) {
      long th = bt * H + h;
      l2norm(q + th * K, K, qn + th * K);
      l2norm(k + th * K, K, kn + th * K);
      gate_row(gate + th * K, dt_bias + (long)h * K, (double)a_log[h], K, gate_mode, lower_bound,
               g + th * K);
      b[th] = sigmoid((double)beta[th]);
    }
  }
  return 0;
}

/* One token of the recurrence on state S (K x V, row-major). */
static void recur_step(double* S, int K, int V, const double* qn, const double* kn, const double* g,
                       double bt, const double* v, double scale, double* u, double* o_out) {
  /* S <- Diag(exp g) S */
  for (int c = 0; c < K; ++c) {
    double d = exp(g[c]);
    double* row = S + (long)c * V;
    for (int j = 0; j < V; ++j) row[j] *= d;
  }
  /* u = S^T k^  (the value the state currently predicts for k^) */
  for (int j = 0; j < V; ++j) u[j] = 0.0;
  for (int c = 0; c < K; ++c) {
    const double* row = S + (long)c * V;
    for (int j = 0; j < V; ++j) u[j] += row[j] * kn[c];
  }
  /* S <- S + beta k^ (v - u)^T, which equals (I - beta k^ k^T) S + beta k^ v^T */
  for (int c = 0; c < K; ++c) {
    double* row = S + (long)c * V;
    double bk = bt * kn[c];
    for (int j = 0; j < V; ++j) row[j] += bk * (v[j] - u[j]);
  }
  /* o = scale * S^T q^ */
  if (o_out) {
    for (int j = 0; j < V; ++j) o_out[j] = 0.0;
    for (int c = 0; c < K; ++c) {
      const double* row = S + (long)c * V;
      for (int j = 0; j < V; ++j) o_out[j] += row[j] * qn[c];
    }
    for (int j = 0; j < V; ++j) o_out[j] *= scale;
  }
}

/* ------------------------------------------------------------------------ */
/* Threaded driver over independent (sequence, head) pairs.                 */
/* ------------------------------------------------------------------------ */
typedef struct {
  int B, T, H, K, V;
  int HK; /* key heads of q and k (raw entries); value head h reads key head h / (H / HK) */
  const double *q, *k, *v;
  const double *gate, *beta, *a_log, *dt_bias;
  /* pre-normalised inputs (recurrence-only entry); NULL when raw is used */
  const double *qn, *kn, *g, *bb;
  int gate_mode;
  double lb, scale;
  int N;
  const int32_t* cu;
  const double* init;
  double* o;
  double* fin;
  double* trans; /* summary mode: transition [N,H,K,K] */
  int summary;
  int next; /* work counter */
  pthread_mutex_t mu;
} job_t;

static int take(job_t* J) {
  pthread_mutex_lock(&J->mu);
  int w = J->next++;
  pthread_mutex_unlock(&J->mu);
  return w;
}

static void seq_range(const job_t* J, int n, long* row, long* t0, long* t1) {
  if (J->cu) {
    *row = 0;
    *t0 = J->cu[n];
    *t1 = J->cu[n + 1];
  } else {
    *row = n;
    *t0 = 0;
    *t1 = J->T;
  }
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  int K = J->K, V = J->V, H = J->H;
  double* S = (double*)malloc(sizeof(double) * (size_t)K * V);
  double* P = J->summary ? (double*)malloc(sizeof(double) * (size_t)K * K) : NULL;
  double* u = (double*)malloc(sizeof(double) * (size_t)(K > V ? K : V));
  double* qn = (double*)malloc(sizeof(double) * K);
  double* kn = (double*)malloc(sizeof(double) * K);
  double* g = (double*)malloc(sizeof(double) * K);
  double* zeros = (double*)calloc((size_t)(K > V ? K : V), sizeof(double));
  for (;;) {
    int w = take(J);
    if (w >= J->N * H) break;
    int n = w / H, h = w % H;
    long row, t0, t1;
    seq_range(J, n, &row, &t0, &t1);
    long sidx = ((long)n * H + h) * (long)K * V;
    for (long i = 0; i < (long)K * V; ++i) S[i] = J->init ? (double)J->init[sidx + i] : 0.0;
    if (P) {
      for (int i = 0; i < K; ++i)
        for (int j = 0; j < K; ++j) P[(long)i * K + j] = (i == j) ? 1.0 : 0.0;
    }
    for (long t = t0; t < t1; ++t) {
      long th = ((row * J->T) + t) * H + h;
      const double *pq, *pk, *pg;
      double bt;
      if (J->qn) {
        pq = J->qn + th * K;
        pk = J->kn + th * K;
        pg = J->g + th * K;
        bt = J->bb[th];
      } else {
        /* grouped value heads: G = H / HK value heads share one key head */
        long thk = ((row * J->T) + t) * J->HK + h / (H / J->HK);
        l2norm(J->q + thk * K, K, qn);
        l2norm(J->k + thk * K, K, kn);
        gate_row(J->gate + th * K, J->dt_bias + (long)h * K, (double)J->a_log[h], K, J->gate_mode,
                 J->lb, g);
        bt = sigmoid((double)J->beta[th]);
        pq = qn;
        pk = kn;
        pg = g;
      }
      recur_step(S, K, V, pq, pk, pg, bt, J->v + th * V, J->scale, u,
                 J->o ? J->o + th * V : NULL);
      if (P) /* the same factor applied to the transition, with zero values */
        recur_step(P, K, K, pq, pk, pg, bt, zeros, 0.0, u, NULL);
    }
    if (J->fin)
      for (long i = 0; i < (long)K * V; ++i) J->fin[sidx + i] = S[i];
    if (P) {
      long pidx = ((long)n * H + h) * (long)K * K;
      memcpy(J->trans + pidx, P, sizeof(double) * (size_t)K * K);
    }
  }
  free(S);
  free(P);
  free(u);
  free(qn);
  free(kn);
  free(g);
  free(zeros);
  return NULL;
}

static int run_job(job_t* J, int threads) {
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  pthread_mutex_init(&J->mu, NULL);
  J->next = 0;
  pthread_t tid[256];
  int started = 0;
  for (int i = 1; i < threads; ++i)
    if (pthread_create(&tid[started], NULL, worker, J) == 0) ++started;
  worker(J);
  for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
  pthread_mutex_destroy(&J->mu);
  return 0;
}

static int check_cu(int B, int T, int N, const int32_t* cu) {
  if (!cu) return N == B ? 0 : 2;
  if (B != 1 || cu[0] != 0 || cu[N] != T) return 2;
  for (int n = 0; n < N; ++n)
    if (cu[n + 1] < cu[n]) return 2;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Public: full forward from raw inputs.                                     */
/*   H value heads, HK key heads (H % HK == 0; HK == H without grouping):   */
/*   q, k [B,T,HK,K]; v [B,T,H,V]; gate [B,T,H,K]; beta [B,T,H];             */
/*   a_log [H], dt_bias [H,K]; o [B,T,H,V] (may be NULL), final_state        */
/*   [N,H,K,V] (may be NULL).                                                */
/* ------------------------------------------------------------------------ */
int oracle_kda_fwd(int B, int T, int H, int HK, int K, int V, const double* q, const double* k,
                   const double* v, const double* gate, const double* beta, const double* a_log,
                   const double* dt_bias, double scale, int gate_mode, double lower_bound, int N,
                   const int32_t* cu_seqlens, const double* initial_state, double* o,
                   double* final_state, int threads) {
  if (B < 0 || T < 0 || H <= 0 || HK <= 0 || H % HK || K <= 0 || V <= 0) return 1;
  if (check_cu(B, T, N, cu_seqlens)) return 2;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.B = B; J.T = T; J.H = H; J.HK = HK; J.K = K; J.V = V;
  J.q = q; J.k = k; J.v = v; J.gate = gate; J.beta = beta; J.a_log = a_log; J.dt_bias = dt_bias;
  J.gate_mode = gate_mode; J.lb = lower_bound; J.scale = scale;
  J.N = N; J.cu = cu_seqlens; J.init = initial_state; J.o = o; J.fin = final_state;
  return run_job(&J, threads);
}

/* ------------------------------------------------------------------------ */
/* Public: recurrence only, from already normalised q^, k^, log-decay g and  */
/* beta (all [B,T,H,*] fp64).  v is fp64, initial_state fp32 as above.      */
/* ------------------------------------------------------------------------ */
int oracle_recurrence(int B, int T, int H, int K, int V, const double* qn, const double* kn,
                      const double* v, const double* g, const double* b, double scale, int N,
                      const int32_t* cu_seqlens, const double* initial_state, double* o,
                      double* final_state, int threads) {
  if (B < 0 || T < 0 || H <= 0 || K <= 0 || V <= 0) return 1;
  if (check_cu(B, T, N, cu_seqlens)) return 2;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.B = B; J.T = T; J.H = H; J.K = K; J.V = V;
  J.qn = qn; J.kn = kn; J.g = g; J.bb = b; J.v = v; J.scale = scale;
  J.N = N; J.cu = cu_seqlens; J.init = initial_state; J.o = o; J.fin = final_state;
  return run_job(&J, threads);
}

/* ------------------------------------------------------------------------ */
/* Public: affine state summary of each row (no document resets).           */
/*   state_ext  [B,H,K,V] = final state of the row started from zero        */
/*   transition [B,H,K,K] = ordered product of the per-token factors        */
/*                          (I - beta k^ k^T) Diag(exp g), later on the left */
/* so that final_state = transition . initial_state + state_ext.            */
/* ------------------------------------------------------------------------ */
int oracle_state_summary(int B, int T, int H, int HK, int K, int V, const double* q,
                         const double* k, const double* v, const double* gate, const double* beta,
                         const double* a_log, const double* dt_bias, int gate_mode,
                         double lower_bound, double* state_ext, double* transition, int threads) {
  if (B < 0 || T < 0 || H <= 0 || HK <= 0 || H % HK || K <= 0 || V <= 0) return 1;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.B = B; J.T = T; J.H = H; J.HK = HK; J.K = K; J.V = V;
  J.q = q; J.k = k; J.v = v; J.gate = gate; J.beta = beta; J.a_log = a_log; J.dt_bias = dt_bias;
  J.gate_mode = gate_mode; J.lb = lower_bound; J.scale = 1.0;
  J.N = B; J.fin = state_ext; J.trans = transition; J.summary = 1;
  return run_job(&J, threads);
}

/* ------------------------------------------------------------------------ */
/* Public: the causal depthwise short convolution and SiLU applied to q, k  */
/* and v before the recurrence (the ShortConv of the Kimi layer: depthwise   */
/* conv1d, stride 1, dilation 1, zero padding of W-1 tokens on the left,     */
/* output cut to the sequence length, then SiLU; without the convolution the */
/* layer applies SiLU alone).  Source: hyper_parallel coverage page,         */
/* `_run_causal_short_conv`, `_validate_layer_short_conv` and the forward of */
/* KimiDeltaAttentionUlyssesCP.                                             */
/*   x, y [B,T,C] fp64 (C channels, e.g. H*K), w [C,W] (tap W-1 weights the */
/*   current token, tap 0 the token W-1 steps back), bias [C] or NULL.      */
/*   y[t,c] = silu(bias[c] + sum_j w[c,j] * x[t-(W-1)+j, c]),               */
/*   silu(z) = z * sigmoid(z).                                              */
/* Tokens before the first token of t's sequence count as zero: with        */
/* cu_seqlens every document is padded on its own (the pages pad each row;  */
/* a packed row holds independent documents, so the padding is taken per     */
/* document).  W = 0: y = silu(x).                                          */
/* ------------------------------------------------------------------------ */
int oracle_short_conv_silu(int B, int T, int C, int W, const double* x, const double* w,
                           const double* bias, int N, const int32_t* cu_seqlens, double* y) {
  if (B < 0 || T < 0 || C <= 0 || W < 0 || (W > 0 && !w)) return 1;
  if (check_cu(B, T, N, cu_seqlens)) return 2;
  for (int n = 0; n < N; ++n) {
    const long row = cu_seqlens ? 0 : n;
    const long t0 = cu_seqlens ? cu_seqlens[n] : 0;
    const long t1 = cu_seqlens ? cu_seqlens[n + 1] : T;
    for (long t = t0; t < t1; ++t)
      for (int c = 0; c < C; ++c) {
        double z;
        if (W == 0) {
          z = x[(row * T + t) * C + c];
        } else {
          z = bias ? bias[c] : 0.0;
          for (int j = 0; j < W; ++j) {
            const long s = t - (W - 1) + j; /* input token of tap j */
            if (s >= t0) z += w[(long)c * W + j] * x[(row * T + s) * C + c];
          }
        }
        y[(row * T + t) * C + c] = z * sigmoid(z);
      }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Public: gradients of the forward (reverse mode, token by token).         */
/*   The forward is the definition above; the loss is                       */
/*     L = sum(d_o * o) + sum(d_final * final_state)                         */
/*   and every input's gradient is dL/d(input), through the in-kernel L2     */
/*   norm, gate and beta sigmoid.  Source for what is differentiated: the    */
/*   pages test chunk_kda forward and backward together (torchtitan PR      */
/*   #4025 commit note) and route state gradients between slices            */
/*   (hyper_parallel page, the backward of _RecvKDAInitialState); the        */
/*   derivative itself is the chain rule applied to the definition.          */
/* Per (sequence, value head): a forward pass that keeps every state, then   */
/* a reverse pass.  With S' = Diag(e^g) S_prev, u = S'^T k^, e = v - u,     */
/* S = S' + beta k^ e^T and o = scale S^T q^, for the incoming dS:           */
/*   dS += scale q^ do^T;  dq^ = scale S do;  dbeta = k^T dS e;             */
/*   de = beta dS^T k^ (= dv);  dk^ = beta dS e - S' de;                    */
/*   dS' = dS - k^ de^T;  dg_c = sum_j dS'_cj S'_cj;  dS_prev = Diag(e^g) dS' */
/* Outputs: dq, dk [B,T,HK,K] (summed over the value heads of a group); dv   */
/* [B,T,H,V]; dgate [B,T,H,K]; dbeta [B,T,H] (of the logit); da_log [H],     */
/* ddt_bias [H,K] (summed over tokens); dinit [N,H,K,V] (may be NULL).       */
/* d_final may be NULL (zero).                                               */
/* ------------------------------------------------------------------------ */
typedef struct {
  job_t f;               /* forward description (raw inputs) */
  const double* d_o;
  const double* d_fin;
  double *dqh, *dkh;     /* [B,T,H,K] per value head, reduced over groups after */
  double *dv, *dgate, *dbeta;
  double *da_part, *ddt_part; /* [N,H], [N,H,K] */
  double* dinit;
  int oom;
} bwd_job_t;

/* gradient of one L2-normalised row: x^ = x / sqrt(sum x^2 + eps) */
static void l2norm_bwd(const double* x, const double* dxh, int n, double* dx) {
  double ss = 0.0, dot = 0.0;
  for (int i = 0; i < n; ++i) {
    ss += x[i] * x[i];
    dot += x[i] * dxh[i];
  }
  const double nr = sqrt(ss + ORACLE_EPS);
  for (int i = 0; i < n; ++i) dx[i] = dxh[i] / nr - x[i] * dot / (nr * nr * nr);
}

/* dg/dx and dg/da_log of one gate entry (x = gate + dt_bias) */
static void gate_grad(double x, double a_log_h, int mode, double lb, double* dgdx, double* dgda) {
  const double A = exp(a_log_h);
  if (mode == GATE_SIGMOID_BOUND) {
    const double s = sigmoid(A * x);
    *dgdx = lb * s * (1.0 - s) * A;
    *dgda = lb * s * (1.0 - s) * A * x;
    return;
  }
  const double g = -A * softplus(x);
  if (mode == GATE_CLAMP_BOUND && !(g > lb)) {
    *dgdx = 0.0;
    *dgda = 0.0;
    return;
  }
  *dgdx = -A * sigmoid(x);
  *dgda = g;
}

static void* bwd_worker(void* arg) {
  bwd_job_t* BJ = (bwd_job_t*)arg;
  job_t* J = &BJ->f;
  const int K = J->K, V = J->V, H = J->H;
  for (;;) {
    int w = take(J);
    if (w >= J->N * H) break;
    const int n = w / H, h = w % H;
    long row, t0, t1;
    seq_range(J, n, &row, &t0, &t1);
    const long L = t1 - t0;
    const long KV = (long)K * V;
    double* S = (double*)malloc(sizeof(double) * (size_t)(L + 1) * KV);  /* S[0] = entering state */
    double* qn = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * K);
    double* kn = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * K);
    double* g = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * K);
    double* bt = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    double* dS = (double*)malloc(sizeof(double) * KV);
    double* Sd = (double*)malloc(sizeof(double) * KV);
    double* u = (double*)malloc(sizeof(double) * (K > V ? K : V));
    double* e = (double*)malloc(sizeof(double) * V);
    double* de = (double*)malloc(sizeof(double) * V);
    double* dqh = (double*)malloc(sizeof(double) * K);
    double* dkh = (double*)malloc(sizeof(double) * K);
    double* dg = (double*)malloc(sizeof(double) * K);
    if (!S || !qn || !kn || !g || !bt || !dS || !Sd || !u || !e || !de || !dqh || !dkh || !dg) {
      BJ->oom = 1;
      free(S); free(qn); free(kn); free(g); free(bt); free(dS); free(Sd); free(u); free(e);
      free(de); free(dqh); free(dkh); free(dg);
      continue;
    }
    const long sidx = ((long)n * H + h) * KV;
    for (long i = 0; i < KV; ++i) S[i] = J->init ? J->init[sidx + i] : 0.0;
    const int G = H / J->HK;
    /* forward, keeping every state */
    for (long t = t0; t < t1; ++t) {
      const long l = t - t0;
      const long th = ((row * J->T) + t) * H + h;
      const long thk = ((row * J->T) + t) * J->HK + h / G;
      l2norm(J->q + thk * K, K, qn + l * K);
      l2norm(J->k + thk * K, K, kn + l * K);
      gate_row(J->gate + th * K, J->dt_bias + (long)h * K, J->a_log[h], K, J->gate_mode, J->lb,
               g + l * K);
      bt[l] = sigmoid(J->beta[th]);
      memcpy(S + (l + 1) * KV, S + l * KV, sizeof(double) * KV);
      recur_step(S + (l + 1) * KV, K, V, qn + l * K, kn + l * K, g + l * K, bt[l], J->v + th * V,
                 J->scale, u, NULL);
    }
    /* reverse */
    for (long i = 0; i < KV; ++i) dS[i] = BJ->d_fin ? BJ->d_fin[sidx + i] : 0.0;
    double da = 0.0;
    double* ddt = BJ->ddt_part + ((long)n * H + h) * K;
    for (int c = 0; c < K; ++c) ddt[c] = 0.0;
    for (long t = t1 - 1; t >= t0; --t) {
      const long l = t - t0;
      const long th = ((row * J->T) + t) * H + h;
      const double* St = S + (l + 1) * KV;
      const double* Sp = S + l * KV;
      const double* q_ = qn + l * K;
      const double* k_ = kn + l * K;
      const double* g_ = g + l * K;
      const double b_ = bt[l];
      const double* do_ = BJ->d_o + th * V;
      const double* v_ = J->v + th * V;
      /* recompute S' = Diag(e^g) S_prev, u = S'^T k^, e = v - u */
      for (int c = 0; c < K; ++c) {
        const double d = exp(g_[c]);
        for (int j = 0; j < V; ++j) Sd[(long)c * V + j] = d * Sp[(long)c * V + j];
      }
      for (int j = 0; j < V; ++j) {
        double acc = 0.0;
        for (int c = 0; c < K; ++c) acc += Sd[(long)c * V + j] * k_[c];
        u[j] = acc;
        e[j] = v_[j] - acc;
      }
      /* output */
      for (int c = 0; c < K; ++c) {
        double acc = 0.0;
        for (int j = 0; j < V; ++j) {
          dS[(long)c * V + j] += J->scale * q_[c] * do_[j];
          acc += St[(long)c * V + j] * do_[j];
        }
        dqh[c] = J->scale * acc;
      }
      /* update S = S' + beta k^ e^T */
      double dbeta = 0.0;
      for (int j = 0; j < V; ++j) {
        double acc = 0.0;
        for (int c = 0; c < K; ++c) acc += dS[(long)c * V + j] * k_[c];
        de[j] = b_ * acc;
        dbeta += acc * e[j];
      }
      for (int c = 0; c < K; ++c) {
        double acc = 0.0, acc2 = 0.0;
        for (int j = 0; j < V; ++j) {
          acc += dS[(long)c * V + j] * e[j];
          acc2 += Sd[(long)c * V + j] * de[j];
        }
        dkh[c] = b_ * acc - acc2;  /* through e (directly) and through u = S'^T k^ */
      }
      /* dS' = dS - k^ de^T, the decay's gradient, and dS_prev */
      for (int c = 0; c < K; ++c) {
        const double d = exp(g_[c]);
        double acc = 0.0;
        for (int j = 0; j < V; ++j) {
          const double dsd = dS[(long)c * V + j] - k_[c] * de[j];
          acc += dsd * Sd[(long)c * V + j];
          dS[(long)c * V + j] = d * dsd;
        }
        dg[c] = acc;
      }
      for (int j = 0; j < V; ++j) BJ->dv[th * V + j] = de[j];
      BJ->dbeta[th] = dbeta * b_ * (1.0 - b_);
      /* raw q, k through the L2 norm (per value head; groups are summed later) */
      const long thk = ((row * J->T) + t) * J->HK + h / G;
      l2norm_bwd(J->q + thk * K, dqh, K, BJ->dqh + th * K);
      l2norm_bwd(J->k + thk * K, dkh, K, BJ->dkh + th * K);
      /* gate */
      for (int c = 0; c < K; ++c) {
        double dgdx, dgda;
        gate_grad(J->gate[th * K + c] + J->dt_bias[(long)h * K + c], J->a_log[h], J->gate_mode,
                  J->lb, &dgdx, &dgda);
        BJ->dgate[th * K + c] = dg[c] * dgdx;
        ddt[c] += dg[c] * dgdx;
        da += dg[c] * dgda;
      }
    }
    BJ->da_part[(long)n * H + h] = da;
    if (BJ->dinit)
      for (long i = 0; i < KV; ++i) BJ->dinit[sidx + i] = dS[i];
    free(S); free(qn); free(kn); free(g); free(bt); free(dS); free(Sd); free(u); free(e);
    free(de); free(dqh); free(dkh); free(dg);
  }
  return NULL;
}

int oracle_kda_bwd(int B, int T, int H, int HK, int K, int V, const double* q, const double* k,
                   const double* v, const double* gate, const double* beta, const double* a_log,
                   const double* dt_bias, double scale, int gate_mode, double lower_bound, int N,
                   const int32_t* cu_seqlens, const double* initial_state, const double* d_o,
                   const double* d_final, double* dq, double* dk, double* dv, double* dgate,
                   double* dbeta, double* da_log, double* ddt_bias, double* dinit, int threads) {
  if (B < 0 || T < 0 || H <= 0 || HK <= 0 || H % HK || K <= 0 || V <= 0) return 1;
  if (check_cu(B, T, N, cu_seqlens)) return 2;
  bwd_job_t BJ;
  memset(&BJ, 0, sizeof(BJ));
  job_t* J = &BJ.f;
  J->B = B; J->T = T; J->H = H; J->HK = HK; J->K = K; J->V = V;
  J->q = q; J->k = k; J->v = v; J->gate = gate; J->beta = beta; J->a_log = a_log;
  J->dt_bias = dt_bias; J->gate_mode = gate_mode; J->lb = lower_bound; J->scale = scale;
  J->N = N; J->cu = cu_seqlens; J->init = initial_state;
  BJ.d_o = d_o; BJ.d_fin = d_final; BJ.dv = dv; BJ.dgate = dgate; BJ.dbeta = dbeta;
  BJ.dinit = dinit;
  const size_t tokh = (size_t)B * T * H;
  BJ.dqh = (double*)calloc(tokh * K + 1, sizeof(double));
  BJ.dkh = (double*)calloc(tokh * K + 1, sizeof(double));
  BJ.da_part = (double*)calloc((size_t)N * H + 1, sizeof(double));
  BJ.ddt_part = (double*)calloc((size_t)N * H * K + 1, sizeof(double));
  if (!BJ.dqh || !BJ.dkh || !BJ.da_part || !BJ.ddt_part) {
    free(BJ.dqh); free(BJ.dkh); free(BJ.da_part); free(BJ.ddt_part);
    return 3;
  }
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  pthread_mutex_init(&J->mu, NULL);
  J->next = 0;
  pthread_t tid[256];
  int started = 0;
  for (int i = 1; i < threads; ++i)
    if (pthread_create(&tid[started], NULL, bwd_worker, &BJ) == 0) ++started;
  bwd_worker(&BJ);
  for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
  pthread_mutex_destroy(&J->mu);
  /* group sums for the key heads, sums over sequences for the gate parameters */
  const int G = H / HK;
  for (long bt = 0; bt < (long)B * T; ++bt)
    for (int hk = 0; hk < HK; ++hk)
      for (int c = 0; c < K; ++c) {
        double sq = 0.0, sk = 0.0;
        for (int gi = 0; gi < G; ++gi) {
          const long th = bt * H + (long)hk * G + gi;
          sq += BJ.dqh[th * K + c];
          sk += BJ.dkh[th * K + c];
        }
        dq[(bt * HK + hk) * K + c] = sq;
        dk[(bt * HK + hk) * K + c] = sk;
      }
  for (int h = 0; h < H; ++h) {
    double a = 0.0;
    for (int n = 0; n < N; ++n) a += BJ.da_part[(long)n * H + h];
    da_log[h] = a;
    for (int c = 0; c < K; ++c) {
      double d = 0.0;
      for (int n = 0; n < N; ++n) d += BJ.ddt_part[((long)n * H + h) * K + c];
      ddt_bias[(long)h * K + c] = d;
    }
  }
  const int oom = BJ.oom;
  free(BJ.dqh); free(BJ.dkh); free(BJ.da_part); free(BJ.ddt_part);
  return oom ? 3 : 0;
}

/* ------------------------------------------------------------------------ */
/* Public: the gated output norm after the forward, o_norm(o, output_gate)  */
/* of the layer (hyper_parallel coverage page, the forward of               */
/* KimiDeltaAttentionUlyssesCP: the output gate projection reshaped to      */
/* [B, T, HV, V], then o_norm(output, output_gate) per value head; the       */
/* torchtitan PR #4025 review names the model's RMSNorm with its reduction   */
/* in fp32).  The pages do not print the norm; the reading taken here is a   */
/* gated RMSNorm over the head's V values:                                  */
/*   y[v] = o[v] / sqrt(mean_v(o^2) + eps) * weight[v] * act(gate[v])        */
/* with act = sigmoid (act_mode 0) or SiLU x*sigmoid(x) (act_mode 1).        */
/*   o, gate, y [R, V] fp64 (R = rows = tokens x heads); weight [V] or NULL. */
/* ------------------------------------------------------------------------ */
int oracle_gated_rms_norm(long R, int V, const double* o, const double* gate,
                          const double* weight, double eps, int act_mode, double* y) {
  if (R < 0 || V <= 0 || (act_mode != 0 && act_mode != 1)) return 1;
  for (long r = 0; r < R; ++r) {
    const double* x = o + r * V;
    double ss = 0.0;
    for (int v = 0; v < V; ++v) ss += x[v] * x[v];
    const double inv = 1.0 / sqrt(ss / V + eps);
    for (int v = 0; v < V; ++v) {
      const double g = gate[r * V + v];
      const double a = act_mode == 0 ? sigmoid(g) : g * sigmoid(g);
      y[r * V + v] = x[v] * inv * (weight ? weight[v] : 1.0) * a;
    }
  }
  return 0;
}

/* Public: final = transition . initial + state_ext (initial may be NULL). */
int oracle_apply_state_summary(int B, int H, int K, int V, const double* state_ext,
                               const double* transition, const double* initial_state,
                               double* final_state) {
  for (long bh = 0; bh < (long)B * H; ++bh) {
    const double* E = state_ext + bh * K * V;
    const double* P = transition + bh * K * K;
    const double* S0 = initial_state ? initial_state + bh * K * V : NULL;
    double* F = final_state + bh * K * V;
    for (int i = 0; i < K; ++i)
      for (int j = 0; j < V; ++j) {
        double acc = E[(long)i * V + j];
        if (S0)
          for (int c = 0; c < K; ++c) acc += P[(long)i * K + c] * S0[(long)c * V + j];
        F[(long)i * V + j] = acc;
      }
  }
  return 0;
}
