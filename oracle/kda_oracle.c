/*
 * KDA oracle: the gated delta rule with per-key-channel decay, token by token,
 * in IEEE fp64.  TEST INFRASTRUCTURE ONLY -- the product library never links,
 * loads or calls this file; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg do.
 *
 * What is computed (per sequence n, value head h, token t, with the query/key
 * head hq = h / (Hv / Hqk)):
 *
 *   qn = q / sqrt(sum(q^2) + 1e-6),  kn likewise          (optional L2 norm)
 *   b  = 1 / (1 + exp(-beta_logit))                          (write strength)
 *   S' = diag(exp(g)) S                  (decay acts on the key index of S)
 *   u  = b * (v - S'^T kn)                                   (delta residual)
 *   S  = S' + kn u^T                                         (rank-one write)
 *   o  = scale * S^T qn                (read after this token's write)
 *
 * S is K x V (K = V = 128); states cross the interface "V-first", i.e. the
 * buffer element [v][k] holds S[k][v].
 *
 * Sources:
 *  - the recurrence S_t = (I - b k k^T) diag(exp g) S_{t-1} + b k v^T with
 *    o_t = scale S_t^T q_t is the problem statement of the chunked KDA forward;
 *  - page "vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.verify", class
 *    KdaTcVerify: the L2 norm with eps 1e-6 added to the sum of squares under
 *    the square root, the sigmoid of the raw beta, decay applied to the state
 *    before the key probe, and each output summing the corrections of all
 *    window tokens up to and including itself (the per-row solve step);
 *  - page "mate.kda" (MATE 0.2.5), chunk_kda: default scale 128^-0.5, beta
 *    given as logits, the GVA divisibility rule Hv % Hqk == 0;
 *    gated_delta_rule_decode: the V-first state layout [pool, HV, V, K].
 *
 * The head map hq = h / (Hv / Hqk) (contiguous groups of value heads share a
 * query/key head) is a reading: the pages only require divisibility.
 *
 * Gate parameters (optional): with a per-head A_log and a per-(head, channel)
 * dt_bias, the g input is a raw gate and the log-decay of a step is
 *   lower_bound * sigmoid(exp(A_log[h]) * (g + dt_bias[h][c]))
 * (the activation of KdaTcVerify on page
 * "vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.verify"; chunk_kda of page
 * "mate.kda" takes A_log, dt_bias and lower_bound = -5 by default).
 *
 * Inputs are read at their stored precision (fp32, bf16 or fp16) and widened
 * to fp64 exactly; nothing is rounded before the outputs leave in fp64.
 * Work is spread over (sequence, value head) units with POSIX threads.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KD 128 /* key width */
#define VD 128 /* value width */

enum { OR_F32 = 0, OR_BF16 = 1, OR_F16 = 2 };

static double widen_bf16(uint16_t h) {
  uint32_t bits = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

static double widen_f16(uint16_t h) {
  int sign = (h >> 15) & 1, ex = (h >> 10) & 31, man = h & 1023;
  double val;
  if (ex == 0)
    val = ldexp((double)man, -24);
  else if (ex == 31)
    val = man ? NAN : INFINITY;
  else
    val = ldexp((double)(man | 1024), ex - 25);
  return sign ? -val : val;
}

static double load_elem(const void *p, int dtype, int64_t i) {
  switch (dtype) {
  case OR_F32: return (double)((const float *)p)[i];
  case OR_BF16: return widen_bf16(((const uint16_t *)p)[i]);
  default: return widen_f16(((const uint16_t *)p)[i]);
  }
}

typedef struct {
  int dtype;
  const void *q, *k, *v, *g, *beta;
  const int64_t *cu;
  int num_seqs, hqk, hv, use_l2norm;
  double scale;
  const double *a_log, *dt_bias; /* gate parameters, or NULL */
  double lower_bound;
  const double *s0;
  double *out, *s_final;
  const int *heads;
  int n_heads;
  int next_unit;
  pthread_mutex_t lock;
} job_t;

/* One (sequence, value-head) chain, token by token. */
static void run_unit(job_t *J, int n, int h) {
  static const double eps = 1e-6;
  double *S = (double *)malloc(sizeof(double) * KD * VD); /* S[k][v] */
  double qn[KD], kn[KD], alpha[KD], vv[VD], u[VD];
  const int grp = J->hv / J->hqk;
  const int hq = h / grp;
  if (J->s0) {
    const double *src = J->s0 + ((int64_t)n * J->hv + h) * VD * KD;
    for (int c = 0; c < KD; ++c)
      for (int r = 0; r < VD; ++r) S[c * VD + r] = src[r * KD + c];
  } else {
    memset(S, 0, sizeof(double) * KD * VD);
  }
  for (int64_t t = J->cu[n]; t < J->cu[n + 1]; ++t) {
    const int64_t qoff = (t * J->hqk + hq) * KD;
    const int64_t voff = (t * J->hv + h) * VD;
    double sq = 0.0, sk = 0.0;
    for (int c = 0; c < KD; ++c) {
      qn[c] = load_elem(J->q, J->dtype, qoff + c);
      kn[c] = load_elem(J->k, J->dtype, qoff + c);
      double gl = load_elem(J->g, J->dtype, voff + c);
      if (J->a_log)
        gl = J->lower_bound /
             (1.0 + exp(-exp(J->a_log[h]) * (gl + J->dt_bias[(int64_t)h * KD + c])));
      alpha[c] = exp(gl);
      sq += qn[c] * qn[c];
      sk += kn[c] * kn[c];
    }
    if (J->use_l2norm) {
      const double rq = 1.0 / sqrt(sq + eps), rk = 1.0 / sqrt(sk + eps);
      for (int c = 0; c < KD; ++c) {
        qn[c] *= rq;
        kn[c] *= rk;
      }
    }
    for (int r = 0; r < VD; ++r) vv[r] = load_elem(J->v, J->dtype, voff + r);
    const double b = 1.0 / (1.0 + exp(-load_elem(J->beta, J->dtype, t * J->hv + h)));

    /* S' = diag(alpha) S ; then u = b (v - S'^T kn) */
    for (int r = 0; r < VD; ++r) u[r] = 0.0;
    for (int c = 0; c < KD; ++c) {
      double *row = S + c * VD;
      for (int r = 0; r < VD; ++r) {
        row[r] *= alpha[c];
        u[r] += row[r] * kn[c];
      }
    }
    for (int r = 0; r < VD; ++r) u[r] = b * (vv[r] - u[r]);
    /* S = S' + kn u^T ; o = scale S^T qn */
    double *o = J->out + voff;
    for (int r = 0; r < VD; ++r) o[r] = 0.0;
    for (int c = 0; c < KD; ++c) {
      double *row = S + c * VD;
      for (int r = 0; r < VD; ++r) {
        row[r] += kn[c] * u[r];
        o[r] += row[r] * qn[c];
      }
    }
    for (int r = 0; r < VD; ++r) o[r] *= J->scale;
  }
  if (J->s_final) {
    double *dst = J->s_final + ((int64_t)n * J->hv + h) * VD * KD;
    for (int c = 0; c < KD; ++c)
      for (int r = 0; r < VD; ++r) dst[r * KD + c] = S[c * VD + r];
  }
  free(S);
}

static void *worker(void *arg) {
  job_t *J = (job_t *)arg;
  const int nh = J->heads ? J->n_heads : J->hv;
  const int total = J->num_seqs * nh;
  for (;;) {
    pthread_mutex_lock(&J->lock);
    const int unit = J->next_unit++;
    pthread_mutex_unlock(&J->lock);
    if (unit >= total) break;
    const int n = unit / nh;
    const int h = J->heads ? J->heads[unit % nh] : unit % nh;
    run_unit(J, n, h);
  }
  return NULL;
}

/*
 * Runs the recurrence for every sequence n in [0, num_seqs) (tokens
 * [cu[n], cu[n+1]) ) and every value head listed in `heads` (all heads when
 * heads == NULL).  Output rows of heads that are not listed are left as they
 * are.  s0 may be NULL (zero start); s_final may be NULL.
 * Returns 0 on success, -1 on a bad argument.
 */
int oracle_kda_recurrence_gated(int dtype, const void *q, const void *k, const void *v,
                                const void *g, const void *beta, const int64_t *cu,
                                int num_seqs, int hqk, int hv, double scale,
                                int use_l2norm, const double *a_log,
                                const double *dt_bias, double lower_bound,
                                const double *s0, double *out, double *s_final,
                                const int *heads, int n_heads, int n_threads) {
  if ((a_log == NULL) != (dt_bias == NULL)) return -1;
  if (hqk <= 0 || hv <= 0 || hv % hqk != 0 || num_seqs < 0 || dtype < 0 || dtype > 2)
    return -1;
  if (heads) {
    for (int i = 0; i < n_heads; ++i)
      if (heads[i] < 0 || heads[i] >= hv) return -1;
  }
  job_t J;
  J.dtype = dtype; J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta;
  J.cu = cu; J.num_seqs = num_seqs; J.hqk = hqk; J.hv = hv;
  J.use_l2norm = use_l2norm; J.scale = scale; J.s0 = s0; J.out = out;
  J.a_log = a_log; J.dt_bias = dt_bias; J.lower_bound = lower_bound;
  J.s_final = s_final; J.heads = heads; J.n_heads = n_heads; J.next_unit = 0;
  pthread_mutex_init(&J.lock, NULL);
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  pthread_t th[256];
  for (int i = 0; i < n_threads; ++i) pthread_create(&th[i], NULL, worker, &J);
  for (int i = 0; i < n_threads; ++i) pthread_join(th[i], NULL);
  pthread_mutex_destroy(&J.lock);
  return 0;
}

/* The recurrence with g taken as the log-decay itself. */
int oracle_kda_recurrence(int dtype, const void *q, const void *k, const void *v,
                          const void *g, const void *beta, const int64_t *cu,
                          int num_seqs, int hqk, int hv, double scale,
                          int use_l2norm, const double *s0, double *out,
                          double *s_final, const int *heads, int n_heads,
                          int n_threads) {
  return oracle_kda_recurrence_gated(dtype, q, k, v, g, beta, cu, num_seqs, hqk, hv, scale,
                                     use_l2norm, NULL, NULL, 0.0, s0, out, s_final, heads,
                                     n_heads, n_threads);
}
