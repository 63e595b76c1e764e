/*
 * Oracle, recurrent form: one STILL layer processed token by token in fp64.
 *
 * TEST INFRASTRUCTURE ONLY. The product path never links or calls this
 * file; only tests/, the smoke check and the bench's CPU-baseline leg do.
 * It shares no code with the HIP path.
 *
 * Pages cited (short tag -> page title):
 *   [P2] "NeurIPS 2026|层内混合注意力：告别位置「伪混合」，STILL首个内容感知的层内混合注意力架构",
 *        sections 亮点一 (固定预算路由, 延迟选择与分块并行), 亮点二
 *   [P3] "STILL: Content-Aware Intra-Layer Hybrid Attention for Efficient
 *        LLM Linearization", sections "Content-Aware Routing with Fixed
 *        Budget", "Delayed Chunk-Level Selection for Unified
 *        Training-Inference Parallelism", "Self-Saliency Score",
 *        "NP-Map: Norm-Preserving Feature Map", "Problems with Existing
 *        Intra-Layer Hybrid Attention"
 *   [P4] "Synergizing Linear and Sparse Attention: A Deep Dive into Hybrid
 *        LLM Architectures", §2 (the linear state's forget gate), §4
 *        (gating; the separately normalised merge)
 *
 * The loop follows the recurrent (decoding) form the pages describe: tokens
 * arrive one by one; when a new chunk begins the previous chunk is decided
 * (Top-lambda by score, permanent); a decided, unselected token that has
 * left the window is accumulated into the linear-attention state; every
 * query attends with softmax to its window, its own chunk's prefix and the
 * kept tokens, and linearly (NP-Map features) to the state. Decode of n
 * steps after a prefill of L tokens is this same loop over L + n tokens
 * ([P3 "Delayed Chunk-Level Selection ..."]: prefill and decode share one
 * routing and memory-update rule).
 *
 * Build: gcc -O3 -march=native -ffp-contract=off -fPIC -shared -pthread.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Merge of the two branches (reading where the pages leave it open):
 *   MERGE_ONE: one normaliser over exp(logit) and gate * <phi(q), phi(k)>;
 *   MERGE_SUM: each branch normalised on its own, y = y_SA + gate * y_LA
 *     [P4 §4 Gating];
 *   MERGE_SOFTMAX_ONLY: the linear branch dropped, y = y_SA (the sparse
 *     attention alternative [P3 "Problems with Existing Intra-Layer Hybrid
 *     Attention"]); the state is still maintained. */
enum { MERGE_ONE = 0, MERGE_SUM = 1, MERGE_SOFTMAX_ONLY = 2 };

/* Routing metric: the score that ranks a chunk's tokens. The default is
 * the Self-Saliency Score; the others are the alternatives the pages'
 * routing-metric ablation compares it with [P3 "Ablation Studies"]:
 *   ROUTE_DIAG     the diagonal attention weight a_diag_t of the window
 *                  softmax, summed over the group's query heads;
 *   ROUTE_QK       the scaled self logit q_t . k_t, summed over the heads;
 *   ROUTE_KEYNORM  ||k_t|| (one value per kv head);
 *   ROUTE_UNIFORM  reading: evenly spaced positions, score 1 at the offsets
 *                  floor(i C / lambda), i < lambda, of each chunk, else 0;
 *   ROUTE_EXTERNAL scores supplied by the caller (random routing draws
 *                  them outside the layer). */
enum { ROUTE_SALIENCY = 0, ROUTE_DIAG, ROUTE_QK, ROUTE_KEYNORM, ROUTE_UNIFORM, ROUTE_EXTERNAL };

typedef struct {
  int L, d, G, W, C, m, t_max, lam, n_dec, merge, route;
  const float* ext; /* [n_units, L] caller scores (ROUTE_EXTERNAL), else null */
  double eps, scale;
  const float *q, *k, *v, *F, *gate;
  double *y, *score, *S, *z, *pending;
  int32_t *sel, *n_pool;
  double *y_sa, *lse_sa, *y_la, *lse_la; /* branch partials, or all null */
  const double* decay; /* [n_units] forget factor of the linear state, or null (1) */
  int fp8_from;        /* queries t >= fp8_from read the kept pool in e4m3; < 0: never */
} oracle_job;

typedef struct {
  const oracle_job* job;
  int first, step, count;
} worker_arg;

/* NP-Map [P3 "NP-Map"]: direction from softmax(x F), unit L2 norm, then the
 * input norm ||x|| is re-injected. u holds d doubles of scratch. */
static void np_map(const double* x, const double* F, int d, double* out, double* u) {
  double nx = 0.0;
  for (int i = 0; i < d; ++i) nx += x[i] * x[i];
  nx = sqrt(nx);
  for (int j = 0; j < d; ++j) u[j] = 0.0;
  for (int i = 0; i < d; ++i) {
    const double xi = x[i];
    const double* row = F + (size_t)i * d;
    for (int j = 0; j < d; ++j) u[j] += xi * row[j];
  }
  double mx = u[0];
  for (int j = 1; j < d; ++j) mx = u[j] > mx ? u[j] : mx;
  double nu = 0.0;
  for (int j = 0; j < d; ++j) {
    u[j] = exp(u[j] - mx);
    nu += u[j] * u[j];
  }
  nu = sqrt(nu);
  for (int j = 0; j < d; ++j) out[j] = nx * u[j] / nu;
}

/* Self-Saliency Score of token t for one head [P3 "Self-Saliency Score"]:
 * KL(a_diag || (1-eps) a_nodiag + eps delta_t) over the window
 * [max(0, t-W+1), t]. For j != t the ratio a_diag_j / ((1-eps) a_nodiag_j)
 * is the same for every j, so the sum collapses to the two-point form
 * p ln(p/eps) + (1-p) ln((1-p)/(1-eps)), p = a_diag_t; 1-p is summed from
 * the other entries (no cancellation). buf holds W doubles. */
static double saliency(const double* qh, const double* K, int t, int W, int d,
                       double scale, double eps, double* buf) {
  const int lo = t - W + 1 > 0 ? t - W + 1 : 0;
  const int n = t - lo + 1;
  for (int j = 0; j < n; ++j) {
    const double* kj = K + (size_t)(lo + j) * d;
    double s = 0.0;
    for (int i = 0; i < d; ++i) s += qh[i] * kj[i];
    buf[j] = scale * s;
  }
  double mx = buf[0];
  for (int j = 1; j < n; ++j) mx = buf[j] > mx ? buf[j] : mx;
  double zall = 0.0, zother = 0.0;
  for (int j = 0; j < n; ++j) {
    const double e = exp(buf[j] - mx);
    zall += e;
    if (j != n - 1) zother += e;
  }
  const double p = exp(buf[n - 1] - mx) / zall;
  const double pn = zother / zall;
  double sc = 0.0;
  if (p > 0.0) sc += p * log(p / eps);
  if (pn > 0.0) sc += pn * log(pn / (1.0 - eps));
  return sc;
}

/* Diagonal attention weight of token t for one head: the window softmax's
 * weight on the token itself. buf holds W doubles. */
static double diag_weight(const double* qh, const double* K, int t, int W, int d, double scale,
                          double* buf) {
  const int lo = t - W + 1 > 0 ? t - W + 1 : 0;
  const int n = t - lo + 1;
  for (int j = 0; j < n; ++j) {
    const double* kj = K + (size_t)(lo + j) * d;
    double s = 0.0;
    for (int i = 0; i < d; ++i) s += qh[i] * kj[i];
    buf[j] = scale * s;
  }
  double mx = buf[0];
  for (int j = 1; j < n; ++j) mx = buf[j] > mx ? buf[j] : mx;
  double z = 0.0;
  for (int j = 0; j < n; ++j) z += exp(buf[j] - mx);
  return exp(buf[n - 1] - mx) / z;
}

/* ROUTE_UNIFORM: 1 if offset r of a chunk of C is one of floor(i C / lam),
 * i = 0 .. lam - 1, else 0. */
static double uniform_mark(int r, int C, int lam) {
  for (int i = 0; i < lam; ++i)
    if ((int)(((long)i * C) / lam) == r) return 1.0;
  return 0.0;
}

static int full_chunks_out_of_window(int c, int W, int C) {
  const long x = (long)c * C - W + 1;
  return x >= 0 ? (int)(x / C) : 0;
}

/* OCP 8-bit floating point, E4M3 ("FN": no infinities, one NaN pattern per
 * sign): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; code
 * (e, m) with e > 0 is 2^(e-7) (1 + m/8), e = 0 is 2^-6 m/8; the largest
 * finite value is 448 (e = 15, m = 6), e = 15, m = 7 is NaN. Reading for
 * the kept pool's storage (the pages name fp8 pools, not a format): a row
 * x of d values is stored as the codes of x_i / s with a power-of-two scale
 * s = 2^e (an E8M0 exponent, as in the OCP microscaling formats), e the
 * smallest integer with amax <= 448 s (amax = max |x_i|; e = 0 for a zero
 * row), at least -126; each x_i / s (exact) rounded to the nearest E4M3
 * value, ties to the even code, magnitudes beyond 448 to 448. */
static uint8_t e4m3_code(float y) {
  const uint8_t sign = y < 0.0f ? 0x80 : 0x00;
  const float a = fabsf(y);
  if (!(a < 448.0f)) return sign | 0x7E;
  if (a < 0.015625f) { /* below 2^-6: multiples of 2^-9 (m = 8 is 2^-6, code 0x08) */
    return sign | (uint8_t)rintf(a * 512.0f);
  }
  int e;
  frexpf(a, &e); /* a = f 2^e, f in [0.5, 1): the binade is 2^(e-1) */
  e -= 1;
  int n = (int)rintf(ldexpf(a, 3 - e)); /* 8 .. 16 eighths of 2^e */
  if (n == 16) { n = 8; e += 1; }
  return sign | (uint8_t)(((e + 7) << 3) | (n - 8));
}

static double e4m3_value(uint8_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  const double v = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
  return (c & 0x80) ? -v : v;
}

/* One row: codes and the scale exponent e (s = 2^e). */
static int e4m3_row(const float* x, int d, uint8_t* codes) {
  float amax = 0.0f;
  for (int i = 0; i < d; ++i) amax = fabsf(x[i]) > amax ? fabsf(x[i]) : amax;
  int e = 0;
  if (amax > 0.0f) {
    int E;
    const float f = frexpf(amax, &E); /* amax = f 2^E, 448 = 0.875 2^9 */
    e = E - 9 + (f > 0.875f ? 1 : 0);
    if (e < -126) e = -126;
  }
  for (int i = 0; i < d; ++i) codes[i] = e4m3_code(ldexpf(x[i], -e));
  return e;
}

/* Rows x [n, d]: codes [n, d], scale exponents [n] (s = 2^e) and, if not
 * null, the values code * s [n, d]. */
int still_oracle_e4m3_rows(int n, int d, const float* x, uint8_t* codes, int32_t* exps,
                           double* values) {
  if (n < 0 || d < 1) return -1;
  for (int r = 0; r < n; ++r) {
    const int e = e4m3_row(x + (size_t)r * d, d, codes + (size_t)r * d);
    if (exps) exps[r] = e;
    if (values)
      for (int i = 0; i < d; ++i) values[(size_t)r * d + i] = ldexp(e4m3_value(codes[(size_t)r * d + i]), e);
  }
  return 0;
}

static void run_unit(const oracle_job* J, int u) {
  const int L = J->L, d = J->d, G = J->G, W = J->W, C = J->C;
  const size_t Ld = (size_t)L * d;
  double* K = malloc(sizeof(double) * Ld);
  double* V = malloc(sizeof(double) * Ld);
  double* Q = malloc(sizeof(double) * Ld * G);
  double* F = malloc(sizeof(double) * (size_t)d * d);
  double* SB = calloc((size_t)d * d, sizeof(double)); /* sum over B(t) */
  double* zB = calloc((size_t)d, sizeof(double));
  double* phi = malloc(sizeof(double) * d);
  double* phq = malloc(sizeof(double) * d);
  double* tmp = malloc(sizeof(double) * d);
  double* logit = malloc(sizeof(double) * (size_t)(L > W ? L : W));
  double* num = malloc(sizeof(double) * d);
  double* lnum = malloc(sizeof(double) * d);
  unsigned char* selected = calloc((size_t)L, 1);
  int* pool = malloc(sizeof(int) * (size_t)(J->m > 0 ? J->m : 1));
  int n_pool = 0, n_la = 0;
  const int want_la = J->y_la != NULL;
  const float* qs = J->q + (size_t)u * G * Ld;
  const float* ks = J->k + (size_t)u * Ld;
  const float* vs = J->v + (size_t)u * Ld;
  for (size_t i = 0; i < Ld; ++i) { K[i] = ks[i]; V[i] = vs[i]; }
  /* the kept pool as an 8-bit store holds every row quantised (only the
   * rows of kept tokens are read) */
  double *K8 = NULL, *V8 = NULL;
  if (J->fp8_from >= 0 && L > 0) {
    uint8_t* codes = malloc((size_t)d);
    K8 = malloc(sizeof(double) * Ld);
    V8 = malloc(sizeof(double) * Ld);
    for (int j = 0; j < L; ++j) {
      const int ek = e4m3_row(ks + (size_t)j * d, d, codes);
      for (int i = 0; i < d; ++i) K8[(size_t)j * d + i] = ldexp(e4m3_value(codes[i]), ek);
      const int ev = e4m3_row(vs + (size_t)j * d, d, codes);
      for (int i = 0; i < d; ++i) V8[(size_t)j * d + i] = ldexp(e4m3_value(codes[i]), ev);
    }
    free(codes);
  }
  for (size_t i = 0; i < Ld * G; ++i) Q[i] = qs[i];
  for (size_t i = 0; i < (size_t)d * d; ++i) F[i] = J->F[(size_t)u * d * d + i];
  double* score = J->score + (size_t)u * L;
  double* yu = J->y + (size_t)u * G * Ld;
  int32_t* selu = J->sel + (size_t)u * J->n_dec * (J->lam > 0 ? J->lam : 0);
  for (int i = 0; i < J->n_dec * J->lam; ++i) selu[i] = -1;

  /* Forget gate of the linear state (reading of [P4 §2]'s gated linear
   * attention with write strength 1 applied to the NP-Map state): the state
   * decays by gam every token, so key j enters the query at t with weight
   * gam^(t - j); gam = 1 is the plain layer. */
  const double gam = J->decay ? J->decay[u] : 1.0;
  int next_la = 0; /* every position below this has been routed to B or kept */
  for (int t = 0; t < L; ++t) {
    const int c = t / C;
    if (gam != 1.0 && t > 0) { /* the state, held at time t - 1, moves to t */
      for (size_t i = 0; i < (size_t)d * d; ++i) SB[i] *= gam;
      for (int a = 0; a < d; ++a) zB[a] *= gam;
    }
    /* Chunk c-1 is decided when chunk c begins [P3 "Delayed Chunk-Level
     * Selection"]: keep its lambda best tokens by (score desc, position
     * asc), while the pool (capacity m - W) has room [P2 固定预算路由]. */
    if (t > 0 && t % C == 0) {
      const int cd = c - 1, base = cd * C;
      const int lam_c = (n_pool + J->lam <= J->m - W) ? J->lam : 0;
      int chosen[1024];
      int n_ch = 0;
      for (int r = 0; r < lam_c; ++r) {
        int best = -1;
        for (int j = base; j < base + C; ++j) {
          if (selected[j]) continue;
          if (best < 0 || score[j] > score[best]) best = j;
        }
        selected[best] = 1;
        chosen[n_ch++] = best;
      }
      /* ascending positions */
      for (int a = 1; a < n_ch; ++a)
        for (int b2 = a; b2 > 0 && chosen[b2 - 1] > chosen[b2]; --b2) {
          const int tmpi = chosen[b2];
          chosen[b2] = chosen[b2 - 1];
          chosen[b2 - 1] = tmpi;
        }
      for (int a = 0; a < n_ch; ++a) {
        selu[cd * J->lam + a] = chosen[a];
        pool[n_pool++] = chosen[a];
      }
    }
    /* Decided, unselected tokens that have left the window join the
     * linear-attention state [P3 "Content-Aware Routing with Fixed
     * Budget"]: positions j <= min(t - W, cC - 1). */
    const int e = (t - W < c * C - 1) ? t - W : c * C - 1;
    while (next_la <= e) {
      const int j = next_la++;
      if (selected[j]) continue;
      np_map(K + (size_t)j * d, F, d, phi, tmp);
      const double wj = gam == 1.0 ? 1.0 : pow(gam, (double)(t - j));
      for (int a = 0; a < d; ++a) {
        zB[a] += wj * phi[a];
        const double pa = wj * phi[a];
        double* row = SB + (size_t)a * d;
        const double* vj = V + (size_t)j * d;
        for (int b2 = 0; b2 < d; ++b2) row[b2] += pa * vj[b2];
      }
      ++n_la;
    }
    /* Routing score of token t (summed over the group's query heads where
     * the metric is per query head). */
    double st = 0.0;
    if (J->route == ROUTE_KEYNORM) {
      for (int i = 0; i < d; ++i) st += K[(size_t)t * d + i] * K[(size_t)t * d + i];
      st = sqrt(st);
    } else if (J->route == ROUTE_UNIFORM) {
      st = uniform_mark(t % C, C, J->lam);
    } else if (J->route == ROUTE_EXTERNAL) {
      st = J->ext[(size_t)u * L + t];
    } else {
      for (int h = 0; h < G; ++h) {
        const double* qh = Q + (size_t)h * Ld + (size_t)t * d;
        if (J->route == ROUTE_DIAG) {
          st += diag_weight(qh, K, t, W, d, J->scale, logit);
        } else if (J->route == ROUTE_QK) {
          double s = 0.0;
          for (int i = 0; i < d; ++i) s += qh[i] * K[(size_t)t * d + i];
          st += J->scale * s;
        } else {
          st += saliency(qh, K, t, W, d, J->scale, J->eps, logit);
        }
      }
    }
    score[t] = st;

    /* Softmax keys: every j in [lo, t] (window or own chunk) plus kept
     * tokens below lo. Linear keys: the state. Merge (reading): one
     * normaliser over the softmax weights exp(s_j) and the gated linear
     * weights g <phi(q), phi(k_j)>, taken in the log domain. */
    int lo = t - W + 1 < c * C ? t - W + 1 : c * C;
    if (lo < 0) lo = 0;
    /* kept tokens below lo come from the pool's store: 8-bit from fp8_from on */
    const int p8 = K8 != NULL && t >= J->fp8_from;
    const double* Kp = p8 ? K8 : K;
    const double* Vp = p8 ? V8 : V;
    int n_keys = 0;
    for (int h = 0; h < G; ++h) {
      const double* qh = Q + (size_t)h * Ld + (size_t)t * d;
      const double g = J->gate[(size_t)u * G + h];
      n_keys = 0;
      for (int p = 0; p < n_pool && pool[p] < lo; ++p) {
        const double* kj = Kp + (size_t)pool[p] * d;
        double s = 0.0;
        for (int i = 0; i < d; ++i) s += qh[i] * kj[i];
        logit[n_keys++] = J->scale * s;
      }
      const int n_pool_keys = n_keys;
      for (int j = lo; j <= t; ++j) {
        const double* kj = K + (size_t)j * d;
        double s = 0.0;
        for (int i = 0; i < d; ++i) s += qh[i] * kj[i];
        logit[n_keys++] = J->scale * s;
      }
      double mx = logit[0];
      for (int a = 1; a < n_keys; ++a) mx = logit[a] > mx ? logit[a] : mx;
      double l = 0.0;
      for (int b2 = 0; b2 < d; ++b2) num[b2] = 0.0;
      for (int a = 0; a < n_keys; ++a) {
        const int j = a < n_pool_keys ? pool[a] : lo + (a - n_pool_keys);
        const double w = exp(logit[a] - mx);
        l += w;
        const double* vj = (a < n_pool_keys ? Vp : V) + (size_t)j * d;
        for (int b2 = 0; b2 < d; ++b2) num[b2] += w * vj[b2];
      }
      double* yt = yu + (size_t)h * Ld + (size_t)t * d;
      /* linear branch without the gate: den_la = <phi(q), z_B>,
       * lnum = phi(q)^T S_B */
      double den_la = 0.0;
      const int use_la = J->merge != MERGE_SOFTMAX_ONLY && g > 0.0;
      if (n_la > 0 && (use_la || want_la)) {
        np_map(qh, F, d, phq, tmp);
        for (int b2 = 0; b2 < d; ++b2) lnum[b2] = 0.0;
        for (int a = 0; a < d; ++a) {
          den_la += phq[a] * zB[a];
          const double pa = phq[a];
          const double* row = SB + (size_t)a * d;
          for (int b2 = 0; b2 < d; ++b2) lnum[b2] += pa * row[b2];
        }
      }
      const double lse_sa = mx + log(l);
      if (use_la && den_la > 0.0 && J->merge == MERGE_ONE) {
        const double lse_la = log(g * den_la);
        const double top = lse_sa > lse_la ? lse_sa : lse_la;
        const double wa = exp(lse_sa - top), wb = exp(lse_la - top);
        for (int b2 = 0; b2 < d; ++b2)
          yt[b2] = (wa * (num[b2] / l) + wb * (lnum[b2] / den_la)) / (wa + wb);
      } else if (use_la && den_la > 0.0) { /* MERGE_SUM */
        for (int b2 = 0; b2 < d; ++b2) yt[b2] = num[b2] / l + g * (lnum[b2] / den_la);
      } else {
        for (int b2 = 0; b2 < d; ++b2) yt[b2] = num[b2] / l;
      }
      if (want_la) {
        const size_t row = ((size_t)u * G + h) * L + t;
        for (int b2 = 0; b2 < d; ++b2) {
          J->y_sa[row * d + b2] = num[b2] / l;
          J->y_la[row * d + b2] = den_la > 0.0 ? lnum[b2] / den_la : 0.0;
        }
        J->lse_sa[row] = lse_sa;
        J->lse_la[row] = den_la > 0.0 ? log(den_la) : -INFINITY;
      }
    }
  }

  /* Exported state: the unselected tokens of the chunks lying wholly before
   * the window of every query of the last chunk (reading: the state absorbs
   * whole chunks), with the forget gate held at the first position past
   * them, R = cf C (key j weighted gam^(R - j)); pending = scores of the
   * undecided last chunk. */
  double* Su = J->S + (size_t)u * d * d;
  double* zu = J->z + (size_t)u * d;
  memset(Su, 0, sizeof(double) * (size_t)d * d);
  memset(zu, 0, sizeof(double) * (size_t)d);
  double* pend = J->pending + (size_t)u * C;
  for (int i = 0; i < C; ++i) pend[i] = NAN;
  if (L > 0) {
    const int c_last = (L - 1) / C;
    const int cf = full_chunks_out_of_window(c_last, W, C);
    for (int j = 0; j < cf * C; ++j) {
      if (selected[j]) continue;
      np_map(K + (size_t)j * d, F, d, phi, tmp);
      const double wj = gam == 1.0 ? 1.0 : pow(gam, (double)(cf * C - j));
      for (int a = 0; a < d; ++a) {
        zu[a] += wj * phi[a];
        for (int b2 = 0; b2 < d; ++b2) Su[(size_t)a * d + b2] += wj * phi[a] * V[(size_t)j * d + b2];
      }
    }
    for (int j = c_last * C; j < L; ++j) pend[j - c_last * C] = score[j];
  }
  J->n_pool[u] = n_pool;

  free(K); free(V); free(Q); free(F); free(SB); free(zB); free(phi); free(phq);
  free(tmp); free(logit); free(num); free(lnum); free(selected); free(pool);
  free(K8); free(V8);
}

static void* worker(void* p) {
  const worker_arg* a = (const worker_arg*)p;
  for (int u = a->first; u < a->count; u += a->step) run_unit(a->job, u);
  return NULL;
}

/* Runs n_units independent (batch row, kv head) units.
 * Inputs (float32 host arrays; bf16 values are exact in float32):
 *   q [n_units, G, L, d], k/v [n_units, L, d], F [n_units, d, d],
 *   gate [n_units, G].
 * Outputs (host, caller-allocated):
 *   y [n_units, G, L, d], score [n_units, L], sel [n_units, n_dec, lam],
 *   S [n_units, d, d], z [n_units, d], pending [n_units, C], n_pool [n_units].
 * merge: MERGE_ONE, MERGE_SUM or MERGE_SOFTMAX_ONLY. route: a ROUTE_*
 * metric; ext [n_units, L]: the caller's scores for ROUTE_EXTERNAL (else
 * ignored, may be null). y_sa, lse_sa, y_la,
 * lse_la: all null, or the branch partials [n_units, G, L, d] / [n_units,
 * G, L]: each branch normalised on its own, the linear one without the
 * gate (y_la = 0, lse_la = -inf where the state is empty), lse = natural
 * log of the branch's weight sum. decay: null, or [n_units] forget factors
 * in (0, 1] of the linear state (key j weighted decay^(t - j) at query t;
 * the exported state holds decay^(R - j), R = the first position past it).
 * fp8_from: queries at t >= fp8_from read the kept tokens below their
 * window band as E4M3 codes times the row's power-of-two scale (e4m3_row);
 * < 0: never.
 * Returns 0, or -1 on invalid sizes. */
int still_oracle_run(int n_units, int L, int d, int G, int W, int C, int m, int t_max,
                     double eps, double scale, const float* q, const float* k,
                     const float* v, const float* F, const float* gate, int n_threads,
                     double* y, double* score, int32_t* sel, double* S, double* z,
                     double* pending, int32_t* n_pool, int merge, double* y_sa,
                     double* lse_sa, double* y_la, double* lse_la, int route,
                     const float* ext, const double* decay, int fp8_from) {
  if (n_units < 0 || L < 0 || d < 1 || G < 1 || W < 1 || C < 1 || m < W || t_max < 1)
    return -1;
  if (merge < MERGE_ONE || merge > MERGE_SOFTMAX_ONLY) return -1;
  if (route < ROUTE_SALIENCY || route > ROUTE_EXTERNAL) return -1;
  if (route == ROUTE_EXTERNAL && !ext) return -1;
  if (!(y_sa && lse_sa && y_la && lse_la) && (y_sa || lse_sa || y_la || lse_la)) return -1;
  for (int u = 0; decay && u < n_units; ++u)
    if (!(decay[u] > 0.0 && decay[u] <= 1.0)) return -1;
  int lam = (m - W) / t_max;
  if (lam > C) lam = C;
  if (lam > 1024) return -1;
  oracle_job J = {L, d, G, W, C, m, t_max, lam, L > 0 ? (L - 1) / C : 0, merge, route, ext,
                  eps, scale,
                  q, k, v, F, gate, y, score, S, z, pending, sel, n_pool,
                  y_sa, lse_sa, y_la, lse_la, decay, fp8_from};
  if (n_threads < 1) n_threads = 1;
  if (n_threads > n_units) n_threads = n_units > 0 ? n_units : 1;
  pthread_t th[256];
  worker_arg args[256];
  if (n_threads > 256) n_threads = 256;
  for (int i = 0; i < n_threads; ++i) {
    args[i].job = &J;
    args[i].first = i;
    args[i].step = n_threads;
    args[i].count = n_units;
    if (n_threads == 1) worker(&args[i]);
    else pthread_create(&th[i], NULL, worker, &args[i]);
  }
  if (n_threads > 1)
    for (int i = 0; i < n_threads; ++i) pthread_join(th[i], NULL);
  return 0;
}
