/* oracle.c -- TEST INFRASTRUCTURE ONLY (see oracle.h).
 *
 * A plain CPU reference of the group-limited top-k MoE layer forward.  Every
 * function loops per token / per expert in the order the method is described
 * in; there is no blocking, fusion or reordering of the arithmetic beyond that.
 * Threads (pthreads) only split independent tokens; each token's arithmetic is
 * sequential, so results do not depend on the thread count.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fPIC -shared -pthread.
 * Contraction must stay off: sigma32 below is specified with explicit fma()
 * and separately rounded adds and multiplies.
 *
 * Citations: [Routing §n] = the page "InternLumina-U2中256个专家的路由秘密：分组
 * 受限Top-K、Expert Bias与Fused MoE详解", section n of its numbered headings.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* element access                                                           */
/* ------------------------------------------------------------------------ */

static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16; /* bf16 is the top half of an fp32 */
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double elem(const void* base, int dt, size_t i) {
  if (dt == ORC_BF16) return bf16_bits_to_double(((const uint16_t*)base)[i]);
  if (dt == ORC_F64) return ((const double*)base)[i];
  return (double)((const float*)base)[i];
}

/* ------------------------------------------------------------------------ */
/* sigma32                                                                  */
/* ------------------------------------------------------------------------ */
/* [Routing §二 step 1] scores each expert independently with a logistic
 * sigmoid of the fp32 logit (no softmax), and returns the score in fp32.  The
 * page does not fix the rounding of that sigmoid, so this build specifies one
 * (implemented a second time, independently, in the HIP library):
 *
 *   sigma32(z) = RN32( 1 / (1 + E(-z)) ), all operations in IEEE fp64, where
 *   E(t) = 2^n * P(r), n = rint(t*log2(e)), r = (t - n*L1) - n*L2 by two fma
 *   (Cody & Waite argument reduction, "Software Manual for the Elementary
 *   Functions", 1980; L1 = RN(ln 2), L2 = RN(ln 2 - L1)), and P the degree-13
 *   Taylor polynomial of exp with coefficients RN(1/i!), evaluated by Horner
 *   with fma from the top coefficient down.
 *   Early exits (each equal to what the formula itself returns):
 *     NaN -> NaN;  -z > 104 -> +0 (the value is below 2^-150);
 *     -z < -40 -> 1 (E < 2^-54, so 1 + E rounds to 1).
 */
static const double LOG2E = 0x1.71547652b82fep+0;  /* RN(1/ln 2)        */
static const double LN2_1 = 0x1.62e42fefa39efp-1;  /* RN(ln 2)          */
static const double LN2_2 = 0x1.abc9e3b39803fp-56; /* RN(ln 2 - LN2_1)  */

static double taylor_c[14];
static pthread_once_t taylor_once = PTHREAD_ONCE_INIT;

static void taylor_init(void) {
  double fact = 1.0; /* i! is exact in fp64 for i <= 18 */
  for (int i = 0; i < 14; ++i) {
    if (i > 0) fact *= (double)i;
    taylor_c[i] = 1.0 / fact;
  }
}

static double pow2i(int n) { /* 2^n for -1022 <= n <= 1023, exact */
  uint64_t bits = (uint64_t)(n + 1023) << 52;
  double d;
  memcpy(&d, &bits, sizeof d);
  return d;
}

float orc_sigmoid32(float z) {
  pthread_once(&taylor_once, taylor_init);
  if (z != z) return z;
  double t = -(double)z;
  if (t > 104.0) return 0.0f;
  if (t < -40.0) return 1.0f;
  double n = rint(t * LOG2E);
  double r = fma(-n, LN2_1, t);
  r = fma(-n, LN2_2, r);
  double p = taylor_c[13];
  for (int i = 12; i >= 0; --i) p = fma(p, r, taylor_c[i]);
  double e = p * pow2i((int)n);
  return (float)(1.0 / (1.0 + e));
}

void orc_sigmoid32_array(const float* z, float* s, int64_t n) {
  for (int64_t i = 0; i < n; ++i) s[i] = orc_sigmoid32(z[i]);
}

/* --- accuracy scan against an independent long-double evaluation --------- */

static float bits_to_float(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}
static uint32_t float_to_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

typedef struct {
  uint64_t start, stop, stride;
  int64_t out[4];
} scan_job_t;

static void* scan_worker(void* arg) {
  scan_job_t* j = (scan_job_t*)arg;
  int64_t checked = 0, not_rn = 0, over1 = 0, nonmono = 0;
  int have_prev = 0;
  uint32_t prev_bits = 0;
  float prev_s = 0.0f;
  for (uint64_t b = j->start; b < j->stop; b += j->stride) {
    uint32_t bits = (uint32_t)b;
    float z = bits_to_float(bits);
    float s = orc_sigmoid32(z);
    ++checked;
    if (z != z) {
      if (s == s) ++over1; /* NaN must map to NaN */
      have_prev = 0;
      continue;
    }
    long double ref = 1.0L / (1.0L + expl(-(long double)z));
    float rn = (float)ref;
    if (float_to_bits(s) != float_to_bits(rn)) ++not_rn;
    /* s and the reference are both >= 0: the bit distance is the ulp distance */
    int64_t d = (int64_t)float_to_bits(s) - (int64_t)float_to_bits(rn);
    if (d > 1 || d < -1) ++over1;
    if (have_prev && ((prev_bits ^ bits) & 0x80000000u) == 0) {
      /* same sign: z increases with the bit pattern for z >= +0 and decreases
       * for z <= -0, so sigma must follow the same direction */
      int positive = (bits & 0x80000000u) == 0;
      if (positive ? (s < prev_s) : (s > prev_s)) ++nonmono;
    }
    have_prev = 1;
    prev_bits = bits;
    prev_s = s;
  }
  j->out[0] = checked;
  j->out[1] = not_rn;
  j->out[2] = over1;
  j->out[3] = nonmono;
  return NULL;
}

void orc_sigmoid32_scan(uint64_t start, uint64_t stop, uint64_t stride, int nthreads,
                        int64_t out[4]) {
  if (nthreads < 1) nthreads = 1;
  if (stride < 1) stride = 1;
  uint64_t count = stop > start ? (stop - start + stride - 1) / stride : 0;
  scan_job_t* jobs = (scan_job_t*)calloc((size_t)nthreads, sizeof(scan_job_t));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  uint64_t per = (count + (uint64_t)nthreads - 1) / (uint64_t)nthreads;
  for (int i = 0; i < nthreads; ++i) {
    uint64_t a = start + (uint64_t)i * per * stride;
    uint64_t e = start + (uint64_t)(i + 1) * per * stride;
    if (a > stop) a = stop;
    if (e > stop) e = stop;
    /* overlap by one step so monotonicity is also checked across chunk edges */
    jobs[i].start = (i > 0 && a >= start + stride) ? a - stride : a;
    jobs[i].stop = e;
    jobs[i].stride = stride;
    pthread_create(&th[i], NULL, scan_worker, &jobs[i]);
  }
  for (int k = 0; k < 4; ++k) out[k] = 0;
  for (int i = 0; i < nthreads; ++i) {
    pthread_join(th[i], NULL);
    for (int k = 0; k < 4; ++k) out[k] += jobs[i].out[k];
    if (i > 0 && jobs[i].start < jobs[i].stop) {
      /* the overlapping first element was counted twice */
      uint32_t bits = (uint32_t)jobs[i].start;
      float z = bits_to_float(bits);
      out[0] -= 1;
      if (z == z) {
        float s = orc_sigmoid32(z);
        float rn = (float)(1.0L / (1.0L + expl(-(long double)z)));
        if (float_to_bits(s) != float_to_bits(rn)) out[1] -= 1;
        int64_t d = (int64_t)float_to_bits(s) - (int64_t)float_to_bits(rn);
        if (d > 1 || d < -1) out[2] -= 1;
      } else if (orc_sigmoid32(z) == orc_sigmoid32(z)) {
        out[2] -= 1;
      }
    }
  }
  free(jobs);
  free(th);
}

/* --- sigma32 of every bit pattern in a range, compared with another's ---- */

typedef struct {
  uint64_t start, n;        /* bit patterns start .. start + n - 1 */
  const float* other;       /* other[i] is the other side's sigma32(pattern start + i) */
  int64_t mismatches, first;
} cmp_job_t;

static void* cmp_worker(void* arg) {
  cmp_job_t* j = (cmp_job_t*)arg;
  j->mismatches = 0;
  j->first = -1;
  for (uint64_t i = 0; i < j->n; ++i) {
    float s = orc_sigmoid32(bits_to_float((uint32_t)(j->start + i)));
    float o = j->other[i];
    int same = float_to_bits(s) == float_to_bits(o) || (s != s && o != o);
    if (!same) {
      if (j->first < 0) j->first = (int64_t)i;
      ++j->mismatches;
    }
  }
  return NULL;
}

void orc_sigmoid32_compare(uint64_t start, uint64_t n, const float* other, int nthreads,
                           int64_t out[2]) {
  if (nthreads < 1) nthreads = 1;
  cmp_job_t* jobs = (cmp_job_t*)calloc((size_t)nthreads, sizeof(cmp_job_t));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  uint64_t per = (n + (uint64_t)nthreads - 1) / (uint64_t)nthreads;
  for (int i = 0; i < nthreads; ++i) {
    uint64_t a = (uint64_t)i * per, e = a + per;
    if (a > n) a = n;
    if (e > n) e = n;
    jobs[i].start = start + a;
    jobs[i].n = e - a;
    jobs[i].other = other + a;
    pthread_create(&th[i], NULL, cmp_worker, &jobs[i]);
  }
  out[0] = 0;
  out[1] = -1;
  for (int i = 0; i < nthreads; ++i) {
    pthread_join(th[i], NULL);
    out[0] += jobs[i].mismatches;
    if (out[1] < 0 && jobs[i].first >= 0) out[1] = (int64_t)((uint64_t)i * per) + jobs[i].first;
  }
  free(jobs);
  free(th);
}

/* ------------------------------------------------------------------------ */
/* thread helper: run fn(ctx, t0, t1) over [0, n) split into contiguous chunks */
/* ------------------------------------------------------------------------ */

typedef void (*range_fn)(void* ctx, int t0, int t1);
typedef struct {
  range_fn fn;
  void* ctx;
  int t0, t1;
} range_job_t;

static void* range_worker(void* arg) {
  range_job_t* j = (range_job_t*)arg;
  j->fn(j->ctx, j->t0, j->t1);
  return NULL;
}

static void parallel_range(range_fn fn, void* ctx, int n, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n) nthreads = n > 0 ? n : 1;
  if (nthreads == 1) {
    fn(ctx, 0, n);
    return;
  }
  range_job_t* jobs = (range_job_t*)calloc((size_t)nthreads, sizeof(range_job_t));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int i = 0; i < nthreads; ++i) {
    jobs[i].fn = fn;
    jobs[i].ctx = ctx;
    jobs[i].t0 = (int)((int64_t)n * i / nthreads);
    jobs[i].t1 = (int)((int64_t)n * (i + 1) / nthreads);
    pthread_create(&th[i], NULL, range_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(jobs);
  free(th);
}

/* ------------------------------------------------------------------------ */
/* R1: router logits                                                        */
/* ------------------------------------------------------------------------ */
/* [Routing §二 step 1]: logits = linear(x, W) with both operands in fp32 and no
 * bias term.  Here the exact inputs are widened to fp64 and each dot product is
 * summed over h in ascending order. */

typedef struct {
  int H, E, xdt;
  const void* x;
  const float* w;
  double* out;
} logits_ctx_t;

static void logits_range(void* vctx, int t0, int t1) {
  logits_ctx_t* c = (logits_ctx_t*)vctx;
  double* xr = (double*)malloc(sizeof(double) * (size_t)c->H);
  for (int t = t0; t < t1; ++t) {
    for (int h = 0; h < c->H; ++h) xr[h] = elem(c->x, c->xdt, (size_t)t * c->H + h);
    for (int e = 0; e < c->E; ++e) {
      const float* wr = c->w + (size_t)e * c->H;
      double acc = 0.0;
      for (int h = 0; h < c->H; ++h) acc += xr[h] * (double)wr[h];
      c->out[(size_t)t * c->E + e] = acc;
    }
  }
  free(xr);
}

void orc_logits(int T, int H, int E, const void* x, int xdt, const float* w_router,
                double* logits, int nthreads) {
  logits_ctx_t c = {H, E, xdt, x, w_router, logits};
  parallel_range(logits_range, &c, T, nthreads);
}

/* ------------------------------------------------------------------------ */
/* R2..R8: one token's selection                                            */
/* ------------------------------------------------------------------------ */

static int select_valid(int E, int n_group, int topk_group, int K) {
  if (E <= 0 || n_group <= 0 || E % n_group != 0) return 0;
  if (E / n_group < 2) return 0;
  if (topk_group < 1 || topk_group > n_group) return 0;
  if (K < 1 || K > topk_group * (E / n_group)) return 0;
  return 1;
}

/* Group score [Routing §二 step 2]: the experts are cut, in index order, into
 * n_group contiguous groups; a group's score is the sum of its two highest
 * (biased, see §三) scores, the two taken as a multiset. */
static float group_top2_sum(const float* sb, int first, int size) {
  float m1 = -INFINITY, m2 = -INFINITY;
  for (int i = 0; i < size; ++i) {
    float v = sb[first + i];
    if (v > m1) {
      m2 = m1;
      m1 = v;
    } else if (v > m2) {
      m2 = v;
    }
  }
  return m1 + m2;
}

/* Returns 0 on success, 1 when a logit is not finite (row left as -1 / 0). */
static int select_token(int E, int n_group, int topk_group, int K, float scale,
                        const float* lam, const float* bias, int32_t* idx, float* w,
                        float* s, float* sb, float* gs, uint8_t* gkeep, uint8_t* taken) {
  for (int e = 0; e < E; ++e) {
    if (!isfinite(lam[e])) {
      for (int j = 0; j < K; ++j) {
        idx[j] = -1;
        w[j] = 0.0f;
      }
      return 1;
    }
  }
  /* [Routing §二 step 1] independent sigmoid score per expert */
  for (int e = 0; e < E; ++e) s[e] = orc_sigmoid32(lam[e]);
  /* [Routing §三] the bias is added only to the scores that compete in the
   * top-k; an absent bias is zero */
  for (int e = 0; e < E; ++e) sb[e] = s[e] + (bias ? bias[e] : 0.0f);
  /* [Routing §二 step 2] group scores */
  int gsize = E / n_group;
  for (int g = 0; g < n_group; ++g) gs[g] = group_top2_sum(sb, g * gsize, gsize);
  /* keep the topk_group best groups; among equal scores the lower group index
   * ranks first */
  memset(gkeep, 0, (size_t)n_group);
  for (int r = 0; r < topk_group; ++r) {
    int best = -1;
    for (int g = 0; g < n_group; ++g) {
      if (gkeep[g]) continue;
      if (best < 0 || gs[g] > gs[best]) best = g;
    }
    gkeep[best] = 1;
  }
  /* every expert of a dropped group gets -inf */
  for (int e = 0; e < E; ++e)
    if (!gkeep[e / gsize]) sb[e] = -INFINITY;
  /* global top-K over all experts by (score descending, index ascending) */
  memset(taken, 0, (size_t)E);
  for (int j = 0; j < K; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || sb[e] > sb[best]) best = e;
    }
    taken[best] = 1;
    idx[j] = best;
  }
  /* [Routing §二 step 3 and §三] weights from the unbiased scores of the K
   * chosen experts: divide by (their sum + 1e-20), then scale.  The sum runs
   * in the order the experts were chosen, in fp32. */
  float S = s[idx[0]];
  for (int j = 1; j < K; ++j) S = S + s[idx[j]];
  float d = S + 1e-20f;
  for (int j = 0; j < K; ++j) {
    float q = s[idx[j]] / d;
    w[j] = q * scale;
  }
  return 0;
}

int orc_select(int T, int E, int n_group, int topk_group, int K, float scale,
               const float* lam, const float* bias, int32_t* idx, float* w, uint8_t* flag) {
  if (!select_valid(E, n_group, topk_group, K)) return -1;
  float* s = (float*)malloc(sizeof(float) * (size_t)E);
  float* sb = (float*)malloc(sizeof(float) * (size_t)E);
  float* gs = (float*)malloc(sizeof(float) * (size_t)n_group);
  uint8_t* gkeep = (uint8_t*)malloc((size_t)n_group);
  uint8_t* taken = (uint8_t*)malloc((size_t)E);
  int nflag = 0;
  for (int t = 0; t < T; ++t) {
    int f = select_token(E, n_group, topk_group, K, scale, lam + (size_t)t * E, bias,
                         idx + (size_t)t * K, w + (size_t)t * K, s, sb, gs, gkeep, taken);
    if (flag) flag[t] = (uint8_t)f;
    nflag += f;
  }
  free(s);
  free(sb);
  free(gs);
  free(gkeep);
  free(taken);
  return nflag;
}

/* ------------------------------------------------------------------------ */
/* interval analysis (test helper)                                          */
/* ------------------------------------------------------------------------ */
/* If every fp32 logit lies in [l - tau, l + tau], tau = tau_abs + tau_rel*|l|
 * (the error of an fp32 dot product grows with the size of its partial sums),
 * then, sigma32 and fp32
 * addition being monotone, every biased score lies in [sb_lo, sb_hi] and every
 * group score (a sum of the two largest) in [gs_lo, gs_hi].  The reference
 * selection idx_ref (made from RN32(l)) is the only possible one when the kept
 * groups and the chosen experts are separated from the rest by those bounds. */

int orc_route_intervals(int T, int E, int n_group, int topk_group, int K,
                        const double* logits, double tau_abs, double tau_rel, const float* bias,
                        const int32_t* idx_ref, uint8_t* decided, float* sb_lo_out,
                        float* sb_hi_out, float* gs_lo_out, float* gs_hi_out) {
  if (!select_valid(E, n_group, topk_group, K)) return -1;
  int gsize = E / n_group;
  float* lo = (float*)malloc(sizeof(float) * (size_t)E);
  float* hi = (float*)malloc(sizeof(float) * (size_t)E);
  float* glo = (float*)malloc(sizeof(float) * (size_t)n_group);
  float* ghi = (float*)malloc(sizeof(float) * (size_t)n_group);
  uint8_t* gin = (uint8_t*)malloc((size_t)n_group);
  uint8_t* ein = (uint8_t*)malloc((size_t)E);
  float* mid = (float*)malloc(sizeof(float) * (size_t)E);
  float* gmid = (float*)malloc(sizeof(float) * (size_t)n_group);
  int n_undecided = 0;
  for (int t = 0; t < T; ++t) {
    const double* l = logits + (size_t)t * E;
    const int32_t* ref = idx_ref + (size_t)t * K;
    for (int e = 0; e < E; ++e) {
      const double tau = tau_abs + tau_rel * fabs(l[e]);
      float a = nextafterf((float)(l[e] - tau), -INFINITY);
      float b = nextafterf((float)(l[e] + tau), INFINITY);
      float bb = bias ? bias[e] : 0.0f;
      lo[e] = orc_sigmoid32(a) + bb;
      hi[e] = orc_sigmoid32(b) + bb;
    }
    for (int g = 0; g < n_group; ++g) {
      glo[g] = group_top2_sum(lo, g * gsize, gsize);
      ghi[g] = group_top2_sum(hi, g * gsize, gsize);
    }
    uint8_t dec = 0;
    if (ref[0] >= 0) {
      /* the kept groups of the reference selection: the same ranking as
       * select_token, on the scores of RN32(l) */
      for (int e = 0; e < E; ++e) mid[e] = orc_sigmoid32((float)l[e]) + (bias ? bias[e] : 0.0f);
      for (int g = 0; g < n_group; ++g) gmid[g] = group_top2_sum(mid, g * gsize, gsize);
      memset(gin, 0, (size_t)n_group);
      for (int r = 0; r < topk_group; ++r) {
        int best = -1;
        for (int g = 0; g < n_group; ++g) {
          if (gin[g]) continue;
          if (best < 0 || gmid[g] > gmid[best]) best = g;
        }
        gin[best] = 1;
      }
      float min_in = INFINITY, max_out = -INFINITY;
      for (int g = 0; g < n_group; ++g) {
        if (gin[g]) min_in = glo[g] < min_in ? glo[g] : min_in;
        else max_out = ghi[g] > max_out ? ghi[g] : max_out;
      }
      int groups_ok = (topk_group == n_group) || (min_in > max_out);
      memset(ein, 0, (size_t)E);
      for (int j = 0; j < K; ++j) ein[ref[j]] = 1;
      float emin = INFINITY, emax = -INFINITY;
      for (int e = 0; e < E; ++e) {
        if (!gin[e / gsize]) continue;
        if (ein[e]) emin = lo[e] < emin ? lo[e] : emin;
        else emax = hi[e] > emax ? hi[e] : emax;
      }
      int set_ok = groups_ok && (emin > emax);
      int order_ok = set_ok;
      for (int j = 0; j + 1 < K && order_ok; ++j)
        if (!(lo[ref[j]] > hi[ref[j + 1]])) order_ok = 0;
      dec = (uint8_t)((set_ok ? 1 : 0) | (order_ok ? 2 : 0));
    }
    decided[t] = dec;
    if (!(dec & 1)) ++n_undecided;
    if (sb_lo_out) memcpy(sb_lo_out + (size_t)t * E, lo, sizeof(float) * (size_t)E);
    if (sb_hi_out) memcpy(sb_hi_out + (size_t)t * E, hi, sizeof(float) * (size_t)E);
    if (gs_lo_out) memcpy(gs_lo_out + (size_t)t * n_group, glo, sizeof(float) * (size_t)n_group);
    if (gs_hi_out) memcpy(gs_hi_out + (size_t)t * n_group, ghi, sizeof(float) * (size_t)n_group);
  }
  free(lo);
  free(hi);
  free(glo);
  free(ghi);
  free(gin);
  free(ein);
  free(mid);
  free(gmid);
  return n_undecided;
}

/* ------------------------------------------------------------------------ */
/* a5: permutation by expert                                                */
/* ------------------------------------------------------------------------ */
/* [Routing §六] counts are the per-expert hit counts (a bincount of the chosen
 * indices); [Routing §四] the eager inference path buckets tokens by expert
 * before running each bucket.  Counting sort over pair ids p = t*K + j in
 * ascending order, so each bucket keeps pair order (stable). */
void orc_permute(int T, int K, int E, const int32_t* idx, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_pair, int32_t* pair_slot) {
  int64_t P = (int64_t)T * K;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < P; ++p) counts[idx[p]] += 1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  for (int e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int64_t p = 0; p < P; ++p) {
    int32_t pos = cursor[idx[p]]++;
    sorted_pair[pos] = (int32_t)p;
    pair_slot[p] = pos;
  }
  free(cursor);
}

/* ------------------------------------------------------------------------ */
/* a6..a8: experts and combine                                              */
/* ------------------------------------------------------------------------ */
/* [Routing §四]: gate_proj, up_proj and down_proj are each one stacked tensor
 * of shape [E][I][H]; every expert is a SwiGLU feed-forward network,
 * down( silu(gate(x)) * up(x) ), with silu(z) = z * sigmoid(z) and no biases.
 * With down stored [I][H], its output is out_h = sum_i a_i * W_down[i][h].
 * [Routing §五]: the one shared expert is an always-on MLP of the same form
 * whose output is added to the weighted routed sum with no weight. */

static void swiglu_ffn(const void* wg, const void* wu, const void* wd, int wdt, size_t base,
                       int I, int H, const double* xr, double* a, double* out) {
  for (int i = 0; i < I; ++i) {
    double g = 0.0, u = 0.0;
    size_t row = base + (size_t)i * H;
    for (int h = 0; h < H; ++h) g += xr[h] * elem(wg, wdt, row + h);
    for (int h = 0; h < H; ++h) u += xr[h] * elem(wu, wdt, row + h);
    a[i] = g / (1.0 + exp(-g)) * u;
  }
  /* out_h = sum_i a_i * W_down[i][h], summed over i in ascending order for
   * every h (looping i outside keeps that order and walks rows contiguously) */
  for (int h = 0; h < H; ++h) out[h] = 0.0;
  for (int i = 0; i < I; ++i) {
    size_t row = base + (size_t)i * H;
    for (int h = 0; h < H; ++h) out[h] += a[i] * elem(wd, wdt, row + h);
  }
}

typedef struct {
  const orc_experts_t* ex;
  const void* x;
  int xdt;
  const int32_t* idx;
  const float* w;
  const int32_t* tokens;
  double* y;
} path_a_ctx_t;

static void path_a_range(void* vctx, int r0, int r1) {
  path_a_ctx_t* c = (path_a_ctx_t*)vctx;
  const orc_experts_t* ex = c->ex;
  int H = ex->H, I = ex->I, Is = ex->I_shared, K = ex->K;
  int amax = I > Is ? I : Is;
  double* xr = (double*)malloc(sizeof(double) * (size_t)H);
  double* a = (double*)malloc(sizeof(double) * (size_t)(amax > 0 ? amax : 1));
  double* o = (double*)malloc(sizeof(double) * (size_t)H);
  for (int r = r0; r < r1; ++r) {
    int t = c->tokens ? c->tokens[r] : r;
    double* yr = c->y + (size_t)r * H;
    for (int h = 0; h < H; ++h) xr[h] = elem(c->x, c->xdt, (size_t)t * H + h);
    /* y = shared(x) + sum_j w_j * expert_{idx_j}(x), accumulated in j order */
    if (Is > 0 && ex->ws_gate) {
      swiglu_ffn(ex->ws_gate, ex->ws_up, ex->ws_down, ex->wdt, 0, Is, H, xr, a, o);
      for (int h = 0; h < H; ++h) yr[h] = o[h];
    } else {
      for (int h = 0; h < H; ++h) yr[h] = 0.0;
    }
    for (int j = 0; j < K; ++j) {
      int e = c->idx[(size_t)t * K + j];
      double wj = (double)c->w[(size_t)t * K + j];
      swiglu_ffn(ex->w_gate, ex->w_up, ex->w_down, ex->wdt, (size_t)e * I * H, I, H, xr, a, o);
      for (int h = 0; h < H; ++h) yr[h] += wj * o[h];
    }
  }
  free(xr);
  free(a);
  free(o);
}

void orc_experts_path_a(const orc_experts_t* ex, const void* x, int xdt, const int32_t* idx,
                        const float* w, const int32_t* tokens, int n_tok, double* y,
                        int nthreads) {
  path_a_ctx_t c = {ex, x, xdt, idx, w, tokens, y};
  parallel_range(path_a_range, &c, n_tok, nthreads);
}

/* path B: per expert, over its bucket of pairs */
typedef struct {
  const orc_experts_t* ex;
  const void* x;
  int xdt;
  const int32_t* offsets;
  const int32_t* sorted_pair;
  double* pair_out; /* [T*K][H], indexed by pair id */
} path_b_ctx_t;

static void path_b_range(void* vctx, int e0, int e1) {
  path_b_ctx_t* c = (path_b_ctx_t*)vctx;
  const orc_experts_t* ex = c->ex;
  int H = ex->H, I = ex->I, K = ex->K;
  double* xr = (double*)malloc(sizeof(double) * (size_t)H);
  double* a = (double*)malloc(sizeof(double) * (size_t)(I > 0 ? I : 1));
  for (int e = e0; e < e1; ++e) {
    for (int q = c->offsets[e]; q < c->offsets[e + 1]; ++q) {
      int p = c->sorted_pair[q];
      int t = p / K;
      for (int h = 0; h < H; ++h) xr[h] = elem(c->x, c->xdt, (size_t)t * H + h);
      swiglu_ffn(ex->w_gate, ex->w_up, ex->w_down, ex->wdt, (size_t)e * I * H, I, H, xr, a,
                 c->pair_out + (size_t)p * H);
    }
  }
  free(xr);
  free(a);
}

void orc_experts_path_b(const orc_experts_t* ex, int T, const void* x, int xdt,
                        const int32_t* idx, const float* w, double* y, int nthreads) {
  int H = ex->H, K = ex->K, E = ex->E, Is = ex->I_shared;
  int64_t P = (int64_t)T * K;
  int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t* sorted_pair = (int32_t*)malloc(sizeof(int32_t) * (size_t)(P > 0 ? P : 1));
  int32_t* pair_slot = (int32_t*)malloc(sizeof(int32_t) * (size_t)(P > 0 ? P : 1));
  double* pair_out = (double*)malloc(sizeof(double) * (size_t)(P > 0 ? P : 1) * (size_t)H);
  orc_permute(T, K, E, idx, counts, offsets, sorted_pair, pair_slot);
  path_b_ctx_t c = {ex, x, xdt, offsets, sorted_pair, pair_out};
  parallel_range(path_b_range, &c, E, nthreads);
  double* xr = (double*)malloc(sizeof(double) * (size_t)H);
  double* a = (double*)malloc(sizeof(double) * (size_t)(Is > 0 ? Is : 1));
  for (int t = 0; t < T; ++t) {
    double* yr = y + (size_t)t * H;
    if (Is > 0 && ex->ws_gate) {
      for (int h = 0; h < H; ++h) xr[h] = elem(x, xdt, (size_t)t * H + h);
      swiglu_ffn(ex->ws_gate, ex->ws_up, ex->ws_down, ex->wdt, 0, Is, H, xr, a, yr);
    } else {
      for (int h = 0; h < H; ++h) yr[h] = 0.0;
    }
    for (int j = 0; j < K; ++j) {
      double wj = (double)w[(size_t)t * K + j];
      const double* o = pair_out + ((size_t)t * K + j) * H;
      for (int h = 0; h < H; ++h) yr[h] += wj * o[h];
    }
  }
  free(xr);
  free(a);
  free(counts);
  free(offsets);
  free(sorted_pair);
  free(pair_slot);
  free(pair_out);
}

/* ------------------------------------------------------------------------ */
/* a9: RMSNorm (layer stack only; not described on the pages)              */
/* ------------------------------------------------------------------------ */
void orc_rmsnorm(int T, int H, const void* x, int xdt, double eps, double* r) {
  for (int t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int h = 0; h < H; ++h) {
      double v = elem(x, xdt, (size_t)t * H + h);
      ss += v * v;
    }
    double inv = 1.0 / sqrt(ss / (double)H + eps);
    for (int h = 0; h < H; ++h) r[(size_t)t * H + h] = elem(x, xdt, (size_t)t * H + h) * inv;
  }
}

/* ------------------------------------------------------------------------ */
/* Load balancing: hit tracking, its statistics, the expert-bias update and */
/* the auxiliary loss                                                        */
/* ------------------------------------------------------------------------ */

/* [Routing §六]: with tracking on, every routing call adds each expert's hits
 * (a bincount of the chosen indices) to a running per-layer count.  Written
 * as one pass over the pairs per expert, independently of orc_permute. */
void orc_track(int T, int K, int E, const int32_t* idx, int64_t* tracking) {
  int64_t P = (int64_t)T * K;
  for (int e = 0; e < E; ++e) {
    int64_t n = 0;
    for (int64_t p = 0; p < P; ++p)
      if (idx[p] == e) n += 1;
    tracking[e] += n;
  }
}

/* [Routing §六] / [Pitfalls, MoE 负载均衡 Loss 别忘加]: the load histogram of
 * each layer's tracked hits h[e], as loads relative to the balanced share
 * (load[e] = h[e] * E / N, N = sum of h; 1 = balanced) and a summary row:
 *   0 N, 1 max load, 2 min load, 3 coefficient of variation
 *   sqrt(mean_e (h[e] - N/E)^2) / (N/E), 4 experts with no hit, 5 the most
 *   and 6 the least hit expert (lowest index on ties), 7 the largest group
 *   load, sum of a group's hits * n_group / N.
 * With N = 0 every ratio is 0, the idle count is E and both indices are 0. */
void orc_expert_stats(int L, int E, int n_group, const int64_t* tracking, float* load,
                      double* summary) {
  int gsize = E / n_group;
  for (int l = 0; l < L; ++l) {
    const int64_t* h = tracking + (size_t)l * E;
    double* s = summary + (size_t)l * ORC_NSTAT;
    int64_t N = 0, idle = 0;
    int hot = 0, cold = 0;
    for (int e = 0; e < E; ++e) {
      N += h[e];
      if (h[e] == 0) idle += 1;
      if (h[e] > h[hot]) hot = e;
      if (h[e] < h[cold]) cold = e;
    }
    int64_t gmax = 0;
    for (int g = 0; g < n_group; ++g) {
      int64_t sg = 0;
      for (int e = g * gsize; e < (g + 1) * gsize; ++e) sg += h[e];
      if (sg > gmax) gmax = sg;
    }
    s[0] = (double)N;
    s[4] = (double)idle;
    s[5] = (double)hot;
    s[6] = (double)cold;
    if (N == 0) {
      for (int e = 0; e < E; ++e) load[(size_t)l * E + e] = 0.0f;
      s[1] = s[2] = s[3] = s[7] = 0.0;
      continue;
    }
    for (int e = 0; e < E; ++e)
      load[(size_t)l * E + e] = (float)((double)(h[e] * E) / (double)N);
    s[1] = (double)(h[hot] * E) / (double)N;
    s[2] = (double)(h[cold] * E) / (double)N;
    double mean = (double)N / (double)E, ss = 0.0;
    for (int e = 0; e < E; ++e) {
      double dv = (double)h[e] - mean;
      ss += dv * dv;
    }
    s[3] = sqrt(ss / (double)E) / mean;
    s[7] = (double)(gmax * n_group) / (double)N;
  }
}

/* [Routing §三]: during training the bias is raised for experts that receive
 * few tokens and lowered for experts that receive many, steering tokens
 * toward idle experts; the weights never see it.  The page gives no rule; the
 * one used here moves each bias against its expert's hit excess, normalised
 * by the largest excess:
 *   cbar = sum(counts) / E,  d = max(max_e |counts[e] - cbar|, 1),
 *   bias_out[e] = RN32(bias_in[e] + (-rate * (counts[e] - cbar)) / d)
 * in fp64.  From a zero bias with rate 0.1 this is the partly rebalancing
 * bias of the skewed-routing workload. */
void orc_bias_update(int E, const int32_t* counts, const float* bias_in, float* bias_out,
                     double rate) {
  int64_t N = 0;
  for (int e = 0; e < E; ++e) N += counts[e];
  double cbar = (double)N / (double)E;
  double d = 1.0;
  for (int e = 0; e < E; ++e) {
    double ex = fabs((double)counts[e] - cbar);
    if (ex > d) d = ex;
  }
  for (int e = 0; e < E; ++e) {
    double v = (-rate * ((double)counts[e] - cbar)) / d;
    bias_out[e] = (float)((double)bias_in[e] + v);
  }
}

/* [Pitfalls, MoE 负载均衡 Loss 别忘加]: the classic load-balancing loss
 * E * sum_i f_i * P_i from the router logits the forward returns.
 *   f_i = counts[i] / T, the fraction of tokens sent to expert i (the counts
 *         of the routing actually taken; sum_i f_i = K),
 *   P_i = (1/T) sum_t softmax(lam[t])_i, the mean router probability.
 * fp64 throughout (exp from libm); T >= 1. */
void orc_aux_loss(int T, int E, const float* lam, const int32_t* counts, double* f, double* P,
                  double* loss) {
  double* p = (double*)malloc(sizeof(double) * (size_t)E);
  for (int e = 0; e < E; ++e) P[e] = 0.0;
  for (int t = 0; t < T; ++t) {
    const float* l = lam + (size_t)t * E;
    double m = (double)l[0];
    for (int e = 1; e < E; ++e)
      if ((double)l[e] > m) m = (double)l[e];
    double z = 0.0;
    for (int e = 0; e < E; ++e) {
      p[e] = exp((double)l[e] - m);
      z += p[e];
    }
    for (int e = 0; e < E; ++e) P[e] += p[e] / z;
  }
  double acc = 0.0;
  for (int e = 0; e < E; ++e) {
    P[e] = P[e] / (double)T;
    f[e] = (double)counts[e] / (double)T;
    acc += f[e] * P[e];
  }
  *loss = (double)E * acc;
  free(p);
}

/* ------------------------------------------------------------------------ */
/* Backward of the layer for a fixed routing                                */
/* ------------------------------------------------------------------------ */
/* The layer's output as a function of its inputs and weights, with the
 * chosen experts held fixed (the choice is piecewise constant in the inputs,
 * so it carries no gradient; the expert bias only enters the choice and so
 * has none either):
 *   lam[t][e] = sum_h x[t][h] * W_r[e][h]                        [Routing §二 step 1]
 *   s = 1 / (1 + exp(-lam))                                       (the logistic sigmoid)
 *   w_j = scale * s_{idx_j} / (sum_k s_{idx_k} + 1e-20)           [Routing §二 step 3]
 *   y[t] = shared(x[t]) + sum_j w_j * expert_{idx_j}(x[t])        [Routing §四, §五]
 *   expert(x) = down(silu(gate x) * (up x)), silu(z) = z / (1 + exp(-z))
 * and, for an upstream gradient dy, the loss L = sum_{t,h} dy[t][h] * y[t][h].
 * Everything here is fp64 with the exact logistic function (the forward's
 * fp32 rounding of the scores is not part of what is differentiated).  The
 * derivatives, written out step by step below, follow from the chain rule:
 *   dL/dw_j   = <dy, expert_j(x)>,  d_o = w_j * dy (the expert's output grad)
 *   d_a_i     = sum_h W_down[i][h] * d_o_h;  dW_down[i][h] += a_i * d_o_h
 *   d_g_i     = d_a_i * u_i * silu'(g_i),  silu'(g) = sig(g) * (1 + g * (1 - sig(g)))
 *   d_u_i     = d_a_i * silu(g_i)
 *   dW_gate[i][h] += d_g_i * x_h,  dW_up[i][h] += d_u_i * x_h
 *   dx_h     += sum_i d_g_i * W_gate[i][h] + d_u_i * W_up[i][h]
 *   dL/ds_m   = scale / D * (dL/dw_m - sum_j dL/dw_j * s_j / D),  D = sum s + 1e-20
 *               (quotient rule; m over the chosen experts)
 *   dL/dlam_m = dL/ds_m * s_m * (1 - s_m) (chosen m; 0 for the others)
 *   dW_r[m][h] += dL/dlam_m * x_h,  dx_h += sum_m dL/dlam_m * W_r[m][h]   */

static double logistic(double z) { return 1.0 / (1.0 + exp(-z)); }

/* One expert on one token row: g, u, a (= silu(g) u) and the output o. */
static void expert_fwd(const void* wg, const void* wu, const void* wd, int wdt, size_t base, int I,
                       int H, const double* xr, double* g, double* u, double* a, double* o) {
  for (int i = 0; i < I; ++i) {
    size_t row = base + (size_t)i * H;
    double gi = 0.0, ui = 0.0;
    for (int h = 0; h < H; ++h) gi += xr[h] * elem(wg, wdt, row + h);
    for (int h = 0; h < H; ++h) ui += xr[h] * elem(wu, wdt, row + h);
    g[i] = gi;
    u[i] = ui;
    a[i] = gi * logistic(gi) * ui;
  }
  if (o) {
    for (int h = 0; h < H; ++h) o[h] = 0.0;
    for (int i = 0; i < I; ++i) {
      size_t row = base + (size_t)i * H;
      for (int h = 0; h < H; ++h) o[h] += a[i] * elem(wd, wdt, row + h);
    }
  }
}

/* Given d_o (the gradient of the expert's output), the gradients of g and u. */
static void expert_bwd_act(const void* wd, int wdt, size_t base, int I, int H, const double* d_o,
                           const double* g, const double* u, double* dg, double* du) {
  for (int i = 0; i < I; ++i) {
    size_t row = base + (size_t)i * H;
    double da = 0.0;
    for (int h = 0; h < H; ++h) da += elem(wd, wdt, row + h) * d_o[h];
    double sg = logistic(g[i]);
    double silu = g[i] * sg;
    double dsilu = sg * (1.0 + g[i] * (1.0 - sg));
    dg[i] = da * u[i] * dsilu;
    du[i] = da * silu;
  }
}

/* The chosen experts' scores and the routing weights of one token. */
static double token_weights(int K, const int32_t* idx, const double* lam, double scale, double* s,
                            double* w) {
  double S = 0.0;
  for (int j = 0; j < K; ++j) {
    s[j] = logistic(lam[idx[j]]);
    S += s[j];
  }
  double D = S + 1e-20;
  for (int j = 0; j < K; ++j) w[j] = scale * s[j] / D;
  return D;
}

typedef struct {
  const orc_experts_t* ex;
  int T, E, rdt, xdt;
  const void* x;
  const void* w_router;
  const double* lam;
  const int32_t* idx;
  double scale;
  const double* dy;
  const int32_t* tokens;
  double *dx, *dweight, *dlogit, *y;
} bwd_tok_ctx_t;

static void bwd_tokens_range(void* vctx, int r0, int r1) {
  bwd_tok_ctx_t* c = (bwd_tok_ctx_t*)vctx;
  const orc_experts_t* ex = c->ex;
  int H = ex->H, I = ex->I, Is = ex->I_shared, K = ex->K, E = c->E;
  int amax = I > Is ? I : Is;
  if (amax < 1) amax = 1;
  double* xr = (double*)malloc(sizeof(double) * (size_t)H);
  double* g = (double*)malloc(sizeof(double) * (size_t)amax);
  double* u = (double*)malloc(sizeof(double) * (size_t)amax);
  double* a = (double*)malloc(sizeof(double) * (size_t)amax);
  double* dg = (double*)malloc(sizeof(double) * (size_t)amax);
  double* du = (double*)malloc(sizeof(double) * (size_t)amax);
  double* o = (double*)malloc(sizeof(double) * (size_t)H);
  double* d_o = (double*)malloc(sizeof(double) * (size_t)H);
  double* s = (double*)malloc(sizeof(double) * (size_t)K);
  double* wj = (double*)malloc(sizeof(double) * (size_t)K);
  double* gw = (double*)malloc(sizeof(double) * (size_t)K);
  for (int r = r0; r < r1; ++r) {
    int t = c->tokens ? c->tokens[r] : r;
    const double* dy = c->dy + (size_t)t * H;
    const int32_t* it = c->idx + (size_t)t * K;
    double* dx = c->dx ? c->dx + (size_t)r * H : NULL;
    double* yr = c->y ? c->y + (size_t)r * H : NULL;
    for (int h = 0; h < H; ++h) xr[h] = elem(c->x, c->xdt, (size_t)t * H + h);
    if (dx)
      for (int h = 0; h < H; ++h) dx[h] = 0.0;
    if (yr)
      for (int h = 0; h < H; ++h) yr[h] = 0.0;
    double D = token_weights(K, it, c->lam + (size_t)t * E, c->scale, s, wj);
    /* shared expert, weight 1 */
    if (Is > 0 && ex->ws_gate) {
      expert_fwd(ex->ws_gate, ex->ws_up, ex->ws_down, ex->wdt, 0, Is, H, xr, g, u, a, o);
      if (yr)
        for (int h = 0; h < H; ++h) yr[h] += o[h];
      if (dx) {
        expert_bwd_act(ex->ws_down, ex->wdt, 0, Is, H, dy, g, u, dg, du);
        for (int i = 0; i < Is; ++i)
          for (int h = 0; h < H; ++h)
            dx[h] += dg[i] * elem(ex->ws_gate, ex->wdt, (size_t)i * H + h) +
                     du[i] * elem(ex->ws_up, ex->wdt, (size_t)i * H + h);
      }
    }
    /* routed experts, in j order */
    for (int j = 0; j < K; ++j) {
      size_t base = (size_t)it[j] * I * H;
      expert_fwd(ex->w_gate, ex->w_up, ex->w_down, ex->wdt, base, I, H, xr, g, u, a, o);
      double d = 0.0;
      for (int h = 0; h < H; ++h) d += dy[h] * o[h];
      gw[j] = d;
      if (yr)
        for (int h = 0; h < H; ++h) yr[h] += wj[j] * o[h];
      if (dx) {
        for (int h = 0; h < H; ++h) d_o[h] = wj[j] * dy[h];
        expert_bwd_act(ex->w_down, ex->wdt, base, I, H, d_o, g, u, dg, du);
        for (int i = 0; i < I; ++i)
          for (int h = 0; h < H; ++h)
            dx[h] += dg[i] * elem(ex->w_gate, ex->wdt, base + (size_t)i * H + h) +
                     du[i] * elem(ex->w_up, ex->wdt, base + (size_t)i * H + h);
      }
    }
    /* router: quotient rule through the normalised weights, then the sigmoid */
    double sgs = 0.0;
    for (int j = 0; j < K; ++j) sgs += gw[j] * s[j];
    double* dl = c->dlogit ? c->dlogit + (size_t)r * E : NULL;
    if (dl)
      for (int e = 0; e < E; ++e) dl[e] = 0.0;
    for (int j = 0; j < K; ++j) {
      double ds = c->scale / D * (gw[j] - sgs / D);
      double dlam = ds * s[j] * (1.0 - s[j]);
      if (dl) dl[it[j]] = dlam;
      if (dx)
        for (int h = 0; h < H; ++h)
          dx[h] += dlam * elem(c->w_router, c->rdt, (size_t)it[j] * H + h);
    }
    if (c->dweight)
      for (int j = 0; j < K; ++j) c->dweight[(size_t)r * K + j] = gw[j];
  }
  free(xr); free(g); free(u); free(a); free(dg); free(du); free(o); free(d_o);
  free(s); free(wj); free(gw);
}

void orc_backward_tokens(const orc_experts_t* ex, int T, int E, const void* x, int xdt,
                         const void* w_router, int rdt, const double* lam, const int32_t* idx,
                         double scale, const double* dy, const int32_t* tokens, int n_tok,
                         double* dx, double* dweight, double* dlogit, double* y, int nthreads) {
  bwd_tok_ctx_t c = {ex, T, E, rdt, xdt, x, w_router, lam, idx, scale, dy, tokens,
                     dx, dweight, dlogit, y};
  parallel_range(bwd_tokens_range, &c, n_tok, nthreads);
}

/* Weight gradients of one expert (e < E: routed, over its pairs in token
 * order; e == E: the shared expert, over every token).  The per-pair vectors
 * a, d_o, d_g, d_u are formed first (in parallel over pairs), then each
 * gradient row is summed over the pairs in order (in parallel over rows). */
typedef struct {
  const orc_experts_t* ex;
  int E, xdt, np, e;
  const void* x;
  const double* lam;
  const int32_t* idx;
  double scale;
  const double* dy;
  const int32_t* ptok; /* token of each pair */
  const int32_t* pj;   /* slot j of each pair (-1: shared) */
  double *A, *DO, *DG, *DU;
} bwd_pair_ctx_t;

static void bwd_pairs_range(void* vctx, int p0, int p1) {
  bwd_pair_ctx_t* c = (bwd_pair_ctx_t*)vctx;
  const orc_experts_t* ex = c->ex;
  int H = ex->H, K = ex->K;
  int shared = c->e >= c->E;
  int I = shared ? ex->I_shared : ex->I;
  const void* wg = shared ? ex->ws_gate : ex->w_gate;
  const void* wu = shared ? ex->ws_up : ex->w_up;
  const void* wd = shared ? ex->ws_down : ex->w_down;
  size_t base = shared ? 0 : (size_t)c->e * I * H;
  double* xr = (double*)malloc(sizeof(double) * (size_t)H);
  double* g = (double*)malloc(sizeof(double) * (size_t)I);
  double* u = (double*)malloc(sizeof(double) * (size_t)I);
  double* s = (double*)malloc(sizeof(double) * (size_t)K);
  double* wj = (double*)malloc(sizeof(double) * (size_t)K);
  for (int p = p0; p < p1; ++p) {
    int t = c->ptok[p];
    for (int h = 0; h < H; ++h) xr[h] = elem(c->x, c->xdt, (size_t)t * H + h);
    double w = 1.0;
    if (!shared) {
      token_weights(K, c->idx + (size_t)t * K, c->lam + (size_t)t * c->E, c->scale, s, wj);
      w = wj[c->pj[p]];
    }
    double* a = c->A + (size_t)p * I;
    double* d_o = c->DO + (size_t)p * H;
    expert_fwd(wg, wu, wd, ex->wdt, base, I, H, xr, g, u, a, NULL);
    for (int h = 0; h < H; ++h) d_o[h] = w * c->dy[(size_t)t * H + h];
    expert_bwd_act(wd, ex->wdt, base, I, H, d_o, g, u, c->DG + (size_t)p * I,
                   c->DU + (size_t)p * I);
  }
  free(xr); free(g); free(u); free(s); free(wj);
}

typedef struct {
  int H, I, np, xdt;
  const void* x;
  const int32_t* ptok;
  const double *A, *DO, *DG, *DU;
  double *dwg, *dwu, *dwd;
} bwd_rows_ctx_t;

static void bwd_rows_range(void* vctx, int i0, int i1) {
  bwd_rows_ctx_t* c = (bwd_rows_ctx_t*)vctx;
  int H = c->H, I = c->I;
  for (int i = i0; i < i1; ++i) {
    double* rg = c->dwg + (size_t)i * H;
    double* ru = c->dwu + (size_t)i * H;
    double* rd = c->dwd + (size_t)i * H;
    for (int h = 0; h < H; ++h) rg[h] = ru[h] = rd[h] = 0.0;
    for (int p = 0; p < c->np; ++p) {
      int t = c->ptok[p];
      double ai = c->A[(size_t)p * I + i];
      double gi = c->DG[(size_t)p * I + i];
      double ui = c->DU[(size_t)p * I + i];
      const double* d_o = c->DO + (size_t)p * H;
      for (int h = 0; h < H; ++h) {
        double xh = elem(c->x, c->xdt, (size_t)t * H + h);
        rg[h] += gi * xh;
        ru[h] += ui * xh;
        rd[h] += ai * d_o[h];
      }
    }
  }
}

void orc_backward_expert_weights(const orc_experts_t* ex, int T, int E, const void* x, int xdt,
                                 const double* lam, const int32_t* idx, double scale,
                                 const double* dy, int e, double* dwg, double* dwu, double* dwd,
                                 int nthreads) {
  int K = ex->K, H = ex->H;
  int shared = e >= E;
  int I = shared ? ex->I_shared : ex->I;
  int np = 0;
  int64_t P = (int64_t)T * K;
  int32_t* ptok = (int32_t*)malloc(sizeof(int32_t) * (size_t)(shared ? (T > 0 ? T : 1) : (P > 0 ? P : 1)));
  int32_t* pj = (int32_t*)malloc(sizeof(int32_t) * (size_t)(shared ? (T > 0 ? T : 1) : (P > 0 ? P : 1)));
  if (shared) {
    for (int t = 0; t < T; ++t) { ptok[np] = t; pj[np] = -1; ++np; }
  } else {
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < K; ++j)
        if (idx[(size_t)t * K + j] == e) { ptok[np] = t; pj[np] = j; ++np; }
  }
  size_t npp = np > 0 ? (size_t)np : 1;
  double* A = (double*)malloc(sizeof(double) * npp * (size_t)I);
  double* DG = (double*)malloc(sizeof(double) * npp * (size_t)I);
  double* DU = (double*)malloc(sizeof(double) * npp * (size_t)I);
  double* DO = (double*)malloc(sizeof(double) * npp * (size_t)H);
  bwd_pair_ctx_t pc = {ex, E, xdt, np, e, x, lam, idx, scale, dy, ptok, pj, A, DO, DG, DU};
  parallel_range(bwd_pairs_range, &pc, np, nthreads);
  bwd_rows_ctx_t rc = {H, I, np, xdt, x, ptok, A, DO, DG, DU, dwg, dwu, dwd};
  parallel_range(bwd_rows_range, &rc, I, nthreads);
  free(ptok); free(pj); free(A); free(DG); free(DU); free(DO);
}

/* dW_r[e][h] = sum_t dlogit[t][e] * x[t][h], summed over t in order. */
void orc_router_weight_grad(int T, int E, int H, const void* x, int xdt, const double* dlogit,
                            double* dwr) {
  for (size_t i = 0; i < (size_t)E * H; ++i) dwr[i] = 0.0;
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double d = dlogit[(size_t)t * E + e];
      if (d == 0.0) continue;
      for (int h = 0; h < H; ++h) dwr[(size_t)e * H + h] += d * elem(x, xdt, (size_t)t * H + h);
    }
}

/* lam[t][e] = sum_h x[t][h] * W_r[e][h] in fp64 from inputs of any dtype. */
void orc_logits_any(int T, int H, int E, const void* x, int xdt, const void* w_router, int rdt,
                    double* lam) {
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h)
        acc += elem(x, xdt, (size_t)t * H + h) * elem(w_router, rdt, (size_t)e * H + h);
      lam[(size_t)t * E + e] = acc;
    }
}
