/* Host sanitizer driver for the oracle (built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_sanitizers.py): calls every
 * function oracle.h declares on small inputs of every dtype, with ragged
 * shapes, a bias, non-finite logits, token subsets and an empty expert, so
 * that an out-of-bounds access or undefined behaviour anywhere in oracle.c
 * is reported.  Exits 0 when the two expert paths agree and every call
 * returned; the sanitizers abort on a finding. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform(void) { /* xorshift64*, in [0, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (double)((rng_state * 0x2545f4914f6cdd1dull) >> 11) * 0x1.0p-53;
}
static double normal(void) {
  double u = uniform() + 1e-300, v = uniform();
  return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) abort();
  return p;
}

/* one layer of every dtype; returns the largest |path A - path B| */
static double layer(int T, int H, int E, int G, int KG, int K, int I, int Is, int dt) {
  const size_t es = dt == ORC_F32 ? 4 : dt == ORC_BF16 ? 2 : 8;
  void* x = xmalloc((size_t)T * H * es);
  float* wr = (float*)xmalloc((size_t)E * H * 4);
  float* bias = (float*)xmalloc((size_t)E * 4);
  void* wg = xmalloc((size_t)E * I * H * es);
  void* wu = xmalloc((size_t)E * I * H * es);
  void* wd = xmalloc((size_t)E * I * H * es);
  void* sg = Is ? xmalloc((size_t)Is * H * es) : NULL;
  void* su = Is ? xmalloc((size_t)Is * H * es) : NULL;
  void* sd = Is ? xmalloc((size_t)Is * H * es) : NULL;
  void* arrs[] = {x, wg, wu, wd, sg, su, sd};
  size_t lens[] = {(size_t)T * H, (size_t)E * I * H, (size_t)E * I * H, (size_t)E * I * H,
                   (size_t)Is * H, (size_t)Is * H, (size_t)Is * H};
  for (int a = 0; a < 7; ++a) {
    if (!arrs[a]) continue;
    for (size_t i = 0; i < lens[a]; ++i) {
      double v = (a == 0 ? 1.0 : 0.05) * normal();
      if (dt == ORC_F32) ((float*)arrs[a])[i] = (float)v;
      else if (dt == ORC_BF16) ((uint16_t*)arrs[a])[i] = to_bf16((float)v);
      else ((double*)arrs[a])[i] = v;
    }
  }
  for (size_t i = 0; i < (size_t)E * H; ++i) wr[i] = (float)(normal() / sqrt((double)H));
  for (int e = 0; e < E; ++e) bias[e] = (float)(0.05 * normal());
  int xdt = dt == ORC_F64 ? ORC_F32 : dt; /* the forward takes fp32 or bf16 activations */
  float* xf = NULL;
  const void* xin = x;
  if (dt == ORC_F64) { /* an fp32 copy for the forward */
    xf = (float*)xmalloc((size_t)T * H * 4);
    for (size_t i = 0; i < (size_t)T * H; ++i) xf[i] = (float)((double*)x)[i];
    xin = xf;
  }
  double* l64 = (double*)xmalloc((size_t)T * E * 8);
  orc_logits(T, H, E, xin, xdt, wr, l64, 3);
  float* lam = (float*)xmalloc((size_t)T * E * 4);
  for (size_t i = 0; i < (size_t)T * E; ++i) lam[i] = (float)l64[i];
  if (T > 2) {
    lam[E + 1] = NAN; /* token 1: a non-finite logit */
    lam[2 * E] = INFINITY;
  }
  int32_t* idx = (int32_t*)xmalloc((size_t)T * K * 4);
  float* w = (float*)xmalloc((size_t)T * K * 4);
  uint8_t* flag = (uint8_t*)xmalloc((size_t)T);
  orc_select(T, E, G, KG, K, 2.5f, lam, bias, idx, w, flag);
  orc_select(T, E, G, KG, K, 2.5f, lam, NULL, idx, w, flag);
  for (int t = 0; t < T; ++t)
    if (flag[t])
      for (int j = 0; j < K; ++j) { /* give flagged tokens a valid routing */
        idx[(size_t)t * K + j] = j;
        w[(size_t)t * K + j] = 0.1f;
      }
  uint8_t* dec = (uint8_t*)xmalloc((size_t)T);
  float* sbl = (float*)xmalloc((size_t)T * E * 4);
  float* sbh = (float*)xmalloc((size_t)T * E * 4);
  float* gl = (float*)xmalloc((size_t)T * G * 4);
  float* gh = (float*)xmalloc((size_t)T * G * 4);
  orc_route_intervals(T, E, G, KG, K, l64, 2e-5, 4e-6, bias, idx, dec, sbl, sbh, gl, gh);
  orc_route_intervals(T, E, G, KG, K, l64, 2e-5, 0.0, NULL, idx, dec, NULL, NULL, NULL, NULL);
  int32_t* counts = (int32_t*)xmalloc((size_t)E * 4);
  int32_t* offs = (int32_t*)xmalloc((size_t)(E + 1) * 4);
  int32_t* sp = (int32_t*)xmalloc((size_t)T * K * 4);
  int32_t* ps = (int32_t*)xmalloc((size_t)T * K * 4);
  orc_permute(T, K, E, idx, counts, offs, sp, ps);
  int64_t* track = (int64_t*)calloc((size_t)E, 8);
  orc_track(T, K, E, idx, track);
  float* load = (float*)xmalloc((size_t)E * 4);
  double summ[ORC_NSTAT];
  orc_expert_stats(1, E, G, track, load, summ);
  float* nb = (float*)xmalloc((size_t)E * 4);
  orc_bias_update(E, counts, bias, nb, 0.1);
  double* f = (double*)xmalloc((size_t)E * 8);
  double* P = (double*)xmalloc((size_t)E * 8);
  double loss;
  for (size_t i = 0; i < (size_t)T * E; ++i) lam[i] = (float)l64[i];
  orc_aux_loss(T, E, lam, counts, f, P, &loss);
  int wdt = dt == ORC_F64 ? ORC_F32 : dt;
  if (dt == ORC_F64) { /* fp32 copies of the expert weights */
    for (int a = 1; a < 7; ++a) {
      if (!arrs[a]) continue;
      float* c = (float*)xmalloc(lens[a] * 4);
      for (size_t i = 0; i < lens[a]; ++i) c[i] = (float)((double*)arrs[a])[i];
      free(arrs[a]);
      arrs[a] = c;
    }
    wg = arrs[1], wu = arrs[2], wd = arrs[3], sg = arrs[4], su = arrs[5], sd = arrs[6];
  }
  orc_experts_t ex = {H, I, Is, E, K, wdt, wg, wu, wd, sg, su, sd};
  double* ya = (double*)xmalloc((size_t)(T > 3 ? T : 3) * H * 8); /* also 3 token rows below */
  double* yb = (double*)xmalloc((size_t)T * H * 8);
  orc_experts_path_a(&ex, xin, xdt, idx, w, NULL, T, ya, 2);
  orc_experts_path_b(&ex, T, xin, xdt, idx, w, yb, 2);
  double worst = 0.0;
  for (size_t i = 0; i < (size_t)T * H; ++i) worst = fmax(worst, fabs(ya[i] - yb[i]));
  int32_t tok[3] = {T - 1, 0, T / 2};
  orc_experts_path_a(&ex, xin, xdt, idx, w, tok, 3, ya, 1);
  double* r = (double*)xmalloc((size_t)T * H * 8);
  orc_rmsnorm(T, H, xin, xdt, 1e-6, r);
  /* backward (activations and router weight of any dtype) */
  double* dy = (double*)xmalloc((size_t)T * H * 8);
  for (size_t i = 0; i < (size_t)T * H; ++i) dy[i] = normal();
  double* lam_any = (double*)xmalloc((size_t)T * E * 8);
  orc_logits_any(T, H, E, x, dt, wr, ORC_F32, lam_any);
  double* dx = (double*)xmalloc((size_t)(T > 3 ? T : 3) * H * 8);
  double* dwt = (double*)xmalloc((size_t)T * K * 8);
  double* dl = (double*)xmalloc((size_t)T * E * 8);
  orc_backward_tokens(&ex, T, E, xin, xdt, wr, ORC_F32, l64, idx, 2.5, dy, NULL, T, dx, dwt, dl,
                      ya, 2);
  orc_backward_tokens(&ex, T, E, xin, xdt, wr, ORC_F32, l64, idx, 2.5, dy, tok, 3, dx, NULL,
                      NULL, NULL, 1);
  int Iw = I > Is ? I : Is;
  double* g1 = (double*)xmalloc((size_t)Iw * H * 8);
  double* g2 = (double*)xmalloc((size_t)Iw * H * 8);
  double* g3 = (double*)xmalloc((size_t)Iw * H * 8);
  orc_backward_expert_weights(&ex, T, E, xin, xdt, l64, idx, 2.5, dy, idx[0], g1, g2, g3, 2);
  if (Is) orc_backward_expert_weights(&ex, T, E, xin, xdt, l64, idx, 2.5, dy, E, g1, g2, g3, 2);
  double* dwr = (double*)xmalloc((size_t)E * H * 8);
  orc_router_weight_grad(T, E, H, xin, xdt, dl, dwr);
  void* frees[] = {x,  wr, bias, wg, wu,  wd,  sg, su, sd, xf, l64, lam, idx, w, flag, dec,
                   sbl, sbh, gl, gh, counts, offs, sp, ps, track, load, nb, f, P, ya, yb, r,
                   dy, lam_any, dx, dwt, dl, g1, g2, g3, dwr};
  for (size_t i = 0; i < sizeof frees / sizeof frees[0]; ++i) free(frees[i]);
  return worst;
}

int main(void) {
  /* sigma32 over a few ranges, a scan and a comparison */
  float z[7] = {0.0f, -0.0f, 1.5f, -104.5f, 40.5f, NAN, INFINITY}, s[7];
  orc_sigmoid32_array(z, s, 7);
  int64_t scan[4], cmp[2];
  orc_sigmoid32_scan(0x3f000000u, 0x3f000000u + 20000u, 7, 3, scan);
  orc_sigmoid32_scan(0xffffff00ull, 0x100000000ull, 1, 2, scan);
  float other[1000];
  float zz[1000];
  for (int i = 0; i < 1000; ++i) {
    uint32_t b = 0x7f7ffc00u + (uint32_t)i; /* runs past the largest finite value into inf/NaN */
    memcpy(&zz[i], &b, 4);
  }
  orc_sigmoid32_array(zz, other, 1000);
  orc_sigmoid32_compare(0x7f7ffc00u, 1000, other, 4, cmp);
  if (cmp[0] != 0) {
    fprintf(stderr, "sigma32 compare: %lld mismatches\n", (long long)cmp[0]);
    return 1;
  }
  /* layers: (T, H, E, groups, kept groups, k, I, I_shared, dtype) */
  const int cases[][9] = {
      {5, 64, 16, 4, 2, 4, 32, 32, ORC_F32},   {7, 64, 16, 4, 2, 4, 32, 0, ORC_BF16},
      {9, 32, 24, 3, 2, 5, 16, 48, ORC_F64},   {1, 32, 8, 1, 1, 8, 8, 8, ORC_BF16},
      {12, 48, 32, 8, 4, 8, 16, 16, ORC_F32},
  };
  for (size_t c = 0; c < sizeof cases / sizeof cases[0]; ++c) {
    const int* k = cases[c];
    double d = layer(k[0], k[1], k[2], k[3], k[4], k[5], k[6], k[7], k[8]);
    if (!(d == 0.0)) {
      fprintf(stderr, "case %zu: path A and path B differ by %g\n", c, d);
      return 1;
    }
  }
  printf("oracle sanitizer driver ok\n");
  return 0;
}
