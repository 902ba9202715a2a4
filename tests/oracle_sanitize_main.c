/* Driver for the sanitizer builds of the oracle (tests/test_oracle_sanitize.py): calls every
 * oracle entry point on a tiny problem with pseudo-random inputs, so that AddressSanitizer,
 * UndefinedBehaviorSanitizer and ThreadSanitizer builds see every code path, including the
 * threaded ones.  It checks return codes only; the values are checked by the other tests. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "prism_oracle.h"

static uint64_t lcg_state = 0x9e3779b97f4a7c15ull;

static float urand(void) {
  lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((lcg_state >> 40) * (1.0 / 16777216.0)) * 2.0f - 1.0f;
}

static void fill(float* x, size_t n) {
  for (size_t i = 0; i < n; ++i) x[i] = urand();
}

#define CHECK(call)                                                    \
  do {                                                                 \
    int rc_ = (call);                                                  \
    if (rc_ < 0) {                                                     \
      fprintf(stderr, "%s returned %d (line %d)\n", #call, rc_, __LINE__); \
      return 1;                                                        \
    }                                                                  \
  } while (0)

int main(void) {
  const int T = 8, H = 16, W = 16, heads = 2, d = 16, groups = 1, nth = 2;
  const int N = T * H * W, Z = N / 512, NB = 8 * Z;
  const double eps = 1e-6, sm = 1.0;
  int32_t edges[48], vol[16];
  CHECK(orc_candidates(edges, vol));

  float* q = malloc(sizeof(float) * N * heads * d);
  float* k = malloc(sizeof(float) * N * heads * d);
  float* v = malloc(sizeof(float) * N * heads * d);
  float* dout = malloc(sizeof(float) * N * heads * d);
  float* a = malloc(sizeof(float) * N);
  fill(q, (size_t)N * heads * d);
  fill(k, (size_t)N * heads * d);
  fill(v, (size_t)N * heads * d);
  fill(dout, (size_t)N * heads * d);
  for (int i = 0; i < N; ++i) a[i] = fabsf(urand());

  double *sig2 = malloc(sizeof(double) * groups * Z * 4), *r = malloc(sizeof(double) * groups * Z * 3);
  double *rho = malloc(sizeof(double) * groups * Z), *abar = malloc(sizeof(double) * Z);
  double *vhat = malloc(sizeof(double) * Z * 3), *g = malloc(sizeof(double) * groups * Z * 3);
  for (int with_audio = 0; with_audio < 2; ++with_audio)
    CHECK(orc_zone_stats(T, H, W, heads, d, groups, v, with_audio ? a : NULL, eps, sig2, r, rho, abar, vhat, g,
                         nth));

  int32_t* volume = malloc(sizeof(int32_t) * groups * Z);
  double* lstar = malloc(sizeof(double) * groups * Z * 3);
  double* dist = malloc(sizeof(double) * groups * Z * 16);
  uint8_t* shape_idx = malloc((size_t)groups * Z);
  int32_t* zbo = malloc(sizeof(int32_t) * groups * (Z + 1));
  CHECK(orc_assign_shapes(groups, Z, g, rho, 0.5, 0.25, volume, lstar, dist, shape_idx, zbo));

  int64_t* pos = malloc(sizeof(int64_t) * groups * N);
  int32_t* bs = malloc(sizeof(int32_t) * groups * (NB + 1));
  int32_t* nblocks = malloc(sizeof(int32_t) * groups);
  CHECK(orc_block_layout(T, H, W, groups, shape_idx, pos, bs, nblocks));

  /* block-order copies: the oracle's permutation is pos; this program only moves rows */
  float* qp = malloc(sizeof(float) * heads * N * d);
  float* kp = malloc(sizeof(float) * heads * N * d);
  float* vp = malloc(sizeof(float) * heads * N * d);
  float* dop = malloc(sizeof(float) * heads * N * d);
  for (int h = 0; h < heads; ++h)
    for (int n = 0; n < N; ++n) {
      const int64_t pr = pos[n];
      memcpy(qp + ((size_t)h * N + pr) * d, q + ((size_t)n * heads + h) * d, sizeof(float) * d);
      memcpy(kp + ((size_t)h * N + pr) * d, k + ((size_t)n * heads + h) * d, sizeof(float) * d);
      memcpy(vp + ((size_t)h * N + pr) * d, v + ((size_t)n * heads + h) * d, sizeof(float) * d);
      memcpy(dop + ((size_t)h * N + pr) * d, dout + ((size_t)n * heads + h) * d, sizeof(float) * d);
    }

  double* qbar = malloc(sizeof(double) * heads * NB * d);
  double* kbar = malloc(sizeof(double) * heads * NB * d);
  CHECK(orc_pool(heads, groups, N, d, NB, bs, nblocks, qp, qbar, nth));
  CHECK(orc_pool(heads, groups, N, d, NB, bs, nblocks, kp, kbar, nth));

  int32_t* cnt = malloc(sizeof(int32_t) * heads * NB);
  int32_t* idx = malloc(sizeof(int32_t) * heads * NB * NB);
  double* info = malloc(sizeof(double) * heads * NB * 5);
  uint8_t* mask = calloc((size_t)heads * NB, 1);
  for (int i = 0; i < heads * NB; i += 3) mask[i] = 1;
  CHECK(orc_select(heads, groups, d, NB, nblocks, qbar, kbar, sm, 2, 0.0, 0.9, NULL, cnt, idx, info, nth));
  CHECK(orc_select(heads, groups, d, NB, nblocks, qbar, kbar, sm, 0, 0.3, 0.0, mask, cnt, idx, info, nth));
  CHECK(orc_select(heads, groups, d, NB, nblocks, qbar, kbar, sm, 0, 0.05, 1.0, NULL, cnt, idx, info, nth));

  double* o = malloc(sizeof(double) * heads * N * d);
  double* lse = malloc(sizeof(double) * heads * N);
  double* delta = malloc(sizeof(double) * heads * N);
  double* dq = malloc(sizeof(double) * heads * N * d);
  double* dk = malloc(sizeof(double) * heads * N * d);
  double* dv = malloc(sizeof(double) * heads * N * d);
  CHECK(orc_attn_fwd(heads, groups, N, d, NB, bs, nblocks, cnt, idx, sm, qp, kp, vp, NULL, o, lse, nth));
  CHECK(orc_attn_fwd(heads, groups, N, d, NB, bs, nblocks, cnt, idx, sm, qp, kp, vp, mask, o, lse, nth));
  CHECK(orc_attn_bwd(heads, groups, N, d, NB, bs, nblocks, cnt, idx, sm, qp, kp, vp, dop, NULL, NULL, dq, dk, dv, lse,
                     delta, nth));
  CHECK(orc_attn_bwd(heads, groups, N, d, NB, bs, nblocks, cnt, idx, sm, qp, kp, vp, dop, mask, mask, dq, dk, dv, lse,
                     delta, nth));

  double* an = malloc(sizeof(double) * N);
  CHECK(orc_audio_norms(N, heads * d, q, 0, an));
  CHECK(orc_audio_norms(N, heads * d, q, 1, an));

  /* bad arguments are rejected, not dereferenced */
  if (orc_zone_stats(7, H, W, heads, d, groups, v, NULL, eps, sig2, r, rho, abar, vhat, g, nth) >= 0) {
    fprintf(stderr, "bad grid accepted\n");
    return 1;
  }

  free(q); free(k); free(v); free(dout); free(a); free(sig2); free(r); free(rho); free(abar); free(vhat);
  free(g); free(volume); free(lstar); free(dist); free(shape_idx); free(zbo); free(pos); free(bs);
  free(nblocks); free(qp); free(kp); free(vp); free(dop); free(qbar); free(kbar); free(cnt); free(idx);
  free(info); free(mask); free(o); free(lse); free(delta); free(dq); free(dk); free(dv); free(an);
  printf("oracle driver ok\n");
  return 0;
}
