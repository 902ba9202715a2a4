/* prism_oracle.c -- plain CPU reference of the Prism hot path (see prism_oracle.h).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the CPU-baseline leg
 * of the benchmark; never by the product path.
 *
 * Written for a reader to check against the pages by eye: one loop nest per formula, fp64
 * arithmetic, no blocking, fusion or reordering beyond what a formula states.  The only
 * parallelism is an outer split over independent zones / rows (pthreads), which changes no
 * arithmetic.
 */
#define _POSIX_C_SOURCE 200809L
#include "prism_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#define ZONE 8       /* Z_T = Z_H = Z_W = 8 (RG KI, macro-zone partitioning) */
#define ZVOL 512     /* tokens per zone */

/* ------------------------------------------------------------------------------------ */
/* a small parallel-for over [0, n): each worker takes chunks from a shared counter      */

typedef void (*task_fn)(void* ctx, int64_t i);
typedef struct { task_fn fn; void* ctx; int64_t n; int64_t next; } pool_t;

static void* pool_worker(void* arg) {
  pool_t* P = (pool_t*)arg;
  for (;;) {
    int64_t i = __atomic_fetch_add(&P->next, 1, __ATOMIC_RELAXED);
    if (i >= P->n) break;
    P->fn(P->ctx, i);
  }
  return NULL;
}

static void parallel_for(int nthreads, int64_t n, task_fn fn, void* ctx) {
  pool_t P = {fn, ctx, n, 0};
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads == 1 || n <= 1) { pool_worker(&P); return; }
  pthread_t th[256];
  int started = 0;
  for (int t = 0; t < nthreads; ++t)
    if (pthread_create(&th[t], NULL, pool_worker, &P) == 0) ++started;
  if (started == 0) pool_worker(&P);
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------------------ */
/* candidate set (RG KI: "16-shape candidate set", volumes {64,128,256}).                 */
/* Reading: edges are powers of two in {2,4,8}; that gives exactly 7 + 6 + 3 = 16 shapes. */

static int g_cand_edges[16][3];
static int g_cand_vol[16];
static int g_cand_n = 0;

static void build_candidates(void) {
  if (g_cand_n) return;
  static const int vols[3] = {64, 128, 256};
  static const int edge[3] = {2, 4, 8};
  int n = 0;
  for (int vi = 0; vi < 3; ++vi)
    for (int a = 0; a < 3; ++a)
      for (int b = 0; b < 3; ++b)
        for (int c = 0; c < 3; ++c)
          if (edge[a] * edge[b] * edge[c] == vols[vi] && n < 16) {
            g_cand_edges[n][0] = edge[a];
            g_cand_edges[n][1] = edge[b];
            g_cand_edges[n][2] = edge[c];
            g_cand_vol[n] = vols[vi];
            ++n;
          }
  g_cand_n = n;
}

int orc_candidates(int32_t* edges, int32_t* volume) {
  build_candidates();
  for (int i = 0; i < g_cand_n; ++i) {
    for (int e = 0; e < 3; ++e) edges[3 * i + e] = g_cand_edges[i][e];
    volume[i] = g_cand_vol[i];
  }
  return g_cand_n;
}

/* ------------------------------------------------------------------------------------ */
/* RG M1: zone statistics                                                                 */

typedef struct {
  int T, H, W, heads, d, groups;
  const float* v;
  double *sig2, *r, *rho;
} zs_ctx;

/* value of channel (head, e) at local zone coordinate (lt,lh,lw) of zone (zt,zh,zw) */
static double vat(const zs_ctx* c, int zt, int zh, int zw, int lt, int lh, int lw, int head, int e) {
  int64_t t = (int64_t)zt * ZONE + lt, h = (int64_t)zh * ZONE + lh, w = (int64_t)zw * ZONE + lw;
  int64_t n = (t * c->H + h) * c->W + w;
  return (double)c->v[(n * c->heads + head) * c->d + e];
}

static void zone_stats_task(void* vctx, int64_t task) {
  const zs_ctx* c = (const zs_ctx*)vctx;
  int ZH = c->H / ZONE, ZW = c->W / ZONE;
  int Z = (c->T / ZONE) * ZH * ZW;
  int grp = (int)(task / Z), m = (int)(task % Z);
  int zt = m / (ZH * ZW), zh = (m / ZW) % ZH, zw = m % ZW;
  int hpg = c->heads / c->groups;
  int D = hpg * c->d; /* channels of the head group (reading: D = the group's channels) */
  double var_ax[3] = {0, 0, 0}, var_tok = 0;
  double x[ZONE][ZONE][ZONE];
  for (int hl = 0; hl < hpg; ++hl) {
    int head = grp * hpg + hl;
    for (int e = 0; e < c->d; ++e) {
      double sum = 0;
      for (int i = 0; i < ZONE; ++i)
        for (int j = 0; j < ZONE; ++j)
          for (int k = 0; k < ZONE; ++k) {
            x[i][j][k] = vat(c, zt, zh, zw, i, j, k, head, e);
            sum += x[i][j][k];
          }
      double mu = sum / ZVOL; /* mu_{m,c}: the zone's channel mean (= mean of slice means) */
      /* slice-pooled profiles Vbar^{(d)}_{m,i,c}: mean over the other two axes */
      for (int ax = 0; ax < 3; ++ax) {
        double acc = 0;
        for (int i = 0; i < ZONE; ++i) {
          double s = 0;
          for (int j = 0; j < ZONE; ++j)
            for (int k = 0; k < ZONE; ++k)
              s += (ax == 0) ? x[i][j][k] : (ax == 1) ? x[j][i][k] : x[j][k][i];
          double vbar = s / (ZONE * ZONE);
          acc += (vbar - mu) * (vbar - mu);
        }
        var_ax[ax] += acc / ZONE; /* (1/Z_d) sum_i (Vbar_i - mu)^2 */
      }
      double acc = 0;
      for (int i = 0; i < ZONE; ++i)
        for (int j = 0; j < ZONE; ++j)
          for (int k = 0; k < ZONE; ++k) acc += (x[i][j][k] - mu) * (x[i][j][k] - mu);
      var_tok += acc / ZVOL;
    }
  }
  double* s2 = c->sig2 + ((int64_t)grp * Z + m) * 4;
  for (int ax = 0; ax < 3; ++ax) s2[ax] = var_ax[ax] / D; /* (1/D) sum_c ... */
  s2[3] = var_tok / D;
  double tot = s2[0] + s2[1] + s2[2];
  double* rr = c->r + ((int64_t)grp * Z + m) * 3;
  for (int ax = 0; ax < 3; ++ax) rr[ax] = (tot > 0) ? s2[ax] / tot : 1.0 / 3.0; /* r_{v,d} */
  /* density reading: axis-explained share of the zone's variance, 0 for a constant zone */
  c->rho[(int64_t)grp * Z + m] = (s2[3] > 0) ? tot / s2[3] : 0.0;
}

int orc_zone_stats(int T, int H, int W, int heads, int d, int groups, const float* v,
                   const float* a, double eps, double* sig2, double* r, double* rho,
                   double* abar, double* vhat, double* g, int nthreads) {
  if (T <= 0 || H <= 0 || W <= 0 || T % ZONE || H % ZONE || W % ZONE) return -1;
  if (heads <= 0 || d <= 0 || groups <= 0 || heads % groups) return -1;
  if (!v || !sig2 || !r || !rho || !abar || !vhat || !g) return -1;
  int ZT = T / ZONE, ZH = H / ZONE, ZW = W / ZONE, Z = ZT * ZH * ZW;
  zs_ctx c = {T, H, W, heads, d, groups, v, sig2, r, rho};
  parallel_for(nthreads, (int64_t)groups * Z, zone_stats_task, &c);

  /* audio coupling (RG M1: abar(m) in [0,1] and vhat_{a,d}(m) "are computed").
   * Reading: A(m) = zone mean of a; abar = A / max_m' A(m'); vhat = the same directional
   * variance as for V, applied to the scalar field a, normalised to sum 1 (1/3 each when
   * the field is flat).  Absent a: abar = vhat = 0. */
  double amax = 0;
  for (int m = 0; m < Z; ++m) {
    int zt = m / (ZH * ZW), zh = (m / ZW) % ZH, zw = m % ZW;
    if (!a) { abar[m] = 0; vhat[3 * m] = vhat[3 * m + 1] = vhat[3 * m + 2] = 0; continue; }
    double x[ZONE][ZONE][ZONE], sum = 0;
    for (int i = 0; i < ZONE; ++i)
      for (int j = 0; j < ZONE; ++j)
        for (int k = 0; k < ZONE; ++k) {
          int64_t t = (int64_t)zt * ZONE + i, h = (int64_t)zh * ZONE + j, w = (int64_t)zw * ZONE + k;
          x[i][j][k] = (double)a[(t * H + h) * W + w];
          sum += x[i][j][k];
        }
    double A = sum / ZVOL;
    double va[3];
    for (int ax = 0; ax < 3; ++ax) {
      double acc = 0;
      for (int i = 0; i < ZONE; ++i) {
        double s = 0;
        for (int j = 0; j < ZONE; ++j)
          for (int k = 0; k < ZONE; ++k)
            s += (ax == 0) ? x[i][j][k] : (ax == 1) ? x[j][i][k] : x[j][k][i];
        double sb = s / (ZONE * ZONE);
        acc += (sb - A) * (sb - A);
      }
      va[ax] = acc / ZONE;
    }
    double vs = va[0] + va[1] + va[2];
    for (int ax = 0; ax < 3; ++ax) vhat[3 * m + ax] = (vs > 0) ? va[ax] / vs : 1.0 / 3.0;
    abar[m] = A; /* normalised below */
    if (A > amax) amax = A;
  }
  for (int m = 0; m < Z; ++m) abar[m] = (a && amax > 0) ? abar[m] / amax : 0.0;

  /* composite indicator (RG M1): g_d = r_{v,d} + abar * vhat_{a,d} + eps */
  for (int grp = 0; grp < groups; ++grp)
    for (int m = 0; m < Z; ++m)
      for (int ax = 0; ax < 3; ++ax) {
        int64_t q = ((int64_t)grp * Z + m) * 3 + ax;
        g[q] = r[q] + abar[m] * vhat[3 * m + ax] + eps;
      }
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* RG M2: block volume and shape                                                          */

int orc_assign_shapes(int groups, int Z, const double* g, const double* rho, double tau128,
                      double tau256, int32_t* volume, double* lstar, double* dist,
                      uint8_t* shape_idx, int32_t* zone_block_off) {
  if (groups <= 0 || Z <= 0 || !g || !rho || !volume || !lstar || !dist || !shape_idx ||
      !zone_block_off)
    return -1;
  build_candidates();
  for (int grp = 0; grp < groups; ++grp) {
    int32_t off = 0;
    for (int m = 0; m < Z; ++m) {
      int64_t zi = (int64_t)grp * Z + m;
      /* volume: denser zone -> smaller blocks (reading of the two thresholds) */
      double rr = rho[zi];
      int B = (rr >= tau128) ? 64 : (rr >= tau256) ? 128 : 256;
      volume[zi] = B;
      /* log2-space optimum: l*_d = -1/2 log2 g_d + 1/3 (S + 1/2 sum_d' log2 g_d') */
      double S = log2((double)B);
      double L[3], Ls = 0;
      for (int ax = 0; ax < 3; ++ax) { L[ax] = log2(g[zi * 3 + ax]); Ls += L[ax]; }
      for (int ax = 0; ax < 3; ++ax) lstar[zi * 3 + ax] = -0.5 * L[ax] + (S + 0.5 * Ls) / 3.0;
      /* nearest candidate of volume B in Euclidean log2 distance; lowest index on ties */
      int best = -1;
      double bestd = INFINITY;
      for (int cidx = 0; cidx < g_cand_n; ++cidx) {
        if (g_cand_vol[cidx] != B) { dist[zi * 16 + cidx] = INFINITY; continue; }
        double dd = 0;
        for (int ax = 0; ax < 3; ++ax) {
          double diff = log2((double)g_cand_edges[cidx][ax]) - lstar[zi * 3 + ax];
          dd += diff * diff;
        }
        dist[zi * 16 + cidx] = dd;
        if (dd < bestd) { bestd = dd; best = cidx; }
      }
      shape_idx[zi] = (uint8_t)best;
      zone_block_off[(int64_t)grp * (Z + 1) + m] = off;
      off += ZVOL / B;
    }
    zone_block_off[(int64_t)grp * (Z + 1) + Z] = off;
  }
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* block order (reading: zones raster, blocks raster within a zone, tokens raster within a */
/* block); every block lies inside one zone because 512 is a multiple of every volume.    */

int orc_block_layout(int T, int H, int W, int groups, const uint8_t* shape_idx, int64_t* pos,
                     int32_t* block_start, int32_t* nblocks) {
  if (T % ZONE || H % ZONE || W % ZONE || groups <= 0 || !shape_idx || !pos || !block_start ||
      !nblocks)
    return -1;
  build_candidates();
  int ZH = H / ZONE, ZW = W / ZONE, Z = (T / ZONE) * ZH * ZW;
  int64_t N = (int64_t)T * H * W;
  for (int grp = 0; grp < groups; ++grp) {
    for (int t = 0; t < T; ++t)
      for (int h = 0; h < H; ++h)
        for (int w = 0; w < W; ++w) {
          int m = ((t / ZONE) * ZH + h / ZONE) * ZW + w / ZONE;
          int lt = t % ZONE, lh = h % ZONE, lw = w % ZONE;
          int s = shape_idx[(int64_t)grp * Z + m];
          if (s >= g_cand_n) return -2;
          int bT = g_cand_edges[s][0], bH = g_cand_edges[s][1], bW = g_cand_edges[s][2];
          int B = bT * bH * bW;
          int beta = ((lt / bT) * (ZONE / bH) + lh / bH) * (ZONE / bW) + lw / bW;
          int iota = ((lt % bT) * bH + lh % bH) * bW + lw % bW;
          int64_t n = ((int64_t)t * H + h) * W + w;
          pos[(int64_t)grp * N + n] = (int64_t)ZVOL * m + (int64_t)beta * B + iota;
        }
    int32_t* bs = block_start + (int64_t)grp * (8 * Z + 1);
    int32_t j = 0;
    for (int m = 0; m < Z; ++m) {
      int s = shape_idx[(int64_t)grp * Z + m];
      int B = g_cand_vol[s];
      for (int b = 0; b < ZVOL / B; ++b) bs[j++] = (int32_t)((int64_t)ZVOL * m + (int64_t)b * B);
    }
    nblocks[grp] = j;
    for (int q = j; q <= 8 * Z; ++q) bs[q] = (int32_t)N;
  }
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* RG M3: block mean-pooling                                                              */

typedef struct {
  int heads, groups, N, d, nbmax;
  const int32_t *block_start, *nblocks;
  const float* x;
  double* xbar;
} pool_ctx;

static void pool_task(void* vctx, int64_t task) {
  const pool_ctx* c = (const pool_ctx*)vctx;
  int head = (int)(task / c->nbmax), j = (int)(task % c->nbmax);
  int grp = head / (c->heads / c->groups);
  const int32_t* bs = c->block_start + (int64_t)grp * (c->nbmax + 1);
  double* out = c->xbar + ((int64_t)head * c->nbmax + j) * c->d;
  if (j >= c->nblocks[grp]) { for (int e = 0; e < c->d; ++e) out[e] = 0; return; }
  int64_t r0 = bs[j], r1 = bs[j + 1];
  for (int e = 0; e < c->d; ++e) {
    double s = 0;
    for (int64_t rr = r0; rr < r1; ++rr) s += (double)c->x[((int64_t)head * c->N + rr) * c->d + e];
    out[e] = s / (double)(r1 - r0);
  }
}

int orc_pool(int heads, int groups, int N, int d, int nbmax, const int32_t* block_start,
             const int32_t* nblocks, const float* xperm, double* xbar, int nthreads) {
  if (heads <= 0 || groups <= 0 || heads % groups || !block_start || !nblocks || !xperm || !xbar)
    return -1;
  pool_ctx c = {heads, groups, N, d, nbmax, block_start, nblocks, xperm, xbar};
  parallel_for(nthreads, (int64_t)heads * nbmax, pool_task, &c);
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* RG M3: hybrid Top-k / Top-p selection                                                  */

typedef struct { double p; double s; int32_t j; } pj_t;

static int cmp_desc(const void* A, const void* B) {
  const pj_t* a = (const pj_t*)A;
  const pj_t* b = (const pj_t*)B;
  if (a->p > b->p) return -1;
  if (a->p < b->p) return 1;
  return (a->j < b->j) ? -1 : (a->j > b->j) ? 1 : 0;
}

static int cmp_int(const void* A, const void* B) {
  int32_t a = *(const int32_t*)A, b = *(const int32_t*)B;
  return (a < b) ? -1 : (a > b) ? 1 : 0;
}

typedef struct {
  int heads, groups, d, nbmax;
  const int32_t* nblocks;
  const double *qbar, *kbar;
  double sm_scale, k_frac, p;
  int32_t k_abs;
  const uint8_t* row_mask;
  int32_t *sel_count, *sel_idx;
  double* info;
} sel_ctx;

static void select_task(void* vctx, int64_t task) {
  const sel_ctx* c = (const sel_ctx*)vctx;
  int head = (int)(task / c->nbmax), i = (int)(task % c->nbmax);
  int grp = head / (c->heads / c->groups);
  int nb = c->nblocks[grp];
  int64_t row = (int64_t)head * c->nbmax + i;
  double* inf = c->info + row * 5;
  if (i >= nb || (c->row_mask && !c->row_mask[row])) {
    if (i >= nb) c->sel_count[row] = 0;
    return;
  }
  pj_t* pj = (pj_t*)malloc(sizeof(pj_t) * (size_t)nb);
  int32_t* out = (int32_t*)malloc(sizeof(int32_t) * (size_t)nb);
  if (!pj || !out) { free(pj); free(out); c->sel_count[row] = -1; return; }
  /* block scores against the pooled representatives, then softmax over all key blocks */
  const double* qi = c->qbar + row * c->d;
  double mx = -INFINITY;
  for (int j = 0; j < nb; ++j) {
    const double* kj = c->kbar + ((int64_t)head * c->nbmax + j) * c->d;
    double s = 0;
    for (int e = 0; e < c->d; ++e) s += qi[e] * kj[e];
    pj[j].p = c->sm_scale * s;
    pj[j].s = pj[j].p;
    pj[j].j = j;
    if (pj[j].p > mx) mx = pj[j].p;
  }
  double den = 0;
  for (int j = 0; j < nb; ++j) { pj[j].p = exp(pj[j].p - mx); den += pj[j].p; }
  for (int j = 0; j < nb; ++j) pj[j].p /= den;
  /* order by probability, descending; ties by block index ascending */
  qsort(pj, (size_t)nb, sizeof(pj_t), cmp_desc);
  /* Top-p: smallest prefix whose cumulative probability reaches p (0 if p <= 0; all blocks
   * if rounding never reaches p) */
  int np = nb;
  double C = 0;
  if (c->p <= 0) np = 0;
  else
    for (int n = 1; n <= nb; ++n) {
      C += pj[n - 1].p;
      if (C >= c->p) { np = n; break; }
    }
  /* Top-k: k from an absolute count or a fraction of the key blocks (ceil), in [1, N_b] */
  int64_t kk = (c->k_abs > 0) ? c->k_abs : (int64_t)ceil(c->k_frac * (double)nb);
  if (kk < 1) kk = 1;
  if (kk > nb) kk = nb;
  /* union of two prefixes of one order = the longer prefix */
  int nsel = (np > kk) ? np : (int)kk;
  for (int n = 0; n < nsel; ++n) out[n] = pj[n].j;
  qsort(out, (size_t)nsel, sizeof(int32_t), cmp_int);
  c->sel_count[row] = nsel;
  int32_t* dst = c->sel_idx + row * c->nbmax;
  for (int n = 0; n < nsel; ++n) dst[n] = out[n];
  inf[0] = (double)kk;
  inf[1] = (double)np;
  inf[2] = (double)nsel;
  /* order margin at the cut: relative gap of the block scores on either side of it */
  inf[3] = (nsel < nb) ? (pj[nsel - 1].s - pj[nsel].s) / fmax(fabs(pj[nsel - 1].s), 1e-300) : INFINITY;
  if (c->p > 0 && np >= kk && np <= nb) {
    /* C_{n_p - 1} and C_{n_p} against p */
    double Cn = 0;
    for (int n = 0; n < np; ++n) Cn += pj[n].p;
    double Cm = Cn - pj[np - 1].p;
    double m1 = fabs(Cn - c->p) / c->p, m2 = fabs(Cm - c->p) / c->p;
    inf[4] = (m1 < m2) ? m1 : m2;
  } else {
    inf[4] = INFINITY;
  }
  free(pj);
  free(out);
}

int orc_select(int heads, int groups, int d, int nbmax, const int32_t* nblocks,
               const double* qbar, const double* kbar, double sm_scale, int32_t k_abs,
               double k_frac, double p, const uint8_t* row_mask, int32_t* sel_count,
               int32_t* sel_idx, double* info, int nthreads) {
  if (heads <= 0 || groups <= 0 || heads % groups || !nblocks || !qbar || !kbar || !sel_count ||
      !sel_idx || !info)
    return -1;
  sel_ctx c = {heads, groups, d, nbmax, nblocks, qbar, kbar, sm_scale, k_frac, p, k_abs,
               row_mask, sel_count, sel_idx, info};
  parallel_for(nthreads, (int64_t)heads * nbmax, select_task, &c);
  for (int64_t q = 0; q < (int64_t)heads * nbmax; ++q)
    if (sel_count[q] < 0) return -3;
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* RG M3: attention restricted to S_i (forward), exact softmax over the selected keys     */

typedef struct {
  int heads, groups, N, d, nbmax;
  const int32_t *block_start, *nblocks, *sel_count, *sel_idx;
  double sm_scale;
  const float *q, *k, *v, *dout;
  double *o, *lse, *delta; /* delta only in the backward */
  const uint8_t* row_need; /* [heads, nbmax] */
  double *dq, *dk, *dv;
  /* transposed selection for the key side of the backward */
  const int32_t *tr_off, *tr_list; /* per (head, key block): query blocks selecting it */
} at_ctx;

/* logits of one query row against every selected key, their LSE, and O (if o != NULL) */
static void row_forward(const at_ctx* c, int head, int i, int64_t row, double* o_row,
                        double* lse_out) {
  int grp = head / (c->heads / c->groups);
  const int32_t* bs = c->block_start + (int64_t)grp * (c->nbmax + 1);
  const int32_t* sel = c->sel_idx + ((int64_t)head * c->nbmax + i) * c->nbmax;
  int cnt = c->sel_count[(int64_t)head * c->nbmax + i];
  const float* qr = c->q + ((int64_t)head * c->N + row) * c->d;
  double mx = -INFINITY;
  for (int s = 0; s < cnt; ++s)
    for (int64_t kc = bs[sel[s]]; kc < bs[sel[s] + 1]; ++kc) {
      const float* kr = c->k + ((int64_t)head * c->N + kc) * c->d;
      double z = 0;
      for (int e = 0; e < c->d; ++e) z += (double)qr[e] * (double)kr[e];
      z *= c->sm_scale;
      if (z > mx) mx = z;
    }
  double den = 0;
  for (int s = 0; s < cnt; ++s)
    for (int64_t kc = bs[sel[s]]; kc < bs[sel[s] + 1]; ++kc) {
      const float* kr = c->k + ((int64_t)head * c->N + kc) * c->d;
      double z = 0;
      for (int e = 0; e < c->d; ++e) z += (double)qr[e] * (double)kr[e];
      den += exp(c->sm_scale * z - mx);
    }
  double lse = (cnt > 0) ? mx + log(den) : -INFINITY;
  *lse_out = lse;
  if (!o_row) return;
  for (int e = 0; e < c->d; ++e) o_row[e] = 0;
  for (int s = 0; s < cnt; ++s)
    for (int64_t kc = bs[sel[s]]; kc < bs[sel[s] + 1]; ++kc) {
      const float* kr = c->k + ((int64_t)head * c->N + kc) * c->d;
      const float* vr = c->v + ((int64_t)head * c->N + kc) * c->d;
      double z = 0;
      for (int e = 0; e < c->d; ++e) z += (double)qr[e] * (double)kr[e];
      double pr = exp(c->sm_scale * z - lse);
      for (int e = 0; e < c->d; ++e) o_row[e] += pr * (double)vr[e];
    }
}

static void fwd_task(void* vctx, int64_t task) {
  const at_ctx* c = (const at_ctx*)vctx;
  int head = (int)(task / c->nbmax), i = (int)(task % c->nbmax);
  int grp = head / (c->heads / c->groups);
  if (i >= c->nblocks[grp]) return;
  if (c->row_need && !c->row_need[task]) return;
  const int32_t* bs = c->block_start + (int64_t)grp * (c->nbmax + 1);
  for (int64_t row = bs[i]; row < bs[i + 1]; ++row)
    row_forward(c, head, i, row, c->o + ((int64_t)head * c->N + row) * c->d,
                c->lse + (int64_t)head * c->N + row);
}

int orc_attn_fwd(int heads, int groups, int N, int d, int nbmax, const int32_t* block_start,
                 const int32_t* nblocks, const int32_t* sel_count, const int32_t* sel_idx,
                 double sm_scale, const float* q, const float* k, const float* v,
                 const uint8_t* qblock_mask, double* o, double* lse, int nthreads) {
  if (heads <= 0 || groups <= 0 || heads % groups || !block_start || !nblocks || !sel_count ||
      !sel_idx || !q || !k || !v || !o || !lse)
    return -1;
  at_ctx c;
  memset(&c, 0, sizeof c);
  c.heads = heads; c.groups = groups; c.N = N; c.d = d; c.nbmax = nbmax;
  c.block_start = block_start; c.nblocks = nblocks; c.sel_count = sel_count; c.sel_idx = sel_idx;
  c.sm_scale = sm_scale; c.q = q; c.k = k; c.v = v; c.o = o; c.lse = lse;
  c.row_need = qblock_mask;
  parallel_for(nthreads, (int64_t)heads * nbmax, fwd_task, &c);
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* backward with the selection held constant:                                             */
/*   P = exp(z - LSE), delta_r = dO_r . O_r, dS = P (dO_r . v_c - delta_r),               */
/*   dQ_r = sm_scale sum_c dS k_c,  dK_c = sm_scale sum_r dS q_r,  dV_c = sum_r P dO_r    */

static void bwd_rowstat_task(void* vctx, int64_t task) {
  const at_ctx* c = (const at_ctx*)vctx;
  int head = (int)(task / c->nbmax), i = (int)(task % c->nbmax);
  int grp = head / (c->heads / c->groups);
  if (i >= c->nblocks[grp] || !c->row_need[task]) return;
  const int32_t* bs = c->block_start + (int64_t)grp * (c->nbmax + 1);
  double* orow = (double*)malloc(sizeof(double) * (size_t)c->d);
  if (!orow) return;
  for (int64_t row = bs[i]; row < bs[i + 1]; ++row) {
    int64_t ri = (int64_t)head * c->N + row;
    row_forward(c, head, i, row, orow, c->lse + ri);
    const float* dor = c->dout + ri * c->d;
    double dl = 0;
    for (int e = 0; e < c->d; ++e) dl += (double)dor[e] * orow[e];
    c->delta[ri] = dl;
  }
  free(orow);
}

static void bwd_dq_task(void* vctx, int64_t task) {
  const at_ctx* c = (const at_ctx*)vctx;
  int head = (int)(task / c->nbmax), i = (int)(task % c->nbmax);
  int grp = head / (c->heads / c->groups);
  if (i >= c->nblocks[grp] || !c->row_need[task]) return;
  const int32_t* bs = c->block_start + (int64_t)grp * (c->nbmax + 1);
  const int32_t* sel = c->sel_idx + ((int64_t)head * c->nbmax + i) * c->nbmax;
  int cnt = c->sel_count[(int64_t)head * c->nbmax + i];
  for (int64_t row = bs[i]; row < bs[i + 1]; ++row) {
    int64_t ri = (int64_t)head * c->N + row;
    const float* qr = c->q + ri * c->d;
    const float* dor = c->dout + ri * c->d;
    double* dqr = c->dq + ri * c->d;
    for (int e = 0; e < c->d; ++e) dqr[e] = 0;
    for (int s = 0; s < cnt; ++s)
      for (int64_t kc = bs[sel[s]]; kc < bs[sel[s] + 1]; ++kc) {
        const float* kr = c->k + ((int64_t)head * c->N + kc) * c->d;
        const float* vr = c->v + ((int64_t)head * c->N + kc) * c->d;
        double z = 0, dp = 0;
        for (int e = 0; e < c->d; ++e) {
          z += (double)qr[e] * (double)kr[e];
          dp += (double)dor[e] * (double)vr[e];
        }
        double pr = exp(c->sm_scale * z - c->lse[ri]);
        double ds = pr * (dp - c->delta[ri]);
        for (int e = 0; e < c->d; ++e) dqr[e] += c->sm_scale * ds * (double)kr[e];
      }
  }
}

static void bwd_dkdv_task(void* vctx, int64_t task) {
  const at_ctx* c = (const at_ctx*)vctx;
  int head = (int)(task / c->nbmax), j = (int)(task % c->nbmax);
  int grp = head / (c->heads / c->groups);
  if (j >= c->nblocks[grp] || !c->row_need[task]) return;
  const int32_t* bs = c->block_start + (int64_t)grp * (c->nbmax + 1);
  int64_t t0 = c->tr_off[task], t1 = c->tr_off[task + 1];
  for (int64_t kc = bs[j]; kc < bs[j + 1]; ++kc) {
    int64_t ki = (int64_t)head * c->N + kc;
    const float* kr = c->k + ki * c->d;
    const float* vr = c->v + ki * c->d;
    double* dkr = c->dk + ki * c->d;
    double* dvr = c->dv + ki * c->d;
    for (int e = 0; e < c->d; ++e) dkr[e] = dvr[e] = 0;
    for (int64_t t = t0; t < t1; ++t) {
      int i = c->tr_list[t];
      for (int64_t row = bs[i]; row < bs[i + 1]; ++row) {
        int64_t ri = (int64_t)head * c->N + row;
        const float* qr = c->q + ri * c->d;
        const float* dor = c->dout + ri * c->d;
        double z = 0, dp = 0;
        for (int e = 0; e < c->d; ++e) {
          z += (double)qr[e] * (double)kr[e];
          dp += (double)dor[e] * (double)vr[e];
        }
        double pr = exp(c->sm_scale * z - c->lse[ri]);
        double ds = pr * (dp - c->delta[ri]);
        for (int e = 0; e < c->d; ++e) {
          dvr[e] += pr * (double)dor[e];
          dkr[e] += c->sm_scale * ds * (double)qr[e];
        }
      }
    }
  }
}

/* wall seconds of the last orc_attn_bwd's three passes (measurement only) */
static double g_bwd_phase_s[3];

static double now_s(void) {
  struct timespec ts;
  clock_gettime(CLOCK_MONOTONIC, &ts);
  return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

void orc_last_bwd_phase_seconds(double* out) {
  for (int i = 0; i < 3; ++i) out[i] = g_bwd_phase_s[i];
}

int orc_attn_bwd(int heads, int groups, int N, int d, int nbmax, const int32_t* block_start,
                 const int32_t* nblocks, const int32_t* sel_count, const int32_t* sel_idx,
                 double sm_scale, const float* q, const float* k, const float* v,
                 const float* dout, const uint8_t* qblock_mask, const uint8_t* kblock_mask,
                 double* dq, double* dk, double* dv, double* lse, double* delta, int nthreads) {
  if (heads <= 0 || groups <= 0 || heads % groups || !block_start || !nblocks || !sel_count ||
      !sel_idx || !q || !k || !v || !dout || !dq || !dk || !dv || !lse || !delta)
    return -1;
  int64_t rows = (int64_t)heads * nbmax;
  /* transposed selection: for each (head, key block) the query blocks that selected it */
  int32_t* tr_off = (int32_t*)calloc((size_t)rows + 1, sizeof(int32_t));
  uint8_t* need = (uint8_t*)calloc((size_t)rows, 1);
  uint8_t* dqneed = (uint8_t*)calloc((size_t)rows, 1);
  if (!tr_off || !need || !dqneed) { free(tr_off); free(need); free(dqneed); return -3; }
  int64_t total = 0;
  for (int head = 0; head < heads; ++head) {
    int grp = head / (heads / groups);
    for (int i = 0; i < nblocks[grp]; ++i) {
      int64_t ri = (int64_t)head * nbmax + i;
      for (int s = 0; s < sel_count[ri]; ++s) tr_off[(int64_t)head * nbmax + sel_idx[ri * nbmax + s] + 1]++;
      total += sel_count[ri];
    }
  }
  for (int64_t q2 = 0; q2 < rows; ++q2) tr_off[q2 + 1] += tr_off[q2];
  int32_t* tr_list = (int32_t*)malloc(sizeof(int32_t) * (size_t)(total > 0 ? total : 1));
  int32_t* fill = (int32_t*)calloc((size_t)rows, sizeof(int32_t));
  if (!tr_list || !fill) { free(tr_off); free(need); free(dqneed); free(tr_list); free(fill); return -3; }
  for (int head = 0; head < heads; ++head) {
    int grp = head / (heads / groups);
    for (int i = 0; i < nblocks[grp]; ++i) {
      int64_t ri = (int64_t)head * nbmax + i;
      for (int s = 0; s < sel_count[ri]; ++s) {
        int64_t kb = (int64_t)head * nbmax + sel_idx[ri * nbmax + s];
        tr_list[tr_off[kb] + fill[kb]++] = i; /* ascending in i */
      }
    }
  }
  /* rows whose statistics are needed: dq rows, plus every query block that selected a key
   * block whose gradient is requested */
  for (int64_t q2 = 0; q2 < rows; ++q2) {
    if (!qblock_mask || qblock_mask[q2]) { need[q2] = 1; dqneed[q2] = 1; }
  }
  for (int64_t kb = 0; kb < rows; ++kb) {
    if (kblock_mask && !kblock_mask[kb]) continue;
    int head = (int)(kb / nbmax);
    for (int32_t t = tr_off[kb]; t < tr_off[kb + 1]; ++t) need[(int64_t)head * nbmax + tr_list[t]] = 1;
  }
  at_ctx c;
  memset(&c, 0, sizeof c);
  c.heads = heads; c.groups = groups; c.N = N; c.d = d; c.nbmax = nbmax;
  c.block_start = block_start; c.nblocks = nblocks; c.sel_count = sel_count; c.sel_idx = sel_idx;
  c.sm_scale = sm_scale; c.q = q; c.k = k; c.v = v; c.dout = dout;
  c.lse = lse; c.delta = delta; c.dq = dq; c.dk = dk; c.dv = dv;
  c.tr_off = tr_off; c.tr_list = tr_list;
  c.row_need = need;
  double t0 = now_s();
  parallel_for(nthreads, rows, bwd_rowstat_task, &c);
  double t1 = now_s();
  /* dQ for the requested query blocks */
  c.row_need = dqneed;
  parallel_for(nthreads, rows, bwd_dq_task, &c);
  double t2 = now_s();
  /* dK, dV for the requested key blocks */
  uint8_t* kmask = (uint8_t*)malloc((size_t)rows);
  if (!kmask) { free(tr_off); free(need); free(dqneed); free(tr_list); free(fill); return -3; }
  for (int64_t kb = 0; kb < rows; ++kb) kmask[kb] = (!kblock_mask || kblock_mask[kb]) ? 1 : 0;
  c.row_need = kmask;
  parallel_for(nthreads, rows, bwd_dkdv_task, &c);
  double t3 = now_s();
  g_bwd_phase_s[0] = t1 - t0;
  g_bwd_phase_s[1] = t2 - t1;
  g_bwd_phase_s[2] = t3 - t2;
  free(kmask);
  free(tr_off); free(need); free(dqneed); free(tr_list); free(fill);
  return 0;
}

/* RG M1 (audio coupling input): a_n = || hhat_n ||_2 over the channels of token n, the
 * cross-attention output norm the zone statistics consume; sum of squares when squared != 0. */
int orc_audio_norms(int64_t N, int channels, const float* hhat, int squared, double* a) {
  if (N < 0 || channels <= 0 || !hhat || !a) return -1;
  for (int64_t n = 0; n < N; ++n) {
    double s = 0.0;
    for (int c = 0; c < channels; ++c) {
      const double x = (double)hhat[n * channels + c];
      s += x * x;
    }
    a[n] = squared ? s : sqrt(s);
  }
  return 0;
}
