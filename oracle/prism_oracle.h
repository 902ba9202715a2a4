/* prism_oracle.h -- plain CPU reference ("oracle") of the Prism dynamic block-sparse
 * video self-attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load or call this library.  The product path (the HIP library
 * and its Python binding) never links it, and it includes nothing from the product.
 *
 * Sources.  "RG" is the reading-guide page of "Prism: Dynamic Sparse Attention for
 * Native 2K Joint Video-Audio Generation Model Training" (arXiv 2610.05416); its
 * "Method" section has three numbered parts:
 *   RG M1  "Variation Indicator Formulation": the directional variance / variation-ratio
 *          equation (sigma^2_{v,d}, r_{v,d}) and the composite-indicator equation g_d(m);
 *   RG M2  "Block Volume and Shape Quantization": volume thresholds, the continuous
 *          optimum b*_d ~ g_d^{-1/2}, the log2-space optimum equation l*_d and the
 *          nearest-candidate rule;
 *   RG M3  "Hybrid Top-k / Top-p Attention": pooled key blocks, block probabilities,
 *          the attended-set equation S_i = Top-k(P_i,k) U Top-p(P_i,p), and the
 *          online-softmax sparse attention over S_i.
 * "RG KI" is that page's "Key ideas" list (8x8x8 macro-zones; 16-shape candidate set).
 * "README" is the Prism project page (its "Core training parameters" table names the
 * bsa_sparsity / bsa_cdf_threshold / enable_ivpq_dynamic_block knobs).
 *
 * Where the pages are silent the oracle follows a stated reading; each function below
 * names the readings it uses.  Floating point is fp64 throughout; inputs are fp32 arrays
 * that hold exactly the values the GPU path receives (bf16 inputs widened exactly).
 *
 * Layouts.  Token order: n = (t*H + h)*W + w, tensors [N, heads, d].  Block order
 * ("permuted"): tensors [heads, N, d].  Zones m = (zt*(H/8) + zh)*(W/8) + zw.
 * G head groups; head h belongs to group h / (heads/G).  NBMAX = 8*Z.
 *
 * Every function returns 0 on success and a negative value on a bad argument.
 */
#ifndef PRISM_ORACLE_H
#define PRISM_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The 16-shape candidate set (RG KI, RG M2), enumerated by the oracle itself:
 * edges in {2,4,8}, volume in {64,128,256}; order = volume ascending, then (bT,bH,bW)
 * lexicographic.  Writes [16][3] edges and [16] volumes; returns the count (16). */
int orc_candidates(int32_t* edges, int32_t* volume);

/* RG M1.  Per head group and zone: directional variance of slice-pooled V (sig2[...,0:3]),
 * token variance (sig2[...,3]), variation ratios r, density rho, audio coupling abar,
 * audio directional shares vhat, and g = r + abar*vhat + eps.
 * a may be NULL (first layer): then abar = vhat = 0.
 * Outputs: sig2 [G,Z,4], r [G,Z,3], rho [G,Z], abar [Z], vhat [Z,3], g [G,Z,3]. */
int orc_zone_stats(int T, int H, int W, int heads, int d, int groups,
                   const float* v, const float* a, double eps,
                   double* sig2, double* r, double* rho, double* abar, double* vhat,
                   double* g, int nthreads);

/* RG M2.  Volume from rho, l* from g (log2-space optimum), nearest candidate of that
 * volume (Euclidean distance in log2 space, lowest index on exact ties).
 * Outputs: volume [G,Z], lstar [G,Z,3], dist [G,Z,16] (squared log2 distance; +inf for
 * candidates of another volume), shape_idx [G,Z], zone_block_off [G,Z+1]. */
int orc_assign_shapes(int groups, int Z, const double* g, const double* rho,
                      double tau128, double tau256,
                      int32_t* volume, double* lstar, double* dist,
                      uint8_t* shape_idx, int32_t* zone_block_off);

/* Block order (reading: zones raster, blocks raster inside a zone, tokens raster inside a
 * block).  pos [G,N]: permuted row of token n.  block_start [G, 8Z+1]: first permuted row
 * of block j (entries past the group's block count hold N).  nblocks [G]. */
int orc_block_layout(int T, int H, int W, int groups, const uint8_t* shape_idx,
                     int64_t* pos, int32_t* block_start, int32_t* nblocks);

/* RG M3 (pooled representatives).  xbar[h][j] = mean of block j's rows of xperm[h];
 * rows j >= nblocks are zero.  xperm [heads,N,d] -> xbar [heads,NBMAX,d]. */
int orc_pool(int heads, int groups, int N, int d, int nbmax,
             const int32_t* block_start, const int32_t* nblocks,
             const float* xperm, double* xbar, int nthreads);

/* RG M3 (attended-set equation).  Scores s_ij = sm_scale * qbar_i . kbar_j, P_i = softmax
 * over the group's blocks, order by P descending (index ascending on ties), n_p = smallest
 * prefix with cumulative P >= p, k = clamp(k_abs>0 ? k_abs : ceil(k_frac*N_b), 1, N_b),
 * S_i = first max(k, n_p) blocks of that order, stored ascending.
 * row_mask [heads,NBMAX] (NULL = all rows) restricts the work.
 * Outputs: sel_count [heads,NBMAX], sel_idx [heads,NBMAX,NBMAX] (row stride NBMAX),
 * info [heads,NBMAX,5] = {k, n_p, n_sel, order margin, cdf margin} (margins: relative gap
 * of the block scores (s_(n) - s_(n+1)) / |s_(n)| at the cut n = n_sel, and
 * min |C_n - p|/p over n in {n_p-1, n_p} when n_p >= k;
 * +inf where not applicable). */
int orc_select(int heads, int groups, int d, int nbmax, const int32_t* nblocks,
               const double* qbar, const double* kbar, double sm_scale,
               int32_t k_abs, double k_frac, double p, const uint8_t* row_mask,
               int32_t* sel_count, int32_t* sel_idx, double* info, int nthreads);

/* RG M3 (attention over S_i).  For each query row of the query blocks marked in
 * qblock_mask [heads,NBMAX] (NULL = all): softmax over every key of the selected blocks of
 * sm_scale*q.k, O = sum p v, LSE natural log.  q,k,v [heads,N,d] in block order.
 * Outputs o [heads,N,d], lse [heads,N] (only the computed rows are written). */
int orc_attn_fwd(int heads, int groups, int N, int d, int nbmax,
                 const int32_t* block_start, const int32_t* nblocks,
                 const int32_t* sel_count, const int32_t* sel_idx, double sm_scale,
                 const float* q, const float* k, const float* v,
                 const uint8_t* qblock_mask, double* o, double* lse, int nthreads);

/* Gradient of orc_attn_fwd with the selection held constant (reading: no gradient flows to
 * statistics, shapes, pooling or selection).  dq for rows of qblock_mask, dk/dv for keys
 * of kblock_mask (NULL = all).  Also returns lse and delta = dO.O (exact O) for every row
 * it needed.  All arrays [heads,N,d] / [heads,N], block order. */
int orc_attn_bwd(int heads, int groups, int N, int d, int nbmax,
                 const int32_t* block_start, const int32_t* nblocks,
                 const int32_t* sel_count, const int32_t* sel_idx, double sm_scale,
                 const float* q, const float* k, const float* v, const float* dout,
                 const uint8_t* qblock_mask, const uint8_t* kblock_mask,
                 double* dq, double* dk, double* dv, double* lse, double* delta,
                 int nthreads);

/* Wall-clock seconds of the last orc_attn_bwd call's three passes (row statistics, dQ,
 * dK/dV), written to out[3]: a measurement aid for the CPU baseline, not part of any result. */
void orc_last_bwd_phase_seconds(double* out);

/* RG M1 (the audio coupling field is the L2 norm of each video token's audio-to-video
 * cross-attention output, taken from the previous layer).  hhat [N, channels] fp32 (token
 * order) -> a [N] = sqrt(sum_c hhat[n][c]^2), or the sum of squares itself when squared != 0. */
int orc_audio_norms(int64_t N, int channels, const float* hhat, int squared, double* a);

#ifdef __cplusplus
}
#endif
#endif
