/* prism.h -- C ABI of the MI355X (gfx950) Prism hot path: content-adaptive dynamic
 * block-sparse video self-attention, forward and backward, for one layer and head group.
 *
 * Sources.  "RG" is the reading-guide page of "Prism: Dynamic Sparse Attention for Native
 * 2K Joint Video-Audio Generation Model Training" (arXiv 2610.05416).  RG M1, M2, M3 are its
 * Method parts 1 ("Variation Indicator Formulation"), 2 ("Block Volume and Shape
 * Quantization") and 3 ("Hybrid Top-k / Top-p Attention"); RG KI is its "Key ideas" list.
 * "README" is the Prism project page (table "Core training parameters").
 *
 * Conventions shared by every call
 * - All tensor pointers are DEVICE pointers owned by the caller; the library allocates
 *   nothing and keeps no state other than a per-thread error message.  Host arrays are
 *   named as such.  `stream` is a hipStream_t passed as void* (NULL = default stream).
 * - Every call validates its arguments on the host first and returns an error code without
 *   launching anything if they are bad.  On success it enqueues work on `stream` and returns;
 *   results are valid once the stream reaches that point.  No exception crosses the ABI.
 * - Tensors are contiguous; tensor pointers must be 16-byte aligned.
 * - Token grid T x H x W, each a positive multiple of 8 (macro-zones of 8x8x8 tokens, RG KI),
 *   N = T*H*W tokens, Z = N/512 zones, NBMAX = 8*Z (the most blocks a group can have).
 *   Token order n = (t*H + h)*W + w; token-order tensors are [N, heads, head_dim].
 *   Zone order m = (zt*(H/8) + zh)*(W/8) + zw.
 * - Block order: zones in zone order, the blocks of a zone in raster order over the zone's
 *   block grid, the tokens of a block in raster order.  Block-order tensors are
 *   [heads, N, head_dim]; block j of group g covers rows [block_start[g][j], block_start[g][j+1]).
 * - heads are split into `groups` head groups of heads/groups consecutive heads; each group
 *   has its own zone statistics, shapes and block layout; selection and attention are per head.
 * - dtype PRISM_BF16: bf16 tensors, fp32 accumulation.  PRISM_F32: fp32 tensors throughout.
 * - Limits: head_dim in {64, 128}; Z <= 2048 (N <= 1,048,576 tokens: a query block's scores,
 *   up to NBMAX = 16,384, are held by one selection workgroup, 64 per thread); every tensor
 *   below 2^31 elements.
 */
#ifndef PRISM_H
#define PRISM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PRISM_ABI_VERSION 3

typedef enum {
  PRISM_OK = 0,
  PRISM_E_NULL = 1,      /* a required pointer is NULL */
  PRISM_E_SHAPE = 2,     /* grid / heads / head_dim / groups not supported */
  PRISM_E_RANGE = 3,     /* a scalar argument is out of range */
  PRISM_E_DTYPE = 4,     /* unknown dtype */
  PRISM_E_ALIGN = 5,     /* a tensor pointer is not 16-byte aligned */
  PRISM_E_WORKSPACE = 6, /* workspace too small */
  PRISM_E_HIP = 7        /* a HIP runtime call failed (detail in prism_last_error) */
} prism_status;

typedef enum { PRISM_F32 = 0, PRISM_BF16 = 1 } prism_dtype;

typedef struct {
  int32_t T, H, W;   /* token grid, each a positive multiple of 8 */
  int32_t heads;     /* attention heads in this call */
  int32_t head_dim;  /* 64 or 128 */
  int32_t groups;    /* head groups (heads % groups == 0) */
  int32_t dtype;     /* prism_dtype of Q, K, V, O and their gradients */
} prism_problem;

/* ---- information ------------------------------------------------------------------- */

int32_t prism_abi_version(void);
const char* prism_status_string(prism_status s);
/* Detail of the last failing call on this thread ("" if none).  Owned by the library. */
const char* prism_last_error(void);
/* The 16-shape candidate set (RG KI; volumes {64,128,256}, RG M2), in the library's index
 * order: volume ascending, then (b_T, b_H, b_W) lexicographic, edges in {2,4,8}.
 * Writes 48 int32 into the HOST array edges ([16][3]); returns 16. */
int32_t prism_shape_table(int32_t* edges);

/* ---- a1 input: the audio coupling field (RG M1) ------------------------------------- *
 * The statistics read, per video token, the L2 norm of that token's audio-to-video
 * cross-attention output, cached from the preceding layer: a[n] = sqrt(sum_c hhat[n][c]^2)
 * with fp32 accumulation (squared = 1: the sum of squares itself, for a caller whose hhat is
 * split over channels across devices and adds the partial sums before the root).
 * hhat: [N, channels] dtype, token order; channels a positive multiple of 8 (at most 2^20).
 * a:    out [N] fp32, the `a` argument of prism_zone_stats. */
prism_status prism_audio_norms(const prism_problem* pb, const void* hhat, int32_t channels,
                               int32_t squared, float* a, void* stream);

/* ---- a1: zone statistics (RG M1) ---------------------------------------------------- *
 * For each head group g and zone m, over the group's D = (heads/groups)*head_dim channels:
 *   sigma^2_{v,d}(m) = (1/D) sum_c (1/8) sum_i (Vbar^{(d)}_{m,i,c} - mu_{m,c})^2, where
 *   Vbar^{(d)}_{m,i,c} is the mean of channel c over the 64 tokens of slice i along axis d and
 *   mu_{m,c} the zone mean (the variation-ratio equation of RG M1);
 *   r_{v,d} = sigma^2_{v,d} / sum_d' sigma^2_{v,d'} (1/3 each if the sum is 0);
 *   rho(m) = sum_d sigma^2_{v,d} / sigma^2_tok, sigma^2_tok = (1/D) sum_c (1/512) sum_x
 *     (V_{x,c} - mu_c)^2 (0 if sigma^2_tok = 0) -- the reading of RG M2's "normalized
 *     spatiotemporal information density";
 *   audio (reading of RG M1's abar and vhat): A(m) = zone mean of a, abar = A / max_m' A(m'),
 *   vhat_d = the same directional variance applied to the field a, normalised to sum 1
 *   (1/3 each if flat); abar = vhat = 0 when a is NULL (no cached norms yet);
 *   g_d(m) = r_{v,d} + abar * vhat_d + eps (composite-indicator equation of RG M1).
 * v:          [N, heads, head_dim] dtype, token order (the layer's values).
 * a:          [N] fp32 audio-to-video cross-attention output norms from the preceding layer,
 *             or NULL.
 * eps:        > 0.
 * g:          out [groups, Z, 3] fp32 (axes T, H, W).
 * rho:        out [groups, Z] fp32.
 * zone_audio: out [Z, 4] fp32 = (abar, vhat_T, vhat_H, vhat_W); required when a != NULL,
 *             ignored (may be NULL) when a == NULL. */
prism_status prism_zone_stats(const prism_problem* pb, const void* v, const float* a, float eps,
                              float* g, float* rho, float* zone_audio, void* stream);

/* ---- a2: block volume and shape (RG M2) --------------------------------------------- *
 * B(m) = 64 if rho >= tau128, 128 if tau256 <= rho < tau128, else 256 (RG M2 thresholds;
 * denser zones get smaller blocks).  l*_d = -1/2 log2 g_d + 1/3 (log2 B + 1/2 sum log2 g)
 * (RG M2 log2-space optimum); the shape is the candidate of volume B nearest to l* in
 * Euclidean log2 distance (lowest index on exact ties).  Decisions are taken in fp32.
 * tau128, tau256: 0 <= tau256 <= tau128.
 * shape_idx:      out [groups, Z] uint8, index into prism_shape_table.
 * zone_block_off: out [groups, Z+1] int32, exclusive scan of 512/B(m); [g][Z] = N_b(g).
 * block_start:    out [groups, NBMAX+1] int32, first block-order row of block j; entries
 *                 j >= N_b(g) hold N. */
prism_status prism_assign_shapes(const prism_problem* pb, const float* g, const float* rho,
                                 float tau128, float tau256, uint8_t* shape_idx,
                                 int32_t* zone_block_off, int32_t* block_start, void* stream);

/* ---- a2 alternative: one fixed shape for every zone ---------------------------------- *
 * The pages' ablation with dynamic block shapes switched off (README "Core training
 * parameters": enable_ivpq_dynamic_block = false uses fixed 4x4x4 blocks; RG "Key ideas"
 * contrasts it with the adaptive shapes): every zone of every group gets candidate
 * shape_index (0..15, an index into prism_shape_table; 3 is 4x4x4), so a1 and a2 are skipped.
 * Outputs as for prism_assign_shapes.  Errors: PRISM_E_RANGE for an index outside 0..15. */
prism_status prism_fixed_shapes(const prism_problem* pb, int32_t shape_index, uint8_t* shape_idx,
                                int32_t* zone_block_off, int32_t* block_start, void* stream);

/* ---- a3: token order <-> block order ------------------------------------------------ *
 * Moves rows between token order [N, heads, head_dim] and block order [heads, N, head_dim]
 * using each group's shape map (the block order described above; the pages ask that each
 * block's tokens be kept together, RG M3 / abstract).  inverse = 0: token -> block order;
 * inverse = 1: block -> token order.  count (1..4) tensors per call: src and dst are HOST
 * arrays of `count` device pointers, dtype per pb.  src and dst must not overlap. */
prism_status prism_permute(const prism_problem* pb, const uint8_t* shape_idx, int32_t inverse,
                           int32_t count, const void* const* src, void* const* dst, void* stream);

/* ---- a4: pooled block representatives (RG M3) --------------------------------------- *
 * xbar[h][j][:] = mean of rows [block_start[j], block_start[j+1]) of x_perm[h] (fp32
 * accumulation), zero for j >= N_b.  count (1..4) tensors: x_perm is a HOST array of device
 * pointers to [heads, N, head_dim] dtype tensors, xbar a HOST array of device pointers to
 * [heads, NBMAX, head_dim] fp32 outputs. */
prism_status prism_pool_blocks(const prism_problem* pb, const int32_t* block_start, int32_t count,
                               const void* const* x_perm, float* const* xbar, void* stream);

/* ---- a3 + a4 in one pass ------------------------------------------------------------ *
 * Token -> block order for count (1..4) tensors, as prism_permute(inverse = 0), and for every
 * tensor i with xbar[i] != NULL also its pooled block means, as prism_pool_blocks on dst[i]
 * (bitwise the same values, rows j >= N_b zero), without reading the permuted tensor again.
 * src, dst, xbar: HOST arrays of count device pointers; xbar itself may be NULL (no pooling).
 * zone_block_off: [groups, Z+1] from prism_assign_shapes / prism_fixed_shapes for the same
 * shape_idx. */
prism_status prism_permute_pool(const prism_problem* pb, const uint8_t* shape_idx,
                                const int32_t* zone_block_off, int32_t count,
                                const void* const* src, void* const* dst, float* const* xbar,
                                void* stream);

/* ---- a5: hybrid Top-k / Top-p block selection (RG M3 attended-set equation) ---------- *
 * Per head h and query block i < N_b: s_ij = sm_scale * qbar_i . kbar_j (fp32), P_i = softmax
 * over the N_b key blocks, order by P descending (block index ascending on ties),
 * n_p = smallest n with cumulative P >= p (0 if p == 0; N_b if never reached),
 * k = clamp(k_abs > 0 ? k_abs : ceil(k_frac * N_b), 1, N_b) evaluated in double
 * (README: bsa_sparsity s keeps a fraction 1 - s), S_i = the first max(k, n_p) blocks of
 * that order (the union of the two prefixes), written in ascending block order.
 * qbar, kbar: [heads, NBMAX, head_dim] fp32 from prism_pool_blocks.
 * sel_count:  out [heads, NBMAX] int32 (0 for i >= N_b).
 * sel_idx:    out [heads, NBMAX, NBMAX] int32, row (h, i) holds S_i in its first
 *             sel_count entries.  The whole array is also used as fp32 score scratch during
 *             the call; entries past sel_count are unspecified afterwards.
 * k_abs >= 0, 0 <= k_frac <= 1, 0 <= p <= 1, sm_scale finite and > 0. */
prism_status prism_select_blocks(const prism_problem* pb, const int32_t* block_start,
                                 const float* qbar, const float* kbar, float sm_scale,
                                 int32_t k_abs, double k_frac, double p, int32_t* sel_count,
                                 int32_t* sel_idx, void* stream);

/* ---- a6: block-sparse attention forward (RG M3: online-softmax attention solely across S_i)
 * For head h and each row r of query block i (block order): exact softmax over every key
 * row of the blocks in S_i of sm_scale * q_r . k_c, O_r = sum p v_c, LSE_r natural log
 * (-inf and O = 0 for an empty list).  No causal mask, dropout or bias.
 * q, k, v, o: [heads, N, head_dim] dtype, block order.  lse: out [heads, N] fp32.
 * o_lo: optional out [heads, N, head_dim] dtype (bf16 problems only; NULL to skip): the
 *       rounding residual of O, o_lo = rnd(O_fp32 - o), so that o + o_lo carries about 16
 *       significant bits.  prism_bsa_bwd uses it to form delta = dO . O without the bf16
 *       rounding of o, which otherwise dominates the gradient error when the softmax is
 *       peaked (dP - delta cancels).
 * workspace: NULL, or device scratch of at least prism_bsa_fwd_workspace_bytes(pb) bytes,
 *       256-byte aligned, contents on entry irrelevant (workspace_bytes is ignored when NULL).
 *       With it, the workgroups whose query blocks have the longest lists are launched
 *       first (the order is built on the device; see prism_set_launch_order), which shortens
 *       the end of the launch; the results are the same with or without it.  After a bf16
 *       call its first heads*N/128 int32 hold that order (items head*N/128 + pair), followed,
 *       256-byte aligned, by the per-pair work estimates it was built from. */
size_t prism_bsa_fwd_workspace_bytes(const prism_problem* pb);
prism_status prism_bsa_fwd(const prism_problem* pb, const int32_t* block_start,
                           const int32_t* sel_count, const int32_t* sel_idx, float sm_scale,
                           const void* q, const void* k, const void* v, void* o, void* o_lo,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ---- a7: block-sparse attention backward -------------------------------------------- *
 * Gradient of prism_bsa_fwd with the selection held constant: delta_r = dO_r . O_r,
 * P = exp(sm_scale q.k - LSE), dV = P^T dO, dS = P (dO v^T - delta), dQ = sm_scale dS K,
 * dK = sm_scale dS^T Q.  o, o_lo and lse are prism_bsa_fwd's outputs for the same inputs
 * (o_lo may be NULL; then delta uses o alone).
 * dout: [heads, N, head_dim] dtype, block order.
 * dq, dk, dv: out [heads, N, head_dim] fp32 for every dtype (gradients leave the fp32
 *       accumulators unrounded), block order, fully overwritten.  For bf16 problems the
 *       matrix-core products with P and dS split each factor into a bf16 head and a bf16
 *       residual, so the gradients keep fp32-level accuracy.
 * workspace: device scratch of at least prism_bsa_bwd_workspace_bytes(pb) bytes, 256-byte
 * aligned; its contents on entry do not matter.  After a bf16 call it holds (each part starting
 * 256-byte aligned, A(x) = x rounded up to a multiple of 256): delta [heads, N] fp32 at 0;
 * lse2 = LSE * log2(e) at A(4*heads*N); the transposed selection bitmap [heads, NBMAX,
 * ceil(NBMAX/32)] uint32 at 2*A(4*heads*N); then the launch orders of the dQ and dK/dV
 * kernels [2][heads*N/64] int32 and the per-atom work estimates they were built from
 * [2][heads*N/64] int32 (readable for inspection; see prism_set_launch_order). */
size_t prism_bsa_bwd_workspace_bytes(const prism_problem* pb);
prism_status prism_bsa_bwd(const prism_problem* pb, const int32_t* block_start,
                           const int32_t* sel_count, const int32_t* sel_idx, float sm_scale,
                           const void* q, const void* k, const void* v, const void* o,
                           const void* o_lo, const void* dout, const float* lse, float* dq,
                           float* dk, float* dv, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ---- a7 without allocation ---------------------------------------------------------- *
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): prism_bsa_bwd with the same arguments and results,
 * minus the workspace, which is a fixed device array inside the library instead, of
 * prism_bsa_bwd_noalloc_max_bytes() bytes (64 MiB; each device the library runs on holds one
 * copy until the process ends).  Problems whose prism_bsa_bwd_workspace_bytes exceed it are
 * refused with PRISM_E_WORKSPACE before anything is launched (the 2K-shaped problem, 4 heads,
 * needs about 46 MB).  The call allocates nothing.  Every call on one device shares that
 * device's array, whose contents on entry do not matter: calls that overlap on one device
 * (different streams, threads) race on it and must be serialised by the caller. */
size_t prism_bsa_bwd_noalloc_max_bytes(void);
prism_status prism_bsa_bwd_noalloc(const prism_problem* pb, const int32_t* block_start,
                                   const int32_t* sel_count, const int32_t* sel_idx, float sm_scale,
                                   const void* q, const void* k, const void* v, const void* o,
                                   const void* o_lo, const void* dout, const float* lse, float* dq,
                                   float* dk, float* dv, void* stream);

/* ---- a6 / a7 with token-order outputs ------------------------------------------------ *
 * The same attention as prism_bsa_fwd / prism_bsa_bwd, with the caller-facing tensors in token
 * order [N, heads, head_dim]: the kernels write each output row straight to its token (the
 * inverse of the block order given by shape_idx, which must be the shape map the block-order
 * q, k, v were permuted with), so the separate inverse permutes of O and of the gradients (and
 * their block-order buffers) are not needed.  Results are bitwise those of the block-order
 * calls followed by prism_permute(inverse = 1).
 * prism_bsa_fwd_tok: q, k, v block order (as for prism_bsa_fwd); o and o_lo out in token order;
 *   lse out [heads, N] in block order; workspace as for prism_bsa_fwd.
 * prism_bsa_bwd_tok: q, k, v block order; o, o_lo (prism_bsa_fwd_tok's outputs) and dout in
 *   token order; lse block order; dq, dk, dv out [N, heads, head_dim] fp32 in token order.
 *   The workspace (prism_bsa_bwd_tok_workspace_bytes, 256-byte aligned) also holds a
 *   block-order copy of dout.
 * Errors as for the block-order calls; shape_idx must be non-NULL. */
prism_status prism_bsa_fwd_tok(const prism_problem* pb, const uint8_t* shape_idx, const int32_t* block_start,
                               const int32_t* sel_count, const int32_t* sel_idx, float sm_scale,
                               const void* q, const void* k, const void* v, void* o, void* o_lo,
                               float* lse, void* workspace, size_t workspace_bytes, void* stream);
size_t prism_bsa_bwd_tok_workspace_bytes(const prism_problem* pb);
prism_status prism_bsa_bwd_tok(const prism_problem* pb, const uint8_t* shape_idx, const int32_t* block_start,
                               const int32_t* sel_count, const int32_t* sel_idx, float sm_scale,
                               const void* q, const void* k, const void* v, const void* o,
                               const void* o_lo, const void* dout, const float* lse, float* dq,
                               float* dk, float* dv, void* workspace, size_t workspace_bytes,
                               void* stream);

/* ---- launch order switch ------------------------------------------------------------- *
 * heavy_first = 1 (the default): the matrix-core attention kernels launch their heaviest units
 * (pairs of atoms, atoms) first; 0: every launch uses the plain order (atoms of a head in the
 * XCD-contiguous order).  Results are bitwise the same either way; the switch is process-wide
 * and not thread-safe, meant for tests and measurements.  PRISM_E_RANGE for other values. */
prism_status prism_set_launch_order(int32_t heavy_first);

/* ---- measurement hook --------------------------------------------------------------- *
 * Records the HIP events start_event / stop_event (hipEvent_t passed as void*, created by
 * the caller) immediately before and after every later launch of the library kernel named
 * `kernel` (e.g. "k_fwd", "k_dq", "k_dkdv", "k_zone_stats", "k_permute", "k_pool",
 * "k_scores", "k_select"), on that launch's stream, so a caller can time one kernel inside a
 * multi-kernel call.  Up to 8 kernels can be traced at once; calling again with the same name
 * replaces its events, and kernel == NULL clears every hook.  The hook is process-wide and
 * not thread-safe; it is meant for benchmarks.  Returns PRISM_E_RANGE when all 8 slots are in
 * use. */
prism_status prism_trace_kernel(const char* kernel, void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif
#endif /* PRISM_H */
