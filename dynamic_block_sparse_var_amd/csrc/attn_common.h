// attn_common.h -- declarations shared by the attention sources (not part of the ABI).
#pragma once

#include "prism_internal.h"

namespace prism {

// Backward workspace: delta [heads, N] fp32, lse2 = LSE * log2(e) [heads, N] fp32, the
// transposed selection bitmap [heads, NBMAX, nw] uint32 (nw = ceil(NBMAX / 32)), then for the
// matrix-core dQ and dK/dV kernels their launch orders [2][items] int32 and the per-atom work
// estimates the orders are built from [2][items] int32 (items = heads * N / 64), each 256-byte
// aligned.
struct BwdWorkspace {
  size_t delta_off, lse2_off, mask_off, mask_words, order_off, work_off, total;
  int nw, items;
};

BwdWorkspace bwd_workspace_layout(const Geom& g);

// order: NULL (plain launch order) or the forward's launch order, items = head * N/128 + pair
prism_status launch_mfma_fwd(const Geom& g, const int32_t* bs, const int32_t* cnt, const int32_t* idx,
                             float sm_scale, const void* q, const void* k, const void* v, void* o, void* o_lo,
                             float* lse, const int32_t* order, const RowMap& out, hipStream_t st);

// Process-wide launch-order switch (prism_set_launch_order): true = heavy units first.
bool heavy_first_order();
prism_status launch_mfma_bwd(const Geom& g, const int32_t* bs, const int32_t* cnt, const int32_t* idx,
                             float sm_scale, const void* q, const void* k, const void* v, const void* dout,
                             const float* lse2, const float* delta, const uint32_t* mask_t, int nw,
                             const int32_t* order_q, const int32_t* order_k, float* dq, float* dk, float* dv,
                             const RowMap& out, hipStream_t st);

}  // namespace prism
