// permute_pool.hip -- token order <-> block order, and block mean-pooling (RG M3).
//
// k_permute: one workgroup per (zone, head, tensor).  A zone's 512 rows of one head map to the
// contiguous block-order range [512 m, 512 m + 512) of that head, so the workgroup streams
// 512 rows of head_dim elements, 16 bytes per thread per step, iterating in the destination's
// order so stores are sequential; every load and store covers whole 128-byte lines.
// k_pool: one workgroup per (block, head, tensor): 16-byte loads of the block's contiguous
// rows, fp32 partial sums per row group, fixed-order LDS reduction, times 1/B (exact).
// k_permute_pool: k_permute and k_pool in one pass over the token-order input.
#include "prism_internal.h"

namespace prism {

namespace {

PRISM_DEVICE_SHAPES

struct PermPtrs {
  const uint8_t* src[4];
  uint8_t* dst[4];
};


template <int CPR_LOG2>  // log2 of 16-byte chunks per row
__global__ __launch_bounds__(256) void k_permute(PermPtrs pp, const uint8_t* __restrict__ shape_idx, int inverse,
                                                 int H, int W, int ZH, int ZW, int Z, int heads, int hpg,
                                                 int64_t N, int rowbytes) {
  const int m = blockIdx.x, h = blockIdx.y, tsel = blockIdx.z;
  const int grp = h / hpg;
  const int zt = m / (ZH * ZW), zh = (m / ZW) % ZH, zw = m % ZW;
  const int s = shape_idx[(int64_t)grp * Z + m];
  const int bT = c_shapes[s].bT, bH = c_shapes[s].bH, bW = c_shapes[s].bW;
  const int lT = ilog2_edge(bT), lH = ilog2_edge(bH), lW = ilog2_edge(bW);
  const int lB = lT + lH + lW;
  const int lnW = 3 - lW, lnH = 3 - lH;  // log2 of blocks along W and H inside the zone
  const uint8_t* src = pp.src[tsel];
  uint8_t* dst = pp.dst[tsel];
  const int64_t tok_stride = (int64_t)heads * rowbytes;
  const int64_t perm_base = ((int64_t)h * N + (int64_t)m * kZoneVol) * rowbytes;
  constexpr int CPR = 1 << CPR_LOG2;
#pragma unroll 4
  for (int q = threadIdx.x; q < kZoneVol * CPR; q += 256) {
    const int lr = q >> CPR_LOG2, ch = q & (CPR - 1);
    int lt, lh, lw, p;
    if (!inverse) {
      // lr = position inside the zone's block-order range
      p = lr;
      const int beta = p >> lB, iota = p & ((1 << lB) - 1);
      const int bw_ = beta & ((1 << lnW) - 1), bh_ = (beta >> lnW) & ((1 << lnH) - 1), bt_ = beta >> (lnW + lnH);
      const int iw = iota & (bW - 1), ih = (iota >> lW) & (bH - 1), it = iota >> (lW + lH);
      lt = (bt_ << lT) + it;
      lh = (bh_ << lH) + ih;
      lw = (bw_ << lW) + iw;
    } else {
      // lr = token raster index inside the zone
      lt = lr >> 6;
      lh = (lr >> 3) & 7;
      lw = lr & 7;
      const int beta = (((lt >> lT) << lnH) + (lh >> lH)) * (1 << lnW) + (lw >> lW);
      const int iota = (((lt & (bT - 1)) << lH) + (lh & (bH - 1))) * bW + (lw & (bW - 1));
      p = (beta << lB) + iota;
    }
    const int64_t n = ((int64_t)(zt * 8 + lt) * H + zh * 8 + lh) * W + zw * 8 + lw;
    const int64_t tok_off = n * tok_stride + (int64_t)h * rowbytes + ch * 16;
    const int64_t perm_off = perm_base + (int64_t)p * rowbytes + ch * 16;
    const int64_t so = inverse ? perm_off : tok_off;
    const int64_t dof = inverse ? tok_off : perm_off;
    *reinterpret_cast<uint4*>(dst + dof) = *reinterpret_cast<const uint4*>(src + so);
  }
}

struct PoolPtrs {
  const uint8_t* x[4];
  float* xbar[4];
};

template <bool BF16, int D>
__global__ __launch_bounds__(256) void k_pool(PoolPtrs pp, const int32_t* __restrict__ block_start, int nbmax,
                                              int hpg, int64_t N) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int EPC = 16 / ESZ;          // elements per 16-byte chunk
  constexpr int CPR = D / EPC;           // chunks per row
  constexpr int RG = 256 / CPR;          // row groups
  __shared__ float red[RG][D + 1];
  const int j = blockIdx.x, h = blockIdx.y, tsel = blockIdx.z;
  const int grp = h / hpg;
  const int32_t* bs = block_start + (int64_t)grp * (nbmax + 1);
  float* out = pp.xbar[tsel] + ((int64_t)h * nbmax + j) * D;
  const int r0 = bs[j], r1 = bs[j + 1];
  if (r0 >= N) {
    for (int e = threadIdx.x; e < D; e += 256) out[e] = 0.f;
    return;
  }
  const int ch = threadIdx.x % CPR, rg = threadIdx.x / CPR;
  const uint8_t* base = pp.x[tsel] + ((int64_t)h * N) * D * ESZ + ch * 16;
  float acc[EPC];
#pragma unroll
  for (int i = 0; i < EPC; ++i) acc[i] = 0.f;
  for (int r = r0 + rg; r < r1; r += RG) {
    const uint4 u = *reinterpret_cast<const uint4*>(base + (int64_t)r * D * ESZ);
    if constexpr (BF16) {
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += bf16_lo(w[i]);
        acc[2 * i + 1] += bf16_hi(w[i]);
      }
    } else {
      acc[0] += __uint_as_float(u.x);
      acc[1] += __uint_as_float(u.y);
      acc[2] += __uint_as_float(u.z);
      acc[3] += __uint_as_float(u.w);
    }
  }
#pragma unroll
  for (int i = 0; i < EPC; ++i) red[rg][ch * EPC + i] = acc[i];
  __syncthreads();
  const float inv = 1.f / (float)(r1 - r0);  // 1/64, 1/128 or 1/256: exact
  for (int e = threadIdx.x; e < D; e += 256) {
    float s = 0.f;
    for (int g2 = 0; g2 < RG; ++g2) s += red[g2][e];
    out[e] = s * inv;
  }
}

// Token -> block order and the pooled block means in one pass: one workgroup per (zone, head,
// tensor) streams the zone's 512 rows in block order exactly as k_permute does and, when the
// tensor has a pooled output, sums each block's rows on the way in k_pool's order (thread
// (chunk, row group), rows r0 + rg + RG*i, then the row groups in order), so xbar is bitwise
// what k_pool gives for the permuted tensor.  The workgroup of zone m also zeroes pooled rows
// N_b + 8m .. N_b + 8m + 7 (so every row past N_b is zero).
template <bool BF16, int D>
__global__ __launch_bounds__(256) void k_permute_pool(PermPtrs pp, PoolPtrs pl, const uint8_t* __restrict__ shape_idx,
                                                      const int32_t* __restrict__ zone_block_off, int H, int W,
                                                      int ZH, int ZW, int Z, int heads, int hpg, int nbmax,
                                                      int64_t N) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int EPC = 16 / ESZ;  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;   // chunks per row
  constexpr int RG = 256 / CPR;  // row groups
  constexpr int RB = D * ESZ;    // bytes per row
  __shared__ float red[RG][D + 1];
  const int m = blockIdx.x, h = blockIdx.y, tsel = blockIdx.z;
  const int grp = h / hpg;
  const int ch = threadIdx.x % CPR, rg = threadIdx.x / CPR;
  const ShapeEntry se = c_shapes[shape_idx[(int64_t)grp * Z + m]];
  const int B = se.vol;
  const uint8_t* src = pp.src[tsel];
  uint8_t* dst = pp.dst[tsel] + ((int64_t)h * N + (int64_t)m * kZoneVol) * RB + ch * 16;
  float* xbar = pl.xbar[tsel];
  const int32_t* zbo = zone_block_off + (int64_t)grp * (Z + 1);
  const float inv = 1.f / (float)B;  // 1/64, 1/128 or 1/256: exact
  for (int b0 = 0; b0 < kZoneVol; b0 += B) {  // one block of the zone
    float acc[EPC];
#pragma unroll
    for (int i = 0; i < EPC; ++i) acc[i] = 0.f;
    for (int p = b0 + rg; p < b0 + B; p += RG) {
      const int64_t n = zone_pos_token(m, p, se.bT, se.bH, se.bW, H, W, ZH, ZW);
      const uint4 u = *reinterpret_cast<const uint4*>(src + (n * heads + h) * RB + ch * 16);
      *reinterpret_cast<uint4*>(dst + (int64_t)p * RB) = u;
      if (xbar) {
        if constexpr (BF16) {
          const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] += bf16_lo(w[i]);
            acc[2 * i + 1] += bf16_hi(w[i]);
          }
        } else {
          acc[0] += __uint_as_float(u.x);
          acc[1] += __uint_as_float(u.y);
          acc[2] += __uint_as_float(u.z);
          acc[3] += __uint_as_float(u.w);
        }
      }
    }
    if (!xbar) continue;
#pragma unroll
    for (int i = 0; i < EPC; ++i) red[rg][ch * EPC + i] = acc[i];
    __syncthreads();
    float* out = xbar + ((int64_t)h * nbmax + zbo[m] + b0 / B) * D;
    for (int e = threadIdx.x; e < D; e += 256) {
      float sum = 0.f;
      for (int g2 = 0; g2 < RG; ++g2) sum += red[g2][e];
      out[e] = sum * inv;
    }
    __syncthreads();
  }
  if (xbar) {
    const int j0 = zbo[Z] + 8 * m;
    for (int e = threadIdx.x; e < 8 * D; e += 256) {
      const int j = j0 + e / D;
      if (j < nbmax) xbar[((int64_t)h * nbmax + j) * D + e % D] = 0.f;
    }
  }
}

}  // namespace

prism_status launch_permute_pool(const Geom& g, const uint8_t* shape_idx, const int32_t* zone_block_off, int count,
                                 const void* const* src, void* const* dst, float* const* xbar, hipStream_t st) {
  PermPtrs pp = {};
  PoolPtrs pl = {};
  for (int i = 0; i < count; ++i) {
    pp.src[i] = static_cast<const uint8_t*>(src[i]);
    pp.dst[i] = static_cast<uint8_t*>(dst[i]);
    pl.xbar[i] = xbar ? xbar[i] : nullptr;
  }
  dim3 grid(g.Z, g.heads, count);
  KernelTrace tr("k_permute_pool", st);
  if (g.bf16) {
    if (g.d == 64)
      hipLaunchKernelGGL((k_permute_pool<true, 64>), grid, dim3(256), 0, st, pp, pl, shape_idx, zone_block_off, g.H,
                         g.W, g.ZH, g.ZW, g.Z, g.heads, g.hpg, g.nbmax, g.N);
    else
      hipLaunchKernelGGL((k_permute_pool<true, 128>), grid, dim3(256), 0, st, pp, pl, shape_idx, zone_block_off, g.H,
                         g.W, g.ZH, g.ZW, g.Z, g.heads, g.hpg, g.nbmax, g.N);
  } else {
    if (g.d == 64)
      hipLaunchKernelGGL((k_permute_pool<false, 64>), grid, dim3(256), 0, st, pp, pl, shape_idx, zone_block_off, g.H,
                         g.W, g.ZH, g.ZW, g.Z, g.heads, g.hpg, g.nbmax, g.N);
    else
      hipLaunchKernelGGL((k_permute_pool<false, 128>), grid, dim3(256), 0, st, pp, pl, shape_idx, zone_block_off, g.H,
                         g.W, g.ZH, g.ZW, g.Z, g.heads, g.hpg, g.nbmax, g.N);
  }
  return check_launch("k_permute_pool");
}

prism_status launch_permute(const Geom& g, const uint8_t* shape_idx, int inverse, int count, const void* const* src,
                            void* const* dst, hipStream_t st) {
  PermPtrs pp = {};
  for (int i = 0; i < count; ++i) {
    pp.src[i] = static_cast<const uint8_t*>(src[i]);
    pp.dst[i] = static_cast<uint8_t*>(dst[i]);
  }
  const int rowbytes = g.d * g.esize;
  dim3 grid(g.Z, g.heads, count);
  KernelTrace tr("k_permute", st);
  switch (rowbytes / 16) {
    case 8:
      hipLaunchKernelGGL(k_permute<3>, grid, dim3(256), 0, st, pp, shape_idx, inverse, g.H, g.W, g.ZH, g.ZW, g.Z,
                         g.heads, g.hpg, g.N, rowbytes);
      break;
    case 16:
      hipLaunchKernelGGL(k_permute<4>, grid, dim3(256), 0, st, pp, shape_idx, inverse, g.H, g.W, g.ZH, g.ZW, g.Z,
                         g.heads, g.hpg, g.N, rowbytes);
      break;
    default:
      hipLaunchKernelGGL(k_permute<5>, grid, dim3(256), 0, st, pp, shape_idx, inverse, g.H, g.W, g.ZH, g.ZW, g.Z,
                         g.heads, g.hpg, g.N, rowbytes);
      break;
  }
  return check_launch("k_permute");
}

prism_status launch_pool(const Geom& g, const int32_t* block_start, int count, const void* const* x,
                         float* const* xbar, hipStream_t st) {
  PoolPtrs pp = {};
  for (int i = 0; i < count; ++i) {
    pp.x[i] = static_cast<const uint8_t*>(x[i]);
    pp.xbar[i] = xbar[i];
  }
  dim3 grid(g.nbmax, g.heads, count);
  KernelTrace tr("k_pool", st);
  if (g.bf16) {
    if (g.d == 64)
      hipLaunchKernelGGL((k_pool<true, 64>), grid, dim3(256), 0, st, pp, block_start, g.nbmax, g.hpg, g.N);
    else
      hipLaunchKernelGGL((k_pool<true, 128>), grid, dim3(256), 0, st, pp, block_start, g.nbmax, g.hpg, g.N);
  } else {
    if (g.d == 64)
      hipLaunchKernelGGL((k_pool<false, 64>), grid, dim3(256), 0, st, pp, block_start, g.nbmax, g.hpg, g.N);
    else
      hipLaunchKernelGGL((k_pool<false, 128>), grid, dim3(256), 0, st, pp, block_start, g.nbmax, g.hpg, g.N);
  }
  return check_launch("k_pool");
}

}  // namespace prism
