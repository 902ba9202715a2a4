// stats.hip -- zone statistics (RG M1) and block volume / shape assignment (RG M2).
//
// k_zone_stats: one workgroup per (zone, head group).  Each thread owns channel pairs of the
// group and walks the zone's 512 tokens in raster order with 4-byte (bf16x2) or 8-byte
// (fp32x2) loads, so each wavefront reads 256-512 contiguous bytes of a token row per load;
// the 64 loads of a T slice are issued together (64 in flight per wave).  Per channel it keeps
// the 8 H-slice and 8 W-slice sums in registers and folds each T slice into a sum of squares as
// soon as it is complete; values are shifted by the zone's first token so the variance formulas
// do not cancel.  Partial variances are reduced over the workgroup in a fixed order
// (deterministic).
// k_zone_finish: one workgroup; global max of the audio zone means, then
// g = r + abar * vhat + eps.
// k_assign_shapes: one workgroup per head group: volume, l*, nearest candidate, exclusive
// scan of blocks per zone, block start rows.
// k_audio_norms: the coupling field the statistics read, a_n = || hhat_n ||_2 of each token's
// cross-attention output: one wave per token row at a time, 16-byte loads, fp32 sums of
// squares per lane, a fixed-order butterfly across the wave.
#include <math.h>

#include "prism_internal.h"

namespace prism {

namespace {

template <bool BF16>
__device__ __forceinline__ float2 load_pair(const void* base, int64_t elem) {
  if constexpr (BF16) {
    uint32_t u = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(base) + elem);
    return make_float2(bf16_lo(u), bf16_hi(u));
  } else {
    return *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(base) + elem);
  }
}

// raw element pairs as loaded (bf16x2 in one dword, or two floats), converted after the loads of
// a whole T slice have been issued
template <bool BF16>
struct RawPair {
  using type = float2;
};
template <>
struct RawPair<true> {
  using type = uint32_t;
};

template <bool BF16>
__device__ __forceinline__ typename RawPair<BF16>::type load_raw(const void* base, int64_t elem) {
  if constexpr (BF16)
    return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(base) + elem);
  else
    return *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(base) + elem);
}

template <bool BF16>
__device__ __forceinline__ float2 raw_pair(typename RawPair<BF16>::type u) {
  if constexpr (BF16)
    return make_float2(bf16_lo(u), bf16_hi(u));
  else
    return u;
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_zone_stats(const void* __restrict__ v, const float* __restrict__ a,
                                                    float* __restrict__ gout, float* __restrict__ rho,
                                                    float* __restrict__ zaud, int H, int W, int ZH, int ZW,
                                                    int Z, int heads, int d, int hpg) {
  const int m = blockIdx.x, grp = blockIdx.y;
  const int zt = m / (ZH * ZW), zh = (m / ZW) % ZH, zw = m % ZW;
  const int D = hpg * d;
  const int64_t rowlen = (int64_t)heads * d;
  const int npairs = D / 2;
  __shared__ float red[4][4];
  __shared__ float aval[512];
  __shared__ float aslice[24];

  float part[4] = {0.f, 0.f, 0.f, 0.f};
  for (int cp = threadIdx.x; cp < npairs; cp += 256) {
    const int64_t c0 = (int64_t)grp * D + 2 * cp;
    float Hs0[8], Hs1[8], Ws0[8], Ws1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) Hs0[i] = Hs1[i] = Ws0[i] = Ws1[i] = 0.f;
    float tsq0 = 0.f, tsq1 = 0.f, sq0 = 0.f, sq1 = 0.f;
    const int64_t n00 = ((int64_t)(zt * 8) * H + zh * 8) * W + zw * 8;
    const float2 shift = load_pair<BF16>(v, n00 * rowlen + c0);
    for (int lt = 0; lt < 8; ++lt) {
      // the slice's 64 loads are all issued before any is used, so a wave keeps 64 of them in
      // flight instead of waiting for each
      typename RawPair<BF16>::type raw[64];
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        const int64_t nrow = ((int64_t)(zt * 8 + lt) * H + zh * 8 + (i >> 3)) * W + zw * 8;
        raw[i] = load_raw<BF16>(v, (nrow + (i & 7)) * rowlen + c0);
      }
      float ts0 = 0.f, ts1 = 0.f;
#pragma unroll
      for (int lh = 0; lh < 8; ++lh) {
        float r0 = 0.f, r1 = 0.f;
#pragma unroll
        for (int lw = 0; lw < 8; ++lw) {
          const float2 x = raw_pair<BF16>(raw[8 * lh + lw]);
          const float y0 = x.x - shift.x, y1 = x.y - shift.y;
          Ws0[lw] += y0;
          Ws1[lw] += y1;
          r0 += y0;
          r1 += y1;
          sq0 = fmaf(y0, y0, sq0);
          sq1 = fmaf(y1, y1, sq1);
        }
        Hs0[lh] += r0;
        Hs1[lh] += r1;
        ts0 += r0;
        ts1 += r1;
      }
      ts0 *= (1.f / 64.f);
      ts1 *= (1.f / 64.f);
      tsq0 = fmaf(ts0, ts0, tsq0);
      tsq1 = fmaf(ts1, ts1, tsq1);
    }
    float tot0 = 0.f, tot1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) { tot0 += Hs0[i]; tot1 += Hs1[i]; }
    const float mu0 = tot0 * (1.f / 512.f), mu1 = tot1 * (1.f / 512.f);
    float vh0 = 0.f, vh1 = 0.f, vw0 = 0.f, vw1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float e;
      e = Hs0[i] * (1.f / 64.f) - mu0; vh0 = fmaf(e, e, vh0);
      e = Hs1[i] * (1.f / 64.f) - mu1; vh1 = fmaf(e, e, vh1);
      e = Ws0[i] * (1.f / 64.f) - mu0; vw0 = fmaf(e, e, vw0);
      e = Ws1[i] * (1.f / 64.f) - mu1; vw1 = fmaf(e, e, vw1);
    }
    part[0] += (tsq0 * 0.125f - mu0 * mu0) + (tsq1 * 0.125f - mu1 * mu1);
    part[1] += vh0 * 0.125f + vh1 * 0.125f;
    part[2] += vw0 * 0.125f + vw1 * 0.125f;
    part[3] += (sq0 * (1.f / 512.f) - mu0 * mu0) + (sq1 * (1.f / 512.f) - mu1 * mu1);
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float s = wave_sum(part[q]);
    if (lane == 0) red[wv][q] = s;
  }

  // audio statistics of this zone (computed once, by the group-0 workgroup)
  const bool do_audio = (a != nullptr) && grp == 0;
  if (do_audio && threadIdx.x < 64) {
    const int lt = threadIdx.x >> 3, lh = threadIdx.x & 7;
    const int64_t nrow = ((int64_t)(zt * 8 + lt) * H + zh * 8 + lh) * W + zw * 8;
    const float4 p0 = *reinterpret_cast<const float4*>(a + nrow);
    const float4 p1 = *reinterpret_cast<const float4*>(a + nrow + 4);
    float* dst = aval + threadIdx.x * 8;
    dst[0] = p0.x; dst[1] = p0.y; dst[2] = p0.z; dst[3] = p0.w;
    dst[4] = p1.x; dst[5] = p1.y; dst[6] = p1.z; dst[7] = p1.w;
  }
  __syncthreads();
  if (do_audio && threadIdx.x < 24) {
    const int ax = threadIdx.x >> 3, i = threadIdx.x & 7;
    float s = 0.f;
    for (int j = 0; j < 8; ++j)
      for (int k = 0; k < 8; ++k) {
        const int idx = (ax == 0) ? (i * 8 + j) * 8 + k : (ax == 1) ? (j * 8 + i) * 8 + k : (j * 8 + k) * 8 + i;
        s += aval[idx];
      }
    aslice[threadIdx.x] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float s2[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) s2[q] = (red[0][q] + red[1][q] + red[2][q] + red[3][q]) / (float)D;
    const float tot = s2[0] + s2[1] + s2[2];
    float* gz = gout + ((int64_t)grp * Z + m) * 3;
#pragma unroll
    for (int ax = 0; ax < 3; ++ax) gz[ax] = (tot > 0.f) ? s2[ax] / tot : (1.f / 3.f);
    rho[(int64_t)grp * Z + m] = (s2[3] > 0.f) ? tot / s2[3] : 0.f;
    if (do_audio) {
      float A = 0.f;
      for (int i = 0; i < 8; ++i) A += aslice[i];
      A *= (1.f / 512.f);
      float va[3];
      for (int ax = 0; ax < 3; ++ax) {
        float acc = 0.f;
        for (int i = 0; i < 8; ++i) {
          const float e = aslice[ax * 8 + i] * (1.f / 64.f) - A;
          acc = fmaf(e, e, acc);
        }
        va[ax] = acc * 0.125f;
      }
      const float vs = va[0] + va[1] + va[2];
      float* za = zaud + (int64_t)m * 4;
      za[0] = A;
      for (int ax = 0; ax < 3; ++ax) za[1 + ax] = (vs > 0.f) ? va[ax] / vs : (1.f / 3.f);
    }
  }
}

__global__ __launch_bounds__(1024) void k_zone_finish(float* __restrict__ gout, float* __restrict__ zaud,
                                                      int has_audio, int Z, int groups, float eps) {
  __shared__ float wmax[16];
  float amax = 0.f;
  if (has_audio)
    for (int m = threadIdx.x; m < Z; m += 1024) amax = fmaxf(amax, zaud[(int64_t)m * 4]);
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = 0.f;
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, wmax[i]);
  for (int m = threadIdx.x; m < Z; m += 1024) {
    float abar = 0.f, vh[3] = {0.f, 0.f, 0.f};
    if (has_audio) {
      float* za = zaud + (int64_t)m * 4;
      abar = (amax > 0.f) ? za[0] / amax : 0.f;
      vh[0] = za[1]; vh[1] = za[2]; vh[2] = za[3];
      za[0] = abar;
    }
    for (int grp = 0; grp < groups; ++grp) {
      float* gz = gout + ((int64_t)grp * Z + m) * 3;
#pragma unroll
      for (int ax = 0; ax < 3; ++ax) gz[ax] = gz[ax] + abar * vh[ax] + eps;
    }
  }
}

// the candidate table, resident in constant memory from load time
PRISM_DEVICE_SHAPES

__device__ __forceinline__ float log2_edge(int e) { return e == 2 ? 1.f : e == 4 ? 2.f : 3.f; }

__global__ __launch_bounds__(1024) void k_assign_shapes(const float* __restrict__ gin, const float* __restrict__ rho,
                                                        float tau128, float tau256, uint8_t* __restrict__ shape_idx,
                                                        int32_t* __restrict__ zone_block_off,
                                                        int32_t* __restrict__ block_start, int Z, int nbmax, int N) {
  const int grp = blockIdx.x;
  __shared__ int nbl[kMaxZones];
  __shared__ int16_t vol_l[kMaxZones];
  __shared__ int wsum[16];
  for (int m = threadIdx.x; m < Z; m += 1024) {
    const int64_t zi = (int64_t)grp * Z + m;
    const float r = rho[zi];
    const int B = (r >= tau128) ? 64 : (r >= tau256) ? 128 : 256;
    const float S = (B == 64) ? 6.f : (B == 128) ? 7.f : 8.f;
    float L[3];
#pragma unroll
    for (int ax = 0; ax < 3; ++ax) L[ax] = log2f(gin[zi * 3 + ax]);
    const float c = (S + 0.5f * (L[0] + L[1] + L[2])) * (1.f / 3.f);
    float ls[3];
#pragma unroll
    for (int ax = 0; ax < 3; ++ax) ls[ax] = -0.5f * L[ax] + c;
    int best = 0;
    float bestd = INFINITY;
    for (int ci = 0; ci < 16; ++ci) {
      if (c_shapes[ci].vol != B) continue;
      const float e0 = log2_edge(c_shapes[ci].bT) - ls[0];
      const float e1 = log2_edge(c_shapes[ci].bH) - ls[1];
      const float e2 = log2_edge(c_shapes[ci].bW) - ls[2];
      const float dd = fmaf(e2, e2, fmaf(e1, e1, e0 * e0));
      if (dd < bestd) { bestd = dd; best = ci; }
    }
    shape_idx[zi] = (uint8_t)best;
    nbl[m] = kZoneVol / B;
    vol_l[m] = (int16_t)B;
  }
  __syncthreads();
  // exclusive scan of nbl over zones: thread t owns zones [2t, 2t+2)
  const int z0 = 2 * threadIdx.x;
  const int a0 = (z0 < Z) ? nbl[z0] : 0;
  const int a1 = (z0 + 1 < Z) ? nbl[z0 + 1] : 0;
  int incl = a0 + a1;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int woff = 0;
  for (int i = 0; i < wv; ++i) woff += wsum[i];
  int total = 0;
  for (int i = 0; i < 16; ++i) total += wsum[i];
  const int excl = woff + incl - (a0 + a1);
  int32_t* zbo = zone_block_off + (int64_t)grp * (Z + 1);
  int32_t* bs = block_start + (int64_t)grp * (nbmax + 1);
  if (z0 < Z) {
    zbo[z0] = excl;
    for (int b = 0; b < a0; ++b) bs[excl + b] = kZoneVol * z0 + b * vol_l[z0];
  }
  if (z0 + 1 < Z) {
    zbo[z0 + 1] = excl + a0;
    for (int b = 0; b < a1; ++b) bs[excl + a0 + b] = kZoneVol * (z0 + 1) + b * vol_l[z0 + 1];
  }
  if (threadIdx.x == 0) zbo[Z] = total;
  for (int j = total + threadIdx.x; j <= nbmax; j += 1024) bs[j] = N;
}

// One shape for every zone: zone m owns blocks [m * nb, (m + 1) * nb) with nb = 512 / B.
__global__ __launch_bounds__(256) void k_fixed_shapes(int shape_index, uint8_t* __restrict__ shape_idx,
                                                      int32_t* __restrict__ zone_block_off,
                                                      int32_t* __restrict__ block_start, int Z, int nbmax, int N) {
  const int grp = blockIdx.y;
  const int B = c_shapes[shape_index].vol;
  const int nb = kZoneVol / B;
  int32_t* zbo = zone_block_off + (int64_t)grp * (Z + 1);
  int32_t* bs = block_start + (int64_t)grp * (nbmax + 1);
  for (int m = blockIdx.x * 256 + threadIdx.x; m <= Z; m += gridDim.x * 256) {
    zbo[m] = m * nb;
    if (m < Z) {
      shape_idx[(int64_t)grp * Z + m] = (uint8_t)shape_index;
      for (int b = 0; b < nb; ++b) bs[m * nb + b] = kZoneVol * m + b * B;
    }
  }
  for (int j = Z * nb + blockIdx.x * 256 + threadIdx.x; j <= nbmax; j += gridDim.x * 256) bs[j] = N;
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_audio_norms(const uint4* __restrict__ x, int64_t N, int chunks, int squared,
                                                     float* __restrict__ a) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t n = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6; n < N; n += nwaves) {
    const uint4* row = x + n * chunks;
    float s = 0.f;
    for (int c = lane; c < chunks; c += 64) {
      const uint4 u = row[c];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (BF16) {
          const float lo = bf16_lo(w[i]), hi = bf16_hi(w[i]);
          s = fmaf(lo, lo, s);
          s = fmaf(hi, hi, s);
        } else {
          const float f = __uint_as_float(w[i]);
          s = fmaf(f, f, s);
        }
      }
    }
    s = wave_sum(s);
    if (lane == 0) a[n] = squared ? s : sqrtf(s);
  }
}

}  // namespace

prism_status launch_audio_norms(const Geom& g, const void* hhat, int channels, int squared, float* a,
                                hipStream_t st) {
  const int chunks = channels * g.esize / 16;
  const int64_t wgs = (g.N + 3) / 4;
  const unsigned grid = (unsigned)(wgs < 8192 ? wgs : 8192);
  KernelTrace tr("k_audio_norms", st);
  if (g.bf16)
    hipLaunchKernelGGL(k_audio_norms<true>, dim3(grid), dim3(256), 0, st, static_cast<const uint4*>(hhat), g.N,
                       chunks, squared, a);
  else
    hipLaunchKernelGGL(k_audio_norms<false>, dim3(grid), dim3(256), 0, st, static_cast<const uint4*>(hhat), g.N,
                       chunks, squared, a);
  return check_launch("k_audio_norms");
}

prism_status launch_zone_stats(const Geom& g, const void* v, const float* a, float eps, float* gout, float* rho,
                               float* zone_audio, hipStream_t st) {
  dim3 grid(g.Z, g.groups);
  {
  KernelTrace tr("k_zone_stats", st);
  if (g.bf16)
    hipLaunchKernelGGL(k_zone_stats<true>, grid, dim3(256), 0, st, v, a, gout, rho, zone_audio, g.H, g.W, g.ZH,
                       g.ZW, g.Z, g.heads, g.d, g.hpg);
  else
    hipLaunchKernelGGL(k_zone_stats<false>, grid, dim3(256), 0, st, v, a, gout, rho, zone_audio, g.H, g.W, g.ZH,
                       g.ZW, g.Z, g.heads, g.d, g.hpg);
  }
  prism_status s = check_launch("k_zone_stats");
  if (s != PRISM_OK) return s;
  hipLaunchKernelGGL(k_zone_finish, dim3(1), dim3(1024), 0, st, gout, zone_audio, a != nullptr ? 1 : 0, g.Z,
                     g.groups, eps);
  return check_launch("k_zone_finish");
}

prism_status launch_assign_shapes(const Geom& g, const float* gin, const float* rho, float tau128, float tau256,
                                  uint8_t* shape_idx, int32_t* zone_block_off, int32_t* block_start,
                                  hipStream_t st) {
  KernelTrace tr("k_assign_shapes", st);
  hipLaunchKernelGGL(k_assign_shapes, dim3(g.groups), dim3(1024), 0, st, gin, rho, tau128, tau256, shape_idx,
                     zone_block_off, block_start, g.Z, g.nbmax, (int)g.N);
  return check_launch("k_assign_shapes");
}

prism_status launch_fixed_shapes(const Geom& g, int shape_index, uint8_t* shape_idx, int32_t* zone_block_off,
                                 int32_t* block_start, hipStream_t st) {
  dim3 grid((unsigned)((g.Z + 256) / 256), g.groups);
  hipLaunchKernelGGL(k_fixed_shapes, grid, dim3(256), 0, st, shape_index, shape_idx, zone_block_off, block_start,
                     g.Z, g.nbmax, (int)g.N);
  return check_launch("k_fixed_shapes");
}

}  // namespace prism
