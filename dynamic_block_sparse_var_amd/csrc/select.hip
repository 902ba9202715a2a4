// select.hip -- hybrid Top-k / Top-p key-block selection (RG M3 attended-set equation).
//
// k_scores: per head, the fp32 block-score matrix s_ij = sm_scale * qbar_i . kbar_j as a tiled
// GEMM (64 x 64 output tiles, 16-deep LDS slabs, 4 x 4 outputs per thread, sequential fp32
// FMA over the head dimension).  The matrix is written into the caller's sel_idx array (same
// [heads, NBMAX, NBMAX] 4-byte footprint), row by row.
// k_select: one 1024-thread workgroup per (query block, head).  It reads its score row into
// LDS as 64-bit keys (order-preserving score bits << 32 | ~index), bitonic-sorts them in
// descending order (ties -> lower index first), takes exp(s - s_max) in sorted order, a
// deterministic block prefix sum for the Top-p cut, then marks the first max(k, n_p) blocks in
// an LDS bitmap and compacts them in ascending index order into the same row.
#include <math.h>

#include "prism_internal.h"

namespace prism {

namespace {

constexpr int kSelMaxKeys = 8192;  // LDS sort capacity (64 KB of 64-bit keys)

__global__ __launch_bounds__(256) void k_scores(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                float* __restrict__ out, const int32_t* __restrict__ block_start,
                                                int nbmax, int hpg, int d, int N, float sm_scale) {
  const int j0 = blockIdx.x * 64, i0 = blockIdx.y * 64, h = blockIdx.z;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  if (bs[i0] >= N || bs[j0] >= N) return;  // tile entirely past the group's blocks
  __shared__ float As[16][68], Bs[16][68];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
  const float* qh = qbar + (int64_t)h * nbmax * d;
  const float* kh = kbar + (int64_t)h * nbmax * d;
  const int lrow = threadIdx.x >> 2, le = (threadIdx.x & 3) * 4;
  for (int e0 = 0; e0 < d; e0 += 16) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i0 + lrow < nbmax) a = *reinterpret_cast<const float4*>(qh + (int64_t)(i0 + lrow) * d + e0 + le);
    if (j0 + lrow < nbmax) b = *reinterpret_cast<const float4*>(kh + (int64_t)(j0 + lrow) * d + e0 + le);
    As[le + 0][lrow] = a.x; As[le + 1][lrow] = a.y; As[le + 2][lrow] = a.z; As[le + 3][lrow] = a.w;
    Bs[le + 0][lrow] = b.x; Bs[le + 1][lrow] = b.y; Bs[le + 2][lrow] = b.z; Bs[le + 3][lrow] = b.w;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float av[4], bv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) av[r] = As[e][ty + 16 * r];
#pragma unroll
      for (int c = 0; c < 4; ++c) bv[c] = Bs[e][tx + 16 * c];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(av[r], bv[c], acc[r][c]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + ty + 16 * r;
    if (i >= nbmax) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = j0 + tx + 16 * c;
      if (j < nbmax) out[((int64_t)h * nbmax + i) * nbmax + j] = sm_scale * acc[r][c];
    }
  }
}

__device__ __forceinline__ uint32_t ord_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

__global__ __launch_bounds__(1024) void k_select(int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_count,
                                                 const int32_t* __restrict__ block_start, int nbmax, int hpg, int N,
                                                 int k_abs, double k_frac, float p) {
  extern __shared__ uint64_t keys[];  // [P2], later reused as the selection bitmap
  __shared__ float wtot[16];
  __shared__ int wcnt[16];
  __shared__ int np_min;
  const int i = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  const int64_t row = (int64_t)h * nbmax + i;
  if (bs[i] >= N) {
    if (tid == 0) sel_count[row] = 0;
    return;
  }
  // number of blocks of this group: first j with bs[j] >= N
  int lo = 0, hi = nbmax;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (bs[mid] < N) lo = mid + 1; else hi = mid;
  }
  const int nb = lo;
  int P2 = 1;
  while (P2 < nb) P2 <<= 1;
  int32_t* rowp = sel_idx + row * nbmax;
  const float* srow = reinterpret_cast<const float*>(rowp);
  for (int j = tid; j < P2; j += 1024)
    keys[j] = (j < nb) ? (((uint64_t)ord_bits(srow[j]) << 32) | (uint32_t)(~(uint32_t)j)) : 0ull;
  if (tid == 0) np_min = nb;
  __syncthreads();
  // bitonic sort, descending
  for (int size = 2; size <= P2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < (P2 >> 1); t += 1024) {
        const int a = 2 * t - (t & (stride - 1));
        const int b = a + stride;
        const uint64_t ka = keys[a], kb = keys[b];
        const bool desc = (a & size) == 0;
        if ((ka < kb) == desc) {
          keys[a] = kb;
          keys[b] = ka;
        }
      }
      __syncthreads();
    }
  }
  // exp(s - s_max) in sorted order, segmented prefix sums (thread t owns [t*CH, t*CH + CH))
  const float smax = unord_bits((uint32_t)(keys[0] >> 32));
  const int CH = (P2 + 1023) / 1024;
  const int r0 = tid * CH;
  float lsum = 0.f;
  for (int r = r0; r < r0 + CH && r < nb; ++r) lsum += expf(unord_bits((uint32_t)(keys[r] >> 32)) - smax);
  // block exclusive scan of lsum (fixed order)
  const int lane = tid & 63, wv = tid >> 6;
  float incl = lsum;
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wtot[wv] = incl;
  __syncthreads();
  float before = 0.f, total = 0.f;
  for (int q = 0; q < 16; ++q) {
    if (q < wv) before += wtot[q];
    total += wtot[q];
  }
  before += incl - lsum;
  const float target = p * total;
  if (p > 0.f) {
    float run = before;
    for (int r = r0; r < r0 + CH && r < nb; ++r) {
      run += expf(unord_bits((uint32_t)(keys[r] >> 32)) - smax);
      if (run >= target) {
        atomicMin(&np_min, r + 1);
        break;
      }
    }
  } else if (tid == 0) {
    np_min = 0;
  }
  __syncthreads();
  const int n_p = np_min;
  long long kk = (k_abs > 0) ? (long long)k_abs : (long long)ceil(k_frac * (double)nb);
  if (kk < 1) kk = 1;
  if (kk > nb) kk = nb;
  const int nsel = (n_p > (int)kk) ? n_p : (int)kk;
  // take this thread's selected block indices out of the key array, then reuse it as a bitmap
  uint32_t myj[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int r = r0 + u;
    myj[u] = (u < CH && r < nsel) ? ~(uint32_t)(keys[r] & 0xffffffffull) : 0xffffffffu;
  }
  __syncthreads();
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(keys);  // NW words fit in the P2 keys
  const int NW = (nb + 31) >> 5;
  for (int w = tid; w < NW; w += 1024) bitmap[w] = 0u;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (myj[u] != 0xffffffffu) atomicOr(&bitmap[myj[u] >> 5], 1u << (myj[u] & 31));
  __syncthreads();
  // ascending compaction: thread t owns bitmap words [t*WPT, t*WPT + WPT)
  const int WPT = (NW + 1023) / 1024;
  int c = 0;
  for (int w = tid * WPT; w < tid * WPT + WPT && w < NW; ++w) c += __popc(bitmap[w]);
  int ci = c;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(ci, o, 64);
    if (lane >= o) ci += y;
  }
  if (lane == 63) wcnt[wv] = ci;
  __syncthreads();
  int pos = ci - c;
  for (int q = 0; q < wv; ++q) pos += wcnt[q];
  for (int w = tid * WPT; w < tid * WPT + WPT && w < NW; ++w) {
    uint32_t bits = bitmap[w];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      rowp[pos++] = (w << 5) + b;
    }
  }
  if (tid == 0) sel_count[row] = nsel;
}

}  // namespace

prism_status launch_select(const Geom& g, const int32_t* block_start, const float* qbar, const float* kbar,
                           float sm_scale, int32_t k_abs, double k_frac, double p, int32_t* sel_count,
                           int32_t* sel_idx, hipStream_t st) {
  if (g.nbmax > kSelMaxKeys)
    return fail(PRISM_E_SHAPE, "%d blocks exceed the selection capacity of %d", g.nbmax, kSelMaxKeys);
  const int tiles = (g.nbmax + 63) / 64;
  {
  KernelTrace tr("k_scores", st);
  hipLaunchKernelGGL(k_scores, dim3(tiles, tiles, g.heads), dim3(256), 0, st, qbar, kbar,
                     reinterpret_cast<float*>(sel_idx), block_start, g.nbmax, g.hpg, g.d, (int)g.N, sm_scale);
  }
  prism_status s = check_launch("k_scores");
  if (s != PRISM_OK) return s;
  int P2 = 1;
  while (P2 < g.nbmax) P2 <<= 1;
  const size_t lds = (size_t)P2 * sizeof(uint64_t);
  KernelTrace tr("k_select", st);
  hipLaunchKernelGGL(k_select, dim3(g.nbmax, g.heads), dim3(1024), lds, st, sel_idx, sel_count, block_start, g.nbmax,
                     g.hpg, (int)g.N, k_abs, k_frac, (float)p);
  return check_launch("k_select");
}

}  // namespace prism
