// select.hip -- hybrid Top-k / Top-p key-block selection (RG M3 attended-set equation).
//
// k_scores: per head, the fp32 block-score matrix s_ij = sm_scale * qbar_i . kbar_j as a tiled
// GEMM (128 x 128 output tiles, 16-deep LDS slabs, 8 x 8 outputs per thread read as float4
// rows, sequential fp32 FMA over the head dimension).  The matrix is written into the caller's sel_idx array (same
// [heads, NBMAX, NBMAX] 4-byte footprint), row by row.
// k_select: one 256-thread workgroup per (query block, head).  Thread t holds the row's entries
// j = t + 256q (q < PER; PER = 32 for rows of up to 8192 blocks, 64 up to 16384) as
// order-preserving 32-bit score keys and their exp(s - s_max).  The
// order of the attended-set equation (score descending, block index ascending on ties) is never
// materialised: the two cuts are found by bisection over the key space, both in the same loop --
// the k-th largest key (counts from wave ballots) and the largest key whose upper set holds at
// least p of the probability mass (fp64 sums in a fixed order, so the result is deterministic and
// p = 1 reaches the total exactly).  Entries equal to the cut key are taken in block-index order,
// then the first max(k, n_p) entries are marked in an LDS bitmap (one ballot per 64 entries) and
// compacted in ascending index order into the same row.
#include <math.h>

#include "prism_internal.h"

namespace prism {

namespace {

constexpr int kSelThreads = 256;
constexpr int kSelMaxKeys = 64 * kSelThreads;  // entries a workgroup holds in registers (PER = 64)

__global__ __launch_bounds__(256) void k_scores(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                float* __restrict__ out, const int32_t* __restrict__ block_start,
                                                int nbmax, int hpg, int d, int N, float sm_scale) {
  constexpr int TS = 128, LD = TS + 4;  // output tile edge; LDS row stride (floats)
  const int j0 = blockIdx.x * TS, i0 = blockIdx.y * TS, h = blockIdx.z;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  if (bs[i0] >= N || bs[j0] >= N) return;  // tile entirely past the group's blocks
  __shared__ __attribute__((aligned(16))) float As[16][LD], Bs[16][LD];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  // thread (tx, ty) owns rows i0 + 8ty.. and columns j0 + 8tx.. of the tile
  float acc[8][8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[r][c] = 0.f;
  const float* qh = qbar + (int64_t)h * nbmax * d;
  const float* kh = kbar + (int64_t)h * nbmax * d;
  for (int e0 = 0; e0 < d; e0 += 16) {
    // the slab: 128 rows x 16 values of qbar and of kbar, stored transposed ([e][row])
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = tid + 256 * q, row = idx >> 2, le = (idx & 3) * 4;
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i0 + row < nbmax) a = *reinterpret_cast<const float4*>(qh + (int64_t)(i0 + row) * d + e0 + le);
      if (j0 + row < nbmax) b = *reinterpret_cast<const float4*>(kh + (int64_t)(j0 + row) * d + e0 + le);
      As[le + 0][row] = a.x; As[le + 1][row] = a.y; As[le + 2][row] = a.z; As[le + 3][row] = a.w;
      Bs[le + 0][row] = b.x; Bs[le + 1][row] = b.y; Bs[le + 2][row] = b.z; Bs[le + 3][row] = b.w;
    }
    __syncthreads();
    // each output accumulates over the head dimension in order, one fma per element
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float4 a0 = *reinterpret_cast<const float4*>(&As[e][8 * ty]);
      const float4 a1 = *reinterpret_cast<const float4*>(&As[e][8 * ty + 4]);
      const float4 b0 = *reinterpret_cast<const float4*>(&Bs[e][8 * tx]);
      const float4 b1 = *reinterpret_cast<const float4*>(&Bs[e][8 * tx + 4]);
      const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[r][c] = fmaf(av[r], bv[c], acc[r][c]);
    }
    __syncthreads();
  }
  const int jc = j0 + 8 * tx;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int i = i0 + 8 * ty + r;
    if (i >= nbmax) continue;
    float* o = out + ((int64_t)h * nbmax + i) * nbmax + jc;
    if (jc + 8 <= nbmax) {
      *reinterpret_cast<float4*>(o) =
          make_float4(sm_scale * acc[r][0], sm_scale * acc[r][1], sm_scale * acc[r][2], sm_scale * acc[r][3]);
      *reinterpret_cast<float4*>(o + 4) =
          make_float4(sm_scale * acc[r][4], sm_scale * acc[r][5], sm_scale * acc[r][6], sm_scale * acc[r][7]);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (jc + c < nbmax) o[c] = sm_scale * acc[r][c];
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

// inclusive scan over the 256 threads of a workgroup (fixed order); part = [4] scratch
__device__ __forceinline__ int block_incl_scan(int v, int* part) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) part[wv] = v;
  __syncthreads();
  for (int q = 0; q < wv; ++q) v += part[q];
  __syncthreads();
  return v;
}

// PER entries per thread: 8 * PER bitmap words per row, PER / 32 of them owned by each thread in
// the tie ranking and the compaction
template <int PER>
__global__ __launch_bounds__(kSelThreads) void k_select(int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_count,
                                                        const int32_t* __restrict__ block_start, int nbmax, int hpg,
                                                        int N, int k_abs, double k_frac, double p) {
  constexpr int kSelPer = PER;
  constexpr int WPT = PER / 32;  // bitmap words per thread
  __shared__ uint32_t sel_bits[8 * PER], tie_bits[8 * PER];
  __shared__ uint32_t red_max[4];
  __shared__ uint32_t red_u[2][4][2];  // per-wave counts, double-buffered across rounds
  __shared__ double red_d[2][4];
  __shared__ int part[4];
  const int i = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  const int64_t row = (int64_t)h * nbmax + i;
  if (bs[i] >= N) {
    if (tid == 0) sel_count[row] = 0;
    return;
  }
  // number of blocks of this group: first j with bs[j] >= N
  int lo_b = 0, hi_b = nbmax;
  while (lo_b < hi_b) {
    const int mid = (lo_b + hi_b) >> 1;
    if (bs[mid] < N) lo_b = mid + 1; else hi_b = mid;
  }
  const int nb = lo_b;
  int32_t* rowp = sel_idx + row * nbmax;
  const float* srow = reinterpret_cast<const float*>(rowp);

  // keys (0 marks an entry past the row: every finite score has a key >= 1) and the row max
  uint32_t u[kSelPer];
  uint32_t mx = 0u;
#pragma unroll
  for (int q = 0; q < kSelPer; ++q) {
    const int j = tid + kSelThreads * q;
    u[q] = (j < nb) ? ord_bits(srow[j]) : 0u;
    mx = max(mx, u[q]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
  if (lane == 0) red_max[wv] = mx;
  __syncthreads();
  mx = max(max(red_max[0], red_max[1]), max(red_max[2], red_max[3]));
  const float smax = unord_bits(mx);
  float e[kSelPer];
#pragma unroll
  for (int q = 0; q < kSelPer; ++q) e[q] = u[q] ? expf(unord_bits(u[q]) - smax) : 0.f;

  // count and mass of the entries with key >= v (block totals, the same for every thread)
  auto count_ge = [&](uint32_t v) __attribute__((always_inline)) {
    uint32_t c = 0u;
#pragma unroll
    for (int q = 0; q < kSelPer; ++q) c += __popcll(__ballot(u[q] >= v));
    return c;
  };
  auto mass_ge = [&](uint32_t v) __attribute__((always_inline)) {
    double m = 0.0;
#pragma unroll
    for (int q = 0; q < kSelPer; ++q) {
      float x = e[q];
      asm volatile("" : "+v"(x));  // widen here, not once for all rounds (64 more registers)
      m += (u[q] >= v) ? (double)x : 0.0;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m += __shfl_xor(m, o, 64);
    return m;
  };

  long long kk = (k_abs > 0) ? (long long)k_abs : (long long)ceil(k_frac * (double)nb);
  if (kk < 1) kk = 1;
  if (kk > nb) kk = nb;
  const uint32_t k = (uint32_t)kk;
  // Block totals of per-wave values (fixed order), through LDS slots alternating between
  // rounds so that one barrier per round suffices.
  int round = 0;
  auto reduce_u = [&](uint32_t v) __attribute__((always_inline)) {
    const int sl = round & 1;
    if (lane == 0) red_u[sl][wv][0] = v;
    __syncthreads();
    ++round;
    return red_u[sl][0][0] + red_u[sl][1][0] + red_u[sl][2][0] + red_u[sl][3][0];
  };
  auto reduce_d = [&](double v) __attribute__((always_inline)) {
    const int sl = round & 1;
    if (lane == 0) red_d[sl][wv] = v;
    __syncthreads();
    ++round;
    return ((red_d[sl][0] + red_d[sl][1]) + red_d[sl][2]) + red_d[sl][3];
  };
  // Top-k cut by bisection over the key space: count(>= lk) >= k > count(>= hk).  lk ends on
  // the key of the k-th entry; cgt_k = count(> lk).
  uint32_t lk = 1u, hk = mx + 1u, cgt_k = 0u;
  while (hk - lk > 1u) {
    const uint32_t mk = lk + (hk - lk) / 2u;
    const uint32_t c = reduce_u(count_ge(mk));
    if (c >= k) lk = mk; else { hk = mk; cgt_k = c; }
  }
  // Top-p: the first k entries (those above lk, then the tied ones at lk in index order, all
  // with the same exp) are enough unless their mass falls short of p * total; only then is the
  // Top-p cut searched, below the Top-k cut: mass(>= lp) >= target > mass(>= hp), which makes
  // lp the key of the entry that reaches the target.
  uint32_t n_p = 0u, lp = lk, cgt_p = 0u;
  if (p > 0.0) {
    const double total = reduce_d(mass_ge(1u));  // the same arithmetic as every mass below
    const double target = p * total;
    const double es_k = (double)expf(unord_bits(lk) - smax);
    double mgt = reduce_d(mass_ge(hk));
    if (mgt + (double)(k - cgt_k) * es_k >= target) {
      n_p = k;  // n_p <= k: the Top-k prefix already holds the target mass
    } else {
      lp = 1u;
      uint32_t hp = hk, cge = (uint32_t)nb;
      cgt_p = cgt_k;
      while (hp - lp > 1u) {
        const uint32_t mp = lp + (hp - lp) / 2u;
        const uint32_t c = reduce_u(count_ge(mp));
        const double m = reduce_d(mass_ge(mp));
        if (m >= target) {
          lp = mp;
          cge = c;
        } else {
          hp = mp;
          cgt_p = c;
          mgt = m;
        }
      }
      // the tied entries at lp (equal scores, equal exp) are taken in index order until the
      // target is reached
      const double es = (double)expf(unord_bits(lp) - smax);
      double t = ceil((target - mgt) / es);
      const double ties = (double)(cge - cgt_p);
      if (t < 1.0) t = 1.0;
      if (t > ties) t = ties;
      n_p = cgt_p + (uint32_t)t;
    }
  }
  const uint32_t nsel = max(k, n_p);
  const uint32_t vcut = (n_p > k) ? lp : lk;
  const uint32_t tneed = nsel - ((n_p > k) ? cgt_p : cgt_k);  // tied entries to take

  // bitmaps of the entries above the cut and at the cut (word w covers entries 32w..32w+31)
#pragma unroll
  for (int q = 0; q < kSelPer; ++q) {
    const uint64_t above = __ballot(u[q] > vcut), at = __ballot(u[q] == vcut);
    if (lane == 0) {
      const int w = 2 * wv + 8 * q;
      sel_bits[w] = (uint32_t)above;
      sel_bits[w + 1] = (uint32_t)(above >> 32);
      tie_bits[w] = (uint32_t)at;
      tie_bits[w + 1] = (uint32_t)(at >> 32);
    }
  }
  __syncthreads();
  // thread t owns words WPT*t .. WPT*t + WPT - 1: the tied entries of rank < tneed (in index
  // order) join the selection
  uint32_t sw[WPT];
  int tc = 0;
#pragma unroll
  for (int x = 0; x < WPT; ++x) {
    sw[x] = sel_bits[WPT * tid + x];
    tc += __popc(tie_bits[WPT * tid + x]);
  }
  int trank = block_incl_scan(tc, part) - tc;
#pragma unroll
  for (int x = 0; x < WPT; ++x) {
    uint32_t tw = tie_bits[WPT * tid + x];
    while (tw) {
      const uint32_t b = tw & (0u - tw);
      tw ^= b;
      if ((uint32_t)trank < tneed) sw[x] |= b;
      ++trank;
    }
  }
  // ascending compaction
  int c = 0;
#pragma unroll
  for (int x = 0; x < WPT; ++x) c += __popc(sw[x]);
  int pos = block_incl_scan(c, part) - c;
#pragma unroll
  for (int x = 0; x < WPT; ++x) {
    uint32_t w = sw[x];
    while (w) {
      const int b = __builtin_ctz(w);
      w &= w - 1u;
      PRISM_ASSERT(pos < nb && ((WPT * tid + x) << 5) + b < nb);
      rowp[pos++] = ((WPT * tid + x) << 5) + b;
    }
  }
  if (tid == 0) sel_count[row] = (int32_t)nsel;
}

}  // namespace

prism_status launch_select(const Geom& g, const int32_t* block_start, const float* qbar, const float* kbar,
                           float sm_scale, int32_t k_abs, double k_frac, double p, int32_t* sel_count,
                           int32_t* sel_idx, hipStream_t st) {
  if (g.nbmax > kSelMaxKeys)
    return fail(PRISM_E_SHAPE, "%d blocks exceed the selection capacity of %d", g.nbmax, kSelMaxKeys);
  const int tiles = (g.nbmax + 127) / 128;
  {
  KernelTrace tr("k_scores", st);
  hipLaunchKernelGGL(k_scores, dim3(tiles, tiles, g.heads), dim3(256), 0, st, qbar, kbar,
                     reinterpret_cast<float*>(sel_idx), block_start, g.nbmax, g.hpg, g.d, (int)g.N, sm_scale);
  }
  prism_status s = check_launch("k_scores");
  if (s != PRISM_OK) return s;
  KernelTrace tr("k_select", st);
  if (g.nbmax <= 32 * kSelThreads)
    hipLaunchKernelGGL(k_select<32>, dim3(g.nbmax, g.heads), dim3(kSelThreads), 0, st, sel_idx, sel_count,
                       block_start, g.nbmax, g.hpg, (int)g.N, k_abs, k_frac, p);
  else
    hipLaunchKernelGGL(k_select<64>, dim3(g.nbmax, g.heads), dim3(kSelThreads), 0, st, sel_idx, sel_count,
                       block_start, g.nbmax, g.hpg, (int)g.N, k_abs, k_frac, p);
  return check_launch("k_select");
}

}  // namespace prism
