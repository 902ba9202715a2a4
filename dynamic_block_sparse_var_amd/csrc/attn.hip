// attn.hip -- block-sparse attention (RG M3: online-softmax attention solely across S_i):
// launch logic, backward helpers, and the fp32 path.
//
// bf16 problems run the MFMA kernels of attn_mfma.hip.  fp32 problems run the kernels below:
// one thread per query row (forward, dQ) or key row (dK/dV), fp32 FMA, expf/logf.  They are
// the plain-precision path for fp32 inputs, not tuned.
//
// Backward helpers shared by both paths:
//   k_mask_t     transposed selection bitmap: bit i of word [h][j][i/32] set when j in S_i;
//                every word is written exactly once (no clearing pass), deterministically,
//   k_delta      delta_r = dO_r . O_r in fp32,
//   k_atom_work, k_launch_order
//                the launch orders of the matrix-core dQ and dK/dV kernels (heavy atoms first).
#include <math.h>

#include <mutex>

#include "attn_common.h"

namespace prism {

namespace {

PRISM_DEVICE_SHAPES

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

template <typename T>
__device__ __forceinline__ void st(T* p, int64_t i, float v);
template <>
__device__ __forceinline__ void st<float>(float* p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }

template <typename T, int D>
__global__ __launch_bounds__(64) void k_ref_fwd(const T* __restrict__ q, const T* __restrict__ k,
                                                const T* __restrict__ v, T* __restrict__ o, float* __restrict__ lse,
                                                const int32_t* __restrict__ block_start,
                                                const int32_t* __restrict__ sel_count,
                                                const int32_t* __restrict__ sel_idx, int nbmax, int hpg, int64_t N,
                                                float sm_scale, RowMap rm) {
  const int h = blockIdx.y;
  const int row = blockIdx.x * 64 + threadIdx.x;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  const int i = block_of_row(bs, nbmax, blockIdx.x * 64);
  const int cnt = sel_count[(int64_t)h * nbmax + i];
  const int32_t* list = sel_idx + ((int64_t)h * nbmax + i) * nbmax;
  const int64_t hb = (int64_t)h * N;
  float qr[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qr[e] = ld(q, (hb + row) * D + e);
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int s = 0; s < cnt; ++s) {
    const int j = list[s];
    for (int c = bs[j]; c < bs[j + 1]; ++c) {
      float z = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) z = fmaf(qr[e], ld(k, (hb + c) * D + e), z);
      z *= sm_scale;
      const float mn = fmaxf(m, z);
      const float alpha = expf(m - mn), pz = expf(z - mn);
      l = l * alpha + pz;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(pz, ld(v, (hb + c) * D + e), acc[e] * alpha);
      m = mn;
    }
  }
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  const int64_t orow = out_row(rm, c_shapes, h / hpg, h, gridDim.y, N, row);
#pragma unroll
  for (int e = 0; e < D; ++e) st(o, orow * D + e, acc[e] * inv);
  lse[hb + row] = (l > 0.f) ? m + logf(l) : -INFINITY;
}

template <typename T, int D>
__global__ __launch_bounds__(64) void k_ref_dq(const T* __restrict__ q, const T* __restrict__ k,
                                               const T* __restrict__ v, const T* __restrict__ dout,
                                               const float* __restrict__ lse, const float* __restrict__ delta,
                                               float* __restrict__ dq, const int32_t* __restrict__ block_start,
                                               const int32_t* __restrict__ sel_count,
                                               const int32_t* __restrict__ sel_idx, int nbmax, int hpg, int64_t N,
                                               float sm_scale, RowMap rm) {
  const int h = blockIdx.y;
  const int row = blockIdx.x * 64 + threadIdx.x;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  const int i = block_of_row(bs, nbmax, blockIdx.x * 64);
  const int cnt = sel_count[(int64_t)h * nbmax + i];
  const int32_t* list = sel_idx + ((int64_t)h * nbmax + i) * nbmax;
  const int64_t hb = (int64_t)h * N;
  float qr[D], dor[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qr[e] = ld(q, (hb + row) * D + e);
    dor[e] = ld(dout, (hb + row) * D + e);
    acc[e] = 0.f;
  }
  const float L = lse[hb + row], dl = delta[hb + row];
  for (int s = 0; s < cnt; ++s) {
    const int j = list[s];
    for (int c = bs[j]; c < bs[j + 1]; ++c) {
      float z = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) {
        z = fmaf(qr[e], ld(k, (hb + c) * D + e), z);
        dp = fmaf(dor[e], ld(v, (hb + c) * D + e), dp);
      }
      const float pz = expf(z * sm_scale - L);
      const float ds = pz * (dp - dl);
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(ds, ld(k, (hb + c) * D + e), acc[e]);
    }
  }
  const int64_t orow = out_row(rm, c_shapes, h / hpg, h, gridDim.y, N, row);
#pragma unroll
  for (int e = 0; e < D; ++e) dq[orow * D + e] = acc[e] * sm_scale;
}

template <typename T, int D>
__global__ __launch_bounds__(64) void k_ref_dkdv(const T* __restrict__ q, const T* __restrict__ k,
                                                 const T* __restrict__ v, const T* __restrict__ dout,
                                                 const float* __restrict__ lse, const float* __restrict__ delta,
                                                 float* __restrict__ dk, float* __restrict__ dv,
                                                 const int32_t* __restrict__ block_start,
                                                 const uint32_t* __restrict__ mask_t, int nbmax, int nw, int hpg,
                                                 int64_t N, float sm_scale, RowMap rm) {
  const int h = blockIdx.y;
  const int key = blockIdx.x * 64 + threadIdx.x;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  const int j = block_of_row(bs, nbmax, blockIdx.x * 64);
  const uint32_t* mrow = mask_t + ((int64_t)h * nbmax + j) * nw;
  const int64_t hb = (int64_t)h * N;
  float kr[D], vr[D], adk[D], adv[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    kr[e] = ld(k, (hb + key) * D + e);
    vr[e] = ld(v, (hb + key) * D + e);
    adk[e] = adv[e] = 0.f;
  }
  for (int w = 0; w < nw; ++w) {
    uint32_t bits = mrow[w];
    while (bits) {
      const int i = (w << 5) + __ffs(bits) - 1;
      bits &= bits - 1;
      for (int r = bs[i]; r < bs[i + 1]; ++r) {
        float z = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) {
          z = fmaf(ld(q, (hb + r) * D + e), kr[e], z);
          dp = fmaf(ld(dout, (hb + r) * D + e), vr[e], dp);
        }
        const float pz = expf(z * sm_scale - lse[hb + r]);
        const float ds = pz * (dp - delta[hb + r]);
#pragma unroll
        for (int e = 0; e < D; ++e) {
          adv[e] = fmaf(pz, ld(dout, (hb + r) * D + e), adv[e]);
          adk[e] = fmaf(ds, ld(q, (hb + r) * D + e), adk[e]);
        }
      }
    }
  }
  const int64_t krow = out_row(rm, c_shapes, h / hpg, h, gridDim.y, N, key);
#pragma unroll
  for (int e = 0; e < D; ++e) {
    dk[krow * D + e] = adk[e] * sm_scale;
    dv[krow * D + e] = adv[e];
  }
}

constexpr int kMaskColMax = 8 * kMaxZones;  // NBMAX bound: one LDS column of mask words (64 KB)

// One workgroup per (word column w, head): the lists of query blocks 32w..32w+31 are ORed into
// an LDS column of NBMAX words (dynamic LDS, 4 * NBMAX bytes) (bit b of word j: block j is in the list of query block 32w + b,
// LDS atomics, order-free), which is then written out: word [h][j][w] for every j, once.
__global__ __launch_bounds__(256) void k_mask_t(uint32_t* __restrict__ mask_t, const int32_t* __restrict__ block_start,
                                                const int32_t* __restrict__ sel_count,
                                                const int32_t* __restrict__ sel_idx, int nbmax, int nw, int hpg,
                                                int64_t N) {
  extern __shared__ uint32_t col[];  // nbmax words
  const int w = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  for (int j = tid; j < nbmax; j += blockDim.x) col[j] = 0u;
  __syncthreads();
  for (int b = 0; b < 32; ++b) {
    const int i = 32 * w + b;
    if (i >= nbmax || bs[i] >= N) break;  // past the group's blocks
    const int64_t row = (int64_t)h * nbmax + i;
    const int cnt = sel_count[row];
    const int32_t* list = sel_idx + row * nbmax;
    for (int s = tid; s < cnt; s += blockDim.x) atomicOr(&col[list[s]], 1u << b);
  }
  __syncthreads();
  uint32_t* out = mask_t + (int64_t)h * nbmax * nw + w;
  for (int j = tid; j < nbmax; j += blockDim.x) out[(int64_t)j * nw] = col[j];
}


// Work estimates for the launch orders of the matrix-core backward, per (head, atom): the
// length of the atom's query-block list (the blocks dQ walks) and the number of query blocks
// whose lists hold the atom's key block (the set bits of its transposed-selection row, the
// blocks dK/dV walks).  One wave per (block, head).
__global__ __launch_bounds__(64) void k_atom_work(int32_t* __restrict__ work_q, int32_t* __restrict__ work_k,
                                                  const uint32_t* __restrict__ mask_t,
                                                  const int32_t* __restrict__ block_start,
                                                  const int32_t* __restrict__ sel_count, int nbmax, int nw, int hpg,
                                                  int64_t N) {
  const int i = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  if (bs[i] >= N) return;
  const uint32_t* row = mask_t + ((int64_t)h * nbmax + i) * nw;
  int c = 0;
  for (int w = lane; w < nw; w += 64) c += __popc(row[w]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  const int q = sel_count[(int64_t)h * nbmax + i];
  const int64_t base = (int64_t)h * (N >> 6);
  for (int a = (bs[i] >> 6) + lane; a < (bs[i + 1] >> 6); a += 64) {
    work_q[base + a] = q;
    work_k[base + a] = c;
  }
}

// Launch order of a matrix-core attention kernel; workgroup s orders item set s (the backward:
// 0 dQ, 1 dK/dV; the forward: its pairs of atoms).  Item = head * natoms + unit (atom or pair);
// the unordered launch runs head by head, units in xcd_atom order.  A few query blocks have
// Top-p-extended lists several times longer than the rest (and their key blocks are selected by
// many more query blocks); launched in place they can start near the end of the launch and hold
// it open long after the other workgroups are done.  So the items whose work exceeds f0/10 (set
// 0) or f1/10 (set 1) times the mean go first; both parts keep the unordered relative order,
// which keeps the neighbouring units that share tiles together on one XCD.  Deterministic.
__global__ __launch_bounds__(1024) void k_launch_order(int32_t* __restrict__ order, const int32_t* __restrict__ work,
                                                       int heads, int natoms, int f0, int f1) {
  __shared__ int part[1024];
  __shared__ unsigned long long tot;
  const int tid = threadIdx.x, side = blockIdx.x;
  const int n = heads * natoms;
  int32_t* ord = order + (int64_t)side * n;
  const int32_t* wk = work + (int64_t)side * n;
  auto item_at = [&](int t) { return (t / natoms) * natoms + xcd_atom(t % natoms, natoms); };
  if (tid == 0) tot = 0ull;
  __syncthreads();
  const int per = (n + 1023) / 1024;
  const int t0 = min(n, tid * per), t1 = min(n, t0 + per);
  unsigned long long sum = 0ull;
  for (int t = t0; t < t1; ++t) sum += (unsigned long long)wk[item_at(t)];
  atomicAdd(&tot, sum);
  __syncthreads();
  // heavy: work > (f / 10) * mean, i.e. 10 * work * n > f * total, in integers
  const unsigned long long total = tot;
  const unsigned long long f = (unsigned long long)(side ? f1 : f0);
  auto heavy = [&](int t) { return 10ull * (unsigned long long)wk[item_at(t)] * (unsigned long long)n > f * total; };
  int c = 0;
  for (int t = t0; t < t1; ++t) c += heavy(t);
  part[tid] = c;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < 1024; ++i) {
      const int x = part[i];
      part[i] = run;
      run += x;
    }
    tot = (unsigned long long)run;
  }
  __syncthreads();
  const int nheavy = (int)tot;
  int ph = part[tid], pl = nheavy + (t0 - part[tid]);
  for (int t = t0; t < t1; ++t) {
    if (heavy(t))
      ord[ph++] = item_at(t);
    else
      ord[pl++] = item_at(t);
  }
}


// Work estimates for the forward's launch order, per (head, pair of atoms): in a zone of 64-row
// blocks twice the longest list among the zone's blocks (the forward matches the blocks into
// pairs itself, so each of the zone's four pairs gets the zone's worst case), in a zone of 128-
// or 256-row blocks twice the list length of the pair's block.  One wave per (zone, head).
__global__ __launch_bounds__(64) void k_pair_work(int32_t* __restrict__ work, const int32_t* __restrict__ block_start,
                                                  const int32_t* __restrict__ sel_count, int nbmax, int hpg, int Z) {
  const int m = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  const int32_t* c = sel_count + (int64_t)h * nbmax;
  const int j0 = block_of_row(bs, nbmax, kZoneVol * m);
  const int B = bs[j0 + 1] - bs[j0];
  if (lane < 4) {
    int w = 0;
    if (B == 64) {
      for (int q = 0; q < 8; ++q) w = max(w, c[j0 + q]);
    } else {
      w = c[j0 + (128 * lane) / B];
    }
    work[((int64_t)h * Z + m) * 4 + lane] = 2 * w;
  }
}

// delta = rowsum(dO * O): LPR lanes per row, 16 bytes per lane per step.  O = o + o_lo when the
// forward stored its rounding residual; o and o_lo are read in block or token order (om), dO in
// block order.  Also lse2 = LSE * log2(e), the row statistic in the base-2 units the
// matrix-core backward uses.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_delta(const T* __restrict__ o, const T* __restrict__ olo,
                                               const T* __restrict__ dout, const float* __restrict__ lse,
                                               float* __restrict__ delta, float* __restrict__ lse2, int64_t rows,
                                               RowMap om, int hpg, int heads, int64_t N) {
  constexpr int EPC = 16 / sizeof(T);
  constexpr int LPR = D / EPC;  // lanes per row (8..32)
  const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gt / LPR;
  const int part = (int)(gt % LPR);
  float acc = 0.f;
  if (row < rows) {
    const int h = (int)(row / N);
    const int64_t orow = out_row(om, c_shapes, h / hpg, h, heads, N, (int)(row - (int64_t)h * N));
    const uint4 a = *reinterpret_cast<const uint4*>(o + orow * D + part * EPC);
    const uint4 b = *reinterpret_cast<const uint4*>(dout + row * D + part * EPC);
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
    if constexpr (sizeof(T) == 2) {
      uint32_t wl[4] = {0u, 0u, 0u, 0u};
      if (olo) {
        const uint4 c = *reinterpret_cast<const uint4*>(olo + orow * D + part * EPC);
        wl[0] = c.x; wl[1] = c.y; wl[2] = c.z; wl[3] = c.w;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = fmaf(bf16_lo(wa[i]) + bf16_lo(wl[i]), bf16_lo(wb[i]), acc);
        acc = fmaf(bf16_hi(wa[i]) + bf16_hi(wl[i]), bf16_hi(wb[i]), acc);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(wa[i]), __uint_as_float(wb[i]), acc);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && part == 0) {
    delta[row] = acc;
    lse2[row] = lse[row] * 1.4426950408889634f;
  }
}

template <typename T, int D>
prism_status run_ref_fwd(const Geom& g, const int32_t* bs, const int32_t* cnt, const int32_t* idx, float sm_scale,
                         const void* q, const void* k, const void* v, void* o, float* lse, const RowMap& out,
                         hipStream_t st) {
  dim3 grid((unsigned)(g.N / 64), g.heads);
  hipLaunchKernelGGL((k_ref_fwd<T, D>), grid, dim3(64), 0, st, (const T*)q, (const T*)k, (const T*)v, (T*)o, lse, bs,
                     cnt, idx, g.nbmax, g.hpg, g.N, sm_scale, out);
  return check_launch("k_ref_fwd");
}

template <typename T, int D>
prism_status run_ref_bwd(const Geom& g, const int32_t* bs, const int32_t* cnt, const int32_t* idx, float sm_scale,
                         const void* q, const void* k, const void* v, const void* dout, const float* lse,
                         const float* delta, const uint32_t* mask_t, int nw, float* dq, float* dk, float* dv,
                         const RowMap& out, hipStream_t st) {
  dim3 grid((unsigned)(g.N / 64), g.heads);
  hipLaunchKernelGGL((k_ref_dq<T, D>), grid, dim3(64), 0, st, (const T*)q, (const T*)k, (const T*)v,
                     (const T*)dout, lse, delta, dq, bs, cnt, idx, g.nbmax, g.hpg, g.N, sm_scale, out);
  prism_status s = check_launch("k_ref_dq");
  if (s != PRISM_OK) return s;
  hipLaunchKernelGGL((k_ref_dkdv<T, D>), grid, dim3(64), 0, st, (const T*)q, (const T*)k, (const T*)v,
                     (const T*)dout, lse, delta, dk, dv, bs, mask_t, g.nbmax, nw, g.hpg, g.N, sm_scale, out);
  return check_launch("k_ref_dkdv");
}

}  // namespace

// The allocation-free backward's workspace: a file-scope device array, one copy per device the
// library runs on, held until the process ends.  Host code never uses its name as an address
// (on the host it is only a stand-in for the symbol); the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

prism_status noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  prism_status s = check_hip(hipGetDevice(&dev), "hipGetDevice");
  if (s != PRISM_OK) return s;
  if (dev < 0 || dev >= kMaxDevices) return fail(PRISM_E_RANGE, "device %d beyond the library's %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    s = check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (s != PRISM_OK) return s;
    addr[dev] = p;
  }
  *out = addr[dev];
  return PRISM_OK;
}

BwdWorkspace bwd_workspace_layout(const Geom& g) {
  BwdWorkspace w;
  w.nw = (g.nbmax + 31) / 32;
  w.delta_off = 0;
  const size_t delta_bytes = ((size_t)g.heads * g.N * sizeof(float) + 255) & ~(size_t)255;
  w.lse2_off = delta_bytes;
  w.mask_off = 2 * delta_bytes;
  const size_t mask_words = (size_t)g.heads * g.nbmax * w.nw;
  w.mask_words = mask_words;
  w.order_off = w.mask_off + ((mask_words * sizeof(uint32_t) + 255) & ~(size_t)255);
  w.items = (int)(g.heads * (g.N / 64));
  const size_t pair_bytes = ((size_t)2 * w.items * sizeof(int32_t) + 255) & ~(size_t)255;
  w.work_off = w.order_off + pair_bytes;
  w.total = w.work_off + pair_bytes;
  return w;
}

size_t bsa_bwd_workspace_bytes(const Geom& g) { return bwd_workspace_layout(g).total; }

// Forward workspace: its launch order [items] int32, then the work estimates [items] int32,
// items = heads * N / 128 (pairs of atoms), each 256-byte aligned.
static size_t fwd_items_bytes(const Geom& g) {
  return ((size_t)g.heads * (size_t)(g.N / 128) * sizeof(int32_t) + 255) & ~(size_t)255;
}
size_t bsa_fwd_workspace_bytes(const Geom& g) { return g.bf16 ? 2 * fwd_items_bytes(g) : 0; }

namespace {
bool g_heavy_first = true;
}
bool heavy_first_order() { return g_heavy_first; }
void set_heavy_first_order(bool on) { g_heavy_first = on; }

prism_status launch_bsa_fwd(const Geom& g, const int32_t* bs, const int32_t* cnt, const int32_t* idx, float sm_scale,
                            const void* q, const void* k, const void* v, void* o, void* o_lo, float* lse,
                            void* ws, const RowMap& out, hipStream_t st) {
  if (g.bf16) {
    int32_t* order = nullptr;
    if (ws && heavy_first_order()) {
      // launch order: pairs of atoms with the longest lists first
      order = static_cast<int32_t*>(ws);
      int32_t* work = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + fwd_items_bytes(g));
      hipLaunchKernelGGL(k_pair_work, dim3(g.Z, g.heads), dim3(64), 0, st, work, bs, cnt, g.nbmax, g.hpg, g.Z);
      prism_status s = check_launch("k_pair_work");
      if (s != PRISM_OK) return s;
      hipLaunchKernelGGL(k_launch_order, dim3(1), dim3(1024), 0, st, order, work, g.heads, (int)(g.N / 128), 15,
                         15);
      s = check_launch("k_launch_order");
      if (s != PRISM_OK) return s;
    }
    return launch_mfma_fwd(g, bs, cnt, idx, sm_scale, q, k, v, o, o_lo, lse, order, out, st);
  }
  if (g.d == 64) return run_ref_fwd<float, 64>(g, bs, cnt, idx, sm_scale, q, k, v, o, lse, out, st);
  return run_ref_fwd<float, 128>(g, bs, cnt, idx, sm_scale, q, k, v, o, lse, out, st);
}

prism_status launch_bsa_bwd(const Geom& g, const int32_t* bs, const int32_t* cnt, const int32_t* idx, float sm_scale,
                            const void* q, const void* k, const void* v, const void* o, const void* o_lo,
                            const void* dout, const float* lse, float* dq, float* dk, float* dv, void* ws,
                            const RowMap& o_in, const RowMap& out, hipStream_t st) {
  const BwdWorkspace w = bwd_workspace_layout(g);
  float* delta = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + w.delta_off);
  float* lse2 = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + w.lse2_off);
  uint32_t* mask_t = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + w.mask_off);
  // transposed selection
  if (g.nbmax > kMaskColMax) return fail(PRISM_E_RANGE, "transposed selection: more than %d blocks", kMaskColMax);
  hipLaunchKernelGGL(k_mask_t, dim3(w.nw, g.heads), dim3(256), (size_t)g.nbmax * sizeof(uint32_t), st, mask_t, bs,
                     cnt, idx, g.nbmax, w.nw, g.hpg, g.N);
  prism_status s = check_launch("k_mask_t");
  if (s != PRISM_OK) return s;
  // launch orders of the matrix-core kernels
  int32_t* order = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + w.order_off);
  if (g.bf16) {
    int32_t* work = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + w.work_off);
    hipLaunchKernelGGL(k_atom_work, dim3(g.nbmax, g.heads), dim3(64), 0, st, work, work + w.items, mask_t, bs, cnt,
                       g.nbmax, w.nw, g.hpg, g.N);
    s = check_launch("k_atom_work");
    if (s != PRISM_OK) return s;
    // dQ: 1.5x the mean; dK/dV: 2.5x, which moves fewer key atoms away from the neighbours that
    // share their query tiles in the L2 (measured: dK/dV -0.8 ms against 1.5x, dQ +0.2 ms at 2.5x)
    // with the heavy-first order switched off no unit counts as heavy: the plain order
    const int off = 1 << 30;
    hipLaunchKernelGGL(k_launch_order, dim3(2), dim3(1024), 0, st, order, work, g.heads, (int)(g.N / 64),
                       heavy_first_order() ? 15 : off, heavy_first_order() ? 25 : off);
    s = check_launch("k_launch_order");
    if (s != PRISM_OK) return s;
  }
  // delta
  const int64_t rows = (int64_t)g.heads * g.N;
  const int lpr = g.d * g.esize / 16;
  const int64_t dblocks = (rows * lpr + 255) / 256;
  if (g.bf16) {
    if (g.d == 64)
      hipLaunchKernelGGL((k_delta<uint16_t, 64>), dim3((unsigned)dblocks), dim3(256), 0, st, (const uint16_t*)o,
                         (const uint16_t*)o_lo, (const uint16_t*)dout, lse, delta, lse2, rows, o_in, g.hpg, g.heads, g.N);
    else
      hipLaunchKernelGGL((k_delta<uint16_t, 128>), dim3((unsigned)dblocks), dim3(256), 0, st, (const uint16_t*)o,
                         (const uint16_t*)o_lo, (const uint16_t*)dout, lse, delta, lse2, rows, o_in, g.hpg, g.heads, g.N);
  } else {
    if (g.d == 64)
      hipLaunchKernelGGL((k_delta<float, 64>), dim3((unsigned)dblocks), dim3(256), 0, st, (const float*)o,
                         (const float*)nullptr, (const float*)dout, lse, delta, lse2, rows, o_in, g.hpg, g.heads, g.N);
    else
      hipLaunchKernelGGL((k_delta<float, 128>), dim3((unsigned)dblocks), dim3(256), 0, st, (const float*)o,
                         (const float*)nullptr, (const float*)dout, lse, delta, lse2, rows, o_in, g.hpg, g.heads, g.N);
  }
  s = check_launch("k_delta");
  if (s != PRISM_OK) return s;
  if (g.bf16)
    return launch_mfma_bwd(g, bs, cnt, idx, sm_scale, q, k, v, dout, lse2, delta, mask_t, w.nw, order,
                           order + w.items, dq, dk, dv, out, st);
  if (g.d == 64)
    return run_ref_bwd<float, 64>(g, bs, cnt, idx, sm_scale, q, k, v, dout, lse, delta, mask_t, w.nw, dq, dk, dv, out,
                                  st);
  return run_ref_bwd<float, 128>(g, bs, cnt, idx, sm_scale, q, k, v, dout, lse, delta, mask_t, w.nw, dq, dk, dv, out,
                                 st);
}

}  // namespace prism
