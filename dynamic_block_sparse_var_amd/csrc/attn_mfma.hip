// attn_mfma.hip -- bf16 block-sparse attention forward and backward on gfx950 matrix cores
// (RG M3: online-softmax attention solely across the selected key blocks S_i).
//
// Work decomposition.  Every block holds 64, 128 or 256 rows and starts on a multiple of 64,
// so the unit of work is a 64-row "atom" of one head.  A workgroup is two wave64s; each wave
// owns 32 rows (or 32 keys) of the atom.  The other operand is streamed in 64-row tiles that
// are staged once per workgroup in LDS, row-major, and shared by both waves; the next tile's
// global loads are issued before the current tile is computed (register double buffering).
// Atoms are assigned so that each of the 8 XCDs walks a contiguous range of atoms
// (neighbouring blocks tend to select the same key blocks, which then stay in that XCD's L2).
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16): operand A holds A[m = lane%32][8 k-values],
// operand B holds B[8 k-values][n = lane%32]; both use lane/32 to pick which half of the 16
// k-slots they hold.  The accumulator holds C[m = 8*jj + 4*(lane/32) + e][n = lane%32] in
// element 4*jj + e.
//  - Reductions over the head dimension read 8 consecutive elements of a tile row with one
//    ds_read_b128 (the k-slot -> d map only has to agree between A and B).
//  - Reductions over keys or query rows need, per lane, 8 rows of one column.  A lane's
//    accumulator holds rows {8*jj + 4*h + e}; for k-step t the slots are mapped to rows
//    16t + 8*(e/4) + 4*h + e%4, so the accumulator converted to bf16 is directly the B (or A)
//    operand of the next product, and the other operand is read from the row-major tile with
//    two ds_read_b64_tr_b16 (gfx950 transposing LDS read: within each 16-lane group, lane i
//    receives element i%4 of the 8-byte reads of lanes 4e + i/4, e = 0..3).
//
// Forward:  S^T = K Q^T (A = K tile, B = Q rows in registers), online softmax per query row
//           (each lane owns one row; the other 32 keys of a tile sit in lane ^ 32; the
//           running max is only raised when a tile exceeds it by 2^8, so the O rescale is
//           rare), O^T += V^T P^T with P split into a bf16 head and residual.
// dQ:       S^T = K Q^T, dP^T = V dO^T, dS^T = P^T * (dP^T - delta), dQ^T += K^T dS^T.
// dK, dV:   key-major: for every query block whose list contains the key block (transposed
//           selection bitmap), S = Q K^T, dP = dO V^T, P, dS, dV += P^T dO, dK += dS^T Q.
// Products with P and dS use a bf16 head plus a bf16 residual of the fp32 value, so the
// results keep fp32-level accuracy.
#include <math.h>

#include "attn_common.h"

namespace prism {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;  // log2 units the running max may lag behind

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two floats -> two bf16 (round to nearest even) in one instruction (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  f32x2 v;
  v[0] = a;
  v[1] = b;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 8 accumulator elements [off, off + 8) as a bf16 head plus a bf16 residual (the residual
// x - head is exact in fp32)
__device__ __forceinline__ void pack8_split(const f32x16& x, int off, bf16x8& hi, bf16x8& lo) {
  u32x4 H, Lo;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = x[off + 2 * i], b = x[off + 2 * i + 1];
    const uint32_t h = cvt2(a, b);
    H[i] = h;
    Lo[i] = cvt2(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xffff0000u));
  }
  hi = as_bf16x8(H);
  lo = as_bf16x8(Lo);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

template <int D>
struct Cfg {
  static constexpr int KP = D + 8;          // row-major tile pitch, elements (2*D + 16 bytes)
  static constexpr int CPR = D / 8;         // 16-byte chunks per row
  static constexpr int RPP = 128 / CPR;     // rows per pass of 128 threads
  static constexpr int NIT = 64 / RPP;      // 16-byte loads per thread for a 64-row tile
  static constexpr int DS = D / 16;         // k-steps over the head dimension
  static constexpr int DB = D / 32;         // 32-wide blocks of the head dimension
  static constexpr int TILE = 64 * KP;      // elements of one staged tile
};

// global -> registers: thread t takes chunk t % CPR of rows t / CPR + RPP * it
template <int D>
__device__ __forceinline__ void gload(const uint16_t* __restrict__ base, u32x4 (&r)[Cfg<D>::NIT], int tid) {
  const int c = tid % Cfg<D>::CPR, r0 = tid / Cfg<D>::CPR;
#pragma unroll
  for (int it = 0; it < Cfg<D>::NIT; ++it)
    r[it] = *reinterpret_cast<const u32x4*>(base + (int64_t)(r0 + Cfg<D>::RPP * it) * D + 8 * c);
}

template <int D>
__device__ __forceinline__ void lstore(uint16_t* s, const u32x4 (&r)[Cfg<D>::NIT], int tid) {
  const int c = tid % Cfg<D>::CPR, r0 = tid / Cfg<D>::CPR;
#pragma unroll
  for (int it = 0; it < Cfg<D>::NIT; ++it)
    *reinterpret_cast<u32x4*>(s + (r0 + Cfg<D>::RPP * it) * Cfg<D>::KP + 8 * c) = r[it];
}

__device__ __forceinline__ u32x4 lds16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ u32x2 lds_tr(const uint16_t* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p)));
}

// Operand holding X[R0 + 8*(e/4) + 4*(lane/32) + e%4][D0 + lane%32], e = 0..7, of a row-major
// tile X (pitch KP) -- the lane's 8 k-slots when the product reduces over rows.
template <int D>
__device__ __forceinline__ bf16x8 lds_rows_operand(const uint16_t* s, int R0, int D0, int lane) {
  const int j = lane & 15;
  const int row = R0 + 4 * (lane >> 5) + (j >> 2);
  const int col = D0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const u32x2 a = lds_tr(s + row * Cfg<D>::KP + col);
  const u32x2 b = lds_tr(s + (row + 8) * Cfg<D>::KP + col);
  u32x4 v;
  v[0] = a[0];
  v[1] = a[1];
  v[2] = b[0];
  v[3] = b[1];
  return as_bf16x8(v);
}

// atoms of one head, spread so that each XCD (workgroup id mod 8) walks a contiguous range
__device__ __forceinline__ int xcd_atom(int bid, int natoms) {
  return ((natoms & 7) == 0) ? (bid & 7) * (natoms >> 3) + (bid >> 3) : bid;
}

// copy a staged 64 x D bf16 tile (pitch KP) to global rows
template <int D>
__device__ __forceinline__ void copy_out(uint16_t* __restrict__ dst, const uint16_t* s, int tid) {
  const int c = tid % Cfg<D>::CPR, r0 = tid / Cfg<D>::CPR;
#pragma unroll
  for (int it = 0; it < Cfg<D>::NIT; ++it) {
    const int r = r0 + Cfg<D>::RPP * it;
    *reinterpret_cast<u32x4*>(dst + (int64_t)r * D + 8 * c) = lds16(s + r * Cfg<D>::KP + 8 * c);
  }
}

// Walks the 64-row tiles of the key blocks in a selection list (wave-uniform state).
struct ListTiles {
  const int32_t* list;
  const int32_t* bs;
  int cnt, sidx, kt, kend;
  __device__ void begin(const int32_t* l, const int32_t* b, int c) {
    list = l;
    bs = b;
    cnt = c;
    sidx = 0;
    kt = kend = 0;
    if (cnt > 0) {
      const int j = list[0];
      kt = bs[j];
      kend = bs[j + 1];
    }
  }
  __device__ bool valid() const { return sidx < cnt; }
  __device__ void next() {
    kt += 64;
    if (kt >= kend) {
      ++sidx;
      if (sidx < cnt) {
        const int j = list[sidx];
        kt = bs[j];
        kend = bs[j + 1];
      }
    }
  }
};

// Walks the 64-row tiles of the query blocks whose bit is set in a transposed-selection row.
struct MaskTiles {
  const uint32_t* mrow;
  const int32_t* bs;
  int nw, wi, rt, rend;
  uint32_t bits;
  __device__ void advance_block() {
    while (true) {
      while (bits == 0u) {
        if (++wi >= nw) return;
        bits = mrow[wi];
      }
      const int qb = (wi << 5) + __ffs(bits) - 1;
      bits &= bits - 1;
      rt = bs[qb];
      rend = bs[qb + 1];
      return;
    }
  }
  __device__ void begin(const uint32_t* m, const int32_t* b, int n) {
    mrow = m;
    bs = b;
    nw = n;
    wi = 0;
    rt = rend = 0;
    bits = (nw > 0) ? mrow[0] : 0u;
    if (nw > 0) advance_block();
  }
  __device__ bool valid() const { return wi < nw; }
  __device__ void next() {
    rt += 64;
    if (rt >= rend) advance_block();
  }
};

// ------------------------------------------------------------------------------------------
// forward

template <int D>
__global__ __launch_bounds__(128, 2) void k_fwd(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                                                uint16_t* __restrict__ Olo, float* __restrict__ LSE,
                                                const int32_t* __restrict__ block_start,
                                                const int32_t* __restrict__ sel_count,
                                                const int32_t* __restrict__ sel_idx, int nbmax, int hpg, int N,
                                                float scale2) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t sK[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[C::TILE];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const int h = blockIdx.y;
  const int natoms = N >> 6;
  const int row0 = xcd_atom(blockIdx.x, natoms) * 64;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  const int qb = block_of_row(bs, nbmax, row0);
  const int64_t hoff = (int64_t)h * N * D;
  const uint16_t* Kh = K + hoff;
  const uint16_t* Vh = V + hoff;

  bf16x8 qop[C::DS];
  {
    const uint16_t* qr = Q + hoff + (int64_t)(row0 + 32 * w + l32) * D + (D / 2) * half;
#pragma unroll
    for (int s = 0; s < C::DS; ++s) qop[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qr + 8 * s));
  }
  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = zero16();
  float mrow = -INFINITY, lrow = 0.f;

  ListTiles it;
  it.begin(sel_idx + ((int64_t)h * nbmax + qb) * nbmax, bs, sel_count[(int64_t)h * nbmax + qb]);
  u32x4 kreg[C::NIT], vreg[C::NIT];
  if (it.valid()) {
    gload<D>(Kh + (int64_t)it.kt * D, kreg, tid);
    gload<D>(Vh + (int64_t)it.kt * D, vreg, tid);
  }
  while (it.valid()) {
    __syncthreads();
    lstore<D>(sK, kreg, tid);
    lstore<D>(sV, vreg, tid);
    __syncthreads();
    it.next();
    if (it.valid()) {
      gload<D>(Kh + (int64_t)it.kt * D, kreg, tid);
      gload<D>(Vh + (int64_t)it.kt * D, vreg, tid);
    }
    // S^T = K Q^T for this wave's 32 rows
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = zero16();
      const uint16_t* ka = sK + (32 * kb + l32) * C::KP + (D / 2) * half;
#pragma unroll
      for (int s = 0; s < C::DS; ++s) sacc[kb] = mfma(as_bf16x8(lds16(ka + 8 * s)), qop[s], sacc[kb]);
    }
    // online softmax in base 2 (logits scaled by sm_scale * log2 e); the running max is
    // raised (and O rescaled) only when this tile exceeds it by more than the slack
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale2;
    if (__any(mx > mrow + kRescaleSlack)) {
      const float mnew = fmaxf(mrow, mx);
      const float alpha = __builtin_amdgcn_exp2f(mrow - mnew);
      lrow *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
      mrow = mnew;
    }
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], scale2, -mrow));
        sacc[kb][r] = pv;
        psum += pv;
      }
    lrow += psum + __shfl_xor(psum, 32, 64);
    // O^T += V^T P^T, P as bf16 head + residual
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bf16x8 p_hi, p_lo;
      pack8_split(sacc[t >> 1], 8 * (t & 1), p_hi, p_lo);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const bf16x8 vt_op = lds_rows_operand<D>(sV, 16 * t, 32 * db, lane);
        oacc[db] = mfma(vt_op, p_hi, oacc[db]);
        oacc[db] = mfma(vt_op, p_lo, oacc[db]);
      }
    }
  }
  const float inv = (lrow > 0.f) ? 1.f / lrow : 0.f;
  if (half == 0) LSE[(int64_t)h * N + row0 + 32 * w + l32] = (lrow > 0.f) ? (mrow + log2f(lrow)) * kLn2 : -INFINITY;
  uint16_t* sO = sK;
  // pass 0 writes O rounded to bf16, pass 1 (if requested) its rounding residual
  for (int pass = 0; pass < (Olo ? 2 : 1); ++pass) {
    __syncthreads();
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float ov[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ov[e] = oacc[db][4 * jj + e] * inv;
          if (pass) ov[e] -= bf16_to_f32(f32_to_bf16(ov[e]));
        }
        u32x2 pk;
        pk[0] = pack_bf16x2(ov[0], ov[1]);
        pk[1] = pack_bf16x2(ov[2], ov[3]);
        *reinterpret_cast<u32x2*>(sO + (32 * w + l32) * C::KP + 32 * db + 8 * jj + 4 * half) = pk;
      }
    __syncthreads();
    copy_out<D>((pass ? Olo : O) + hoff + (int64_t)row0 * D, sO, tid);
  }
}

// ------------------------------------------------------------------------------------------
// backward, query-major: dQ

template <int D>
__global__ __launch_bounds__(128, 1) void k_dq(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                               const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                                               const float* __restrict__ LSE, const float* __restrict__ delta,
                                               float* __restrict__ dQ, const int32_t* __restrict__ block_start,
                                               const int32_t* __restrict__ sel_count,
                                               const int32_t* __restrict__ sel_idx, int nbmax, int hpg, int N,
                                               float scale2, float sm_scale) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t sK[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[C::TILE];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const int h = blockIdx.y;
  const int natoms = N >> 6;
  const int row0 = xcd_atom(blockIdx.x, natoms) * 64;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  const int qb = block_of_row(bs, nbmax, row0);
  const int64_t hoff = (int64_t)h * N * D;
  const uint16_t* Kh = K + hoff;
  const uint16_t* Vh = V + hoff;
  const int myrow = row0 + 32 * w + l32;

  bf16x8 qop[C::DS], doop[C::DS];
  {
    const uint16_t* qr = Q + hoff + (int64_t)myrow * D + (D / 2) * half;
    const uint16_t* dr = dO + hoff + (int64_t)myrow * D + (D / 2) * half;
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      qop[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qr + 8 * s));
      doop[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(dr + 8 * s));
    }
  }
  const float lse2 = LSE[(int64_t)h * N + myrow] * kLog2e;
  const float dl = delta[(int64_t)h * N + myrow];
  f32x16 dqacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dqacc[db] = zero16();

  ListTiles it;
  it.begin(sel_idx + ((int64_t)h * nbmax + qb) * nbmax, bs, sel_count[(int64_t)h * nbmax + qb]);
  u32x4 kreg[C::NIT], vreg[C::NIT];
  if (it.valid()) {
    gload<D>(Kh + (int64_t)it.kt * D, kreg, tid);
    gload<D>(Vh + (int64_t)it.kt * D, vreg, tid);
  }
  while (it.valid()) {
    __syncthreads();
    lstore<D>(sK, kreg, tid);
    lstore<D>(sV, vreg, tid);
    __syncthreads();
    it.next();
    if (it.valid()) {
      gload<D>(Kh + (int64_t)it.kt * D, kreg, tid);
      gload<D>(Vh + (int64_t)it.kt * D, vreg, tid);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sacc = zero16(), dpacc = zero16();
      const uint16_t* ka = sK + (32 * kb + l32) * C::KP + (D / 2) * half;
      const uint16_t* va = sV + (32 * kb + l32) * C::KP + (D / 2) * half;
#pragma unroll
      for (int s = 0; s < C::DS; ++s) {
        sacc = mfma(as_bf16x8(lds16(ka + 8 * s)), qop[s], sacc);
        dpacc = mfma(as_bf16x8(lds16(va + 8 * s)), doop[s], dpacc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale2, -lse2));
        sacc[r] = pv * (dpacc[r] - dl);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        bf16x8 ds_hi, ds_lo;
        pack8_split(sacc, 8 * tt, ds_hi, ds_lo);
        const int t = 2 * kb + tt;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const bf16x8 kt_op = lds_rows_operand<D>(sK, 16 * t, 32 * db, lane);
          dqacc[db] = mfma(kt_op, ds_hi, dqacc[db]);
          dqacc[db] = mfma(kt_op, ds_lo, dqacc[db]);
        }
      }
    }
  }
  // fp32 output: lane holds dQ[myrow][32db + 8jj + 4half + e]
  float* dqr = dQ + hoff + (int64_t)myrow * D + 4 * half;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float4 v4;
      v4.x = dqacc[db][4 * jj + 0] * sm_scale;
      v4.y = dqacc[db][4 * jj + 1] * sm_scale;
      v4.z = dqacc[db][4 * jj + 2] * sm_scale;
      v4.w = dqacc[db][4 * jj + 3] * sm_scale;
      *reinterpret_cast<float4*>(dqr + 32 * db + 8 * jj) = v4;
    }
}

// ------------------------------------------------------------------------------------------
// backward, key-major: dK, dV

template <int D>
__global__ __launch_bounds__(128, 1) void k_dkdv(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                 const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                                                 const float* __restrict__ LSE, const float* __restrict__ delta,
                                                 float* __restrict__ dK, float* __restrict__ dV,
                                                 const int32_t* __restrict__ block_start,
                                                 const uint32_t* __restrict__ mask_t, int nbmax, int nw, int hpg,
                                                 int N, float scale2, float sm_scale) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[C::TILE];
  __shared__ __attribute__((aligned(16))) float sL[64];
  __shared__ __attribute__((aligned(16))) float sD[64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const int h = blockIdx.y;
  const int natoms = N >> 6;
  const int key0 = xcd_atom(blockIdx.x, natoms) * 64;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  const int kb_idx = block_of_row(bs, nbmax, key0);
  const int64_t hoff = (int64_t)h * N * D;
  const int mykey = key0 + 32 * w + l32;

  bf16x8 kop[C::DS], vop[C::DS];
  {
    const uint16_t* kr = K + hoff + (int64_t)mykey * D + (D / 2) * half;
    const uint16_t* vr = V + hoff + (int64_t)mykey * D + (D / 2) * half;
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      kop[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(kr + 8 * s));
      vop[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(vr + 8 * s));
    }
  }
  f32x16 dkacc[C::DB], dvacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    dkacc[db] = zero16();
    dvacc[db] = zero16();
  }

  MaskTiles it;
  it.begin(mask_t + ((int64_t)h * nbmax + kb_idx) * nw, bs, nw);
  u32x4 qreg[C::NIT], oreg[C::NIT];
  float lv = 0.f, dv = 0.f;
  auto prefetch = [&](int rt) {
    gload<D>(Q + hoff + (int64_t)rt * D, qreg, tid);
    gload<D>(dO + hoff + (int64_t)rt * D, oreg, tid);
    if (tid < 64) {
      lv = LSE[(int64_t)h * N + rt + tid] * kLog2e;
      dv = delta[(int64_t)h * N + rt + tid];
    }
  };
  if (it.valid()) prefetch(it.rt);
  while (it.valid()) {
    __syncthreads();
    lstore<D>(sQ, qreg, tid);
    lstore<D>(sdO, oreg, tid);
    if (tid < 64) {
      sL[tid] = lv;
      sD[tid] = dv;
    }
    __syncthreads();
    it.next();
    if (it.valid()) prefetch(it.rt);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      // S = Q K^T and dP = dO V^T for query rows 32rb.. of the tile, this wave's 32 keys
      f32x16 sacc = zero16(), dpacc = zero16();
      const uint16_t* qa = sQ + (32 * rb + l32) * C::KP + (D / 2) * half;
      const uint16_t* oa = sdO + (32 * rb + l32) * C::KP + (D / 2) * half;
#pragma unroll
      for (int s = 0; s < C::DS; ++s) {
        sacc = mfma(as_bf16x8(lds16(qa + 8 * s)), kop[s], sacc);
        dpacc = mfma(as_bf16x8(lds16(oa + 8 * s)), vop[s], dpacc);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int rr = 32 * rb + 8 * jj + 4 * half;
        const float4 L4 = *reinterpret_cast<const float4*>(sL + rr);
        const float4 D4 = *reinterpret_cast<const float4*>(sD + rr);
        const float Lv[4] = {L4.x, L4.y, L4.z, L4.w}, Dv[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * jj + e;
          const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale2, -Lv[e]));
          sacc[r] = pv;
          dpacc[r] = pv * (dpacc[r] - Dv[e]);
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8 pa_hi, pa_lo, da_hi, da_lo;
        pack8_split(sacc, 8 * t, pa_hi, pa_lo);
        pack8_split(dpacc, 8 * t, da_hi, da_lo);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const bf16x8 dot_op = lds_rows_operand<D>(sdO, 32 * rb + 16 * t, 32 * db, lane);
          const bf16x8 qt_op = lds_rows_operand<D>(sQ, 32 * rb + 16 * t, 32 * db, lane);
          dvacc[db] = mfma(pa_hi, dot_op, dvacc[db]);
          dvacc[db] = mfma(pa_lo, dot_op, dvacc[db]);
          dkacc[db] = mfma(da_hi, qt_op, dkacc[db]);
          dkacc[db] = mfma(da_lo, qt_op, dkacc[db]);
        }
      }
    }
  }
  // fp32 outputs: accumulators hold [key = 8jj + 4half + e][d = 32db + l32]; 32 lanes store
  // 128 contiguous bytes of one key row per instruction
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 32 * w + 8 * (r >> 2) + 4 * half + (r & 3);
      const int64_t off = hoff + (int64_t)key * D + 32 * db + l32;
      dK[off] = dkacc[db][r] * sm_scale;
      dV[off] = dvacc[db][r];
    }
}

}  // namespace

prism_status launch_mfma_fwd(const Geom& g, const int32_t* bs, const int32_t* cnt, const int32_t* idx, float sm_scale,
                             const void* q, const void* k, const void* v, void* o, void* o_lo, float* lse,
                             hipStream_t st) {
  dim3 grid((unsigned)(g.N / 64), g.heads);
  const float scale2 = sm_scale * kLog2e;
  KernelTrace tr("k_fwd", st);
  if (g.d == 64)
    hipLaunchKernelGGL(k_fwd<64>, grid, dim3(128), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (uint16_t*)o, (uint16_t*)o_lo, lse, bs, cnt, idx, g.nbmax, g.hpg,
                       (int)g.N, scale2);
  else
    hipLaunchKernelGGL(k_fwd<128>, grid, dim3(128), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (uint16_t*)o, (uint16_t*)o_lo, lse, bs, cnt, idx, g.nbmax, g.hpg,
                       (int)g.N, scale2);
  return check_launch("k_fwd");
}

prism_status launch_mfma_bwd(const Geom& g, const int32_t* bs, const int32_t* cnt, const int32_t* idx, float sm_scale,
                             const void* q, const void* k, const void* v, const void* dout, const float* lse,
                             const float* delta, const uint32_t* mask_t, int nw, float* dq, float* dk, float* dv,
                             hipStream_t st) {
  dim3 grid((unsigned)(g.N / 64), g.heads);
  const float scale2 = sm_scale * kLog2e;
  {
    KernelTrace tr("k_dq", st);
    if (g.d == 64)
      hipLaunchKernelGGL(k_dq<64>, grid, dim3(128), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                         (const uint16_t*)v, (const uint16_t*)dout, lse, delta, dq, bs, cnt, idx, g.nbmax, g.hpg,
                         (int)g.N, scale2, sm_scale);
    else
      hipLaunchKernelGGL(k_dq<128>, grid, dim3(128), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                         (const uint16_t*)v, (const uint16_t*)dout, lse, delta, dq, bs, cnt, idx, g.nbmax, g.hpg,
                         (int)g.N, scale2, sm_scale);
  }
  prism_status s = check_launch("k_dq");
  if (s != PRISM_OK) return s;
  KernelTrace tr("k_dkdv", st);
  if (g.d == 64)
    hipLaunchKernelGGL(k_dkdv<64>, grid, dim3(128), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (const uint16_t*)dout, lse, delta, dk, dv, bs, mask_t, g.nbmax, nw,
                       g.hpg, (int)g.N, scale2, sm_scale);
  else
    hipLaunchKernelGGL(k_dkdv<128>, grid, dim3(128), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (const uint16_t*)dout, lse, delta, dk, dv, bs, mask_t, g.nbmax, nw,
                       g.hpg, (int)g.N, scale2, sm_scale);
  return check_launch("k_dkdv");
}

}  // namespace prism
