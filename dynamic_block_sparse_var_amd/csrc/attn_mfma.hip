// attn_mfma.hip -- bf16 block-sparse attention forward and backward on gfx950 matrix cores
// (RG M3: online-softmax attention solely across the selected key blocks S_i).
//
// Work decomposition.  Every block holds 64, 128 or 256 rows and starts on a multiple of 64,
// so the unit of work is a 64-row "atom" of one head.  A workgroup is two wave64s; each wave
// owns 32 rows of the atom.  Key (or query) tiles of 64 rows are staged in LDS once per
// workgroup and shared by both waves.  Atoms are assigned so that each of the 8 XCDs walks a
// contiguous range of atoms (neighbouring blocks tend to select the same key blocks, which
// then stay in that XCD's L2).
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16): operand A holds A[m = lane%32][8 k-values],
// operand B holds B[8 k-values][n = lane%32]; both use lane/32 to pick which half of the 16
// k-slots they hold.  The accumulator holds C[m = 8*jj + 4*(lane/32) + e][n = lane%32] in
// element 4*jj + e.  Reductions over the head dimension read 8 consecutive elements of a
// row-major tile (the k-slot -> d map just has to agree between A and B).  Reductions over
// keys or query rows read a transposed tile whose 64-wide rows store row index r at
// position tpos(r) (bits 2 and 3 swapped), which makes the 8 rows an accumulator lane holds
// for one k-step contiguous, so the accumulator itself is the next product's B (or A)
// operand after conversion to bf16.
//
// Forward:  S^T = K Q^T (A = K tile, B = Q rows kept in registers), online softmax per query
//           row (each lane owns one row, the other 32 keys of the tile sit in lane ^ 32),
//           O^T += V^T P^T (A = transposed V tile, B = P^T straight from the accumulator).
// dQ:       S^T = K Q^T, dP^T = V dO^T, dS^T = P^T * (dP^T - delta), dQ^T += K^T dS^T.
// dK, dV:   key-major: for every query block whose list contains the key block (transposed
//           selection bitmap), S = Q K^T, dP = dO V^T, P, dS, dV += P^T dO, dK += dS^T Q.
#include <math.h>

#include "attn_common.h"

namespace prism {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 8 accumulator elements [off, off + 8) -> bf16 operand (round to nearest even)
__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int off) {
  f32x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = x[off + i];
  return __builtin_convertvector(v, bf16x8);
}

// the same 8 elements as a bf16 head plus a bf16 residual: hi + lo carries ~16 significant bits
__device__ __forceinline__ void pack8_split(const f32x16& x, int off, bf16x8& hi, bf16x8& lo) {
  f32x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = x[off + i];
  hi = __builtin_convertvector(v, bf16x8);
  const f32x8 back = __builtin_convertvector(hi, f32x8);
  lo = __builtin_convertvector(v - back, bf16x8);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ int tpos(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Transposed tiles are 64 elements (128 bytes) wide.  The eight 16-byte granules of row d are
// stored XOR-swizzled by (d/8 + d) mod 8: the 8 rows a group of 8 lanes reads in one
// ds_read_b128 (consecutive d) then cover all 32 banks, and the writers (rows 8 apart) collide
// at most pairwise.  toff(d, p) = element offset of position p (p % 8 == 0 for reads).
__device__ __forceinline__ int toff(int d, int p) {
  return d * 64 + ((((p >> 3) ^ ((d >> 3) + d)) & 7) << 3) + (p & 7);
}

template <int D>
struct Cfg {
  static constexpr int KP = D + 8;          // row-major tile pitch, elements (2*D + 16 bytes)
  static constexpr int TP = 64;             // transposed tile pitch, elements (swizzled, see toff)
  static constexpr int CPR = D / 8;         // 16-byte chunks per row
  static constexpr int QPP = 128 / CPR;     // 4-row quads per pass of 128 threads
  static constexpr int NP = D / 64;         // passes per 64-row tile (16 quads)
  static constexpr int RPP = 128 / CPR;     // rows per pass (epilogue copy)
  static constexpr int DS = D / 16;         // k-steps over the head dimension
  static constexpr int DB = D / 32;         // 32-wide blocks of the head dimension
};

// global -> registers: thread t takes chunk t % CPR of rows 4q..4q+3 for quads q = t/CPR + QPP*it
template <int D>
__device__ __forceinline__ void gload_quads(const uint16_t* __restrict__ base, u32x4 (&r)[Cfg<D>::NP][4], int tid) {
  const int c = tid % Cfg<D>::CPR, q0 = tid / Cfg<D>::CPR;
#pragma unroll
  for (int it = 0; it < Cfg<D>::NP; ++it) {
    const int q = q0 + Cfg<D>::QPP * it;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r[it][e] = *reinterpret_cast<const u32x4*>(base + (int64_t)(4 * q + e) * D + 8 * c);
  }
}

template <int D>
__device__ __forceinline__ void lstore_rows(uint16_t* s, const u32x4 (&r)[Cfg<D>::NP][4], int tid) {
  const int c = tid % Cfg<D>::CPR, q0 = tid / Cfg<D>::CPR;
#pragma unroll
  for (int it = 0; it < Cfg<D>::NP; ++it) {
    const int q = q0 + Cfg<D>::QPP * it;
#pragma unroll
    for (int e = 0; e < 4; ++e) *reinterpret_cast<u32x4*>(s + (4 * q + e) * Cfg<D>::KP + 8 * c) = r[it][e];
  }
}

// transposed store: element i of the 4 rows of a quad -> 4 consecutive positions of row 8c+i
template <int D>
__device__ __forceinline__ void lstore_trans(uint16_t* s, const u32x4 (&r)[Cfg<D>::NP][4], int tid) {
  const int c = tid % Cfg<D>::CPR, q0 = tid / Cfg<D>::CPR;
#pragma unroll
  for (int it = 0; it < Cfg<D>::NP; ++it) {
    const int q = q0 + Cfg<D>::QPP * it;
    const int col = tpos(4 * q);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int wd = i >> 1;
      u32x2 out;
      if (i & 1) {
        out[0] = (r[it][0][wd] >> 16) | (r[it][1][wd] & 0xffff0000u);
        out[1] = (r[it][2][wd] >> 16) | (r[it][3][wd] & 0xffff0000u);
      } else {
        out[0] = (r[it][0][wd] & 0xffffu) | (r[it][1][wd] << 16);
        out[1] = (r[it][2][wd] & 0xffffu) | (r[it][3][wd] << 16);
      }
      *reinterpret_cast<u32x2*>(s + toff(8 * c + i, col)) = out;
    }
  }
}

__device__ __forceinline__ u32x4 lds16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// atoms of one head, spread so that each XCD (workgroup id mod 8) walks a contiguous range
__device__ __forceinline__ int xcd_atom(int bid, int natoms) {
  return ((natoms & 7) == 0) ? (bid & 7) * (natoms >> 3) + (bid >> 3) : bid;
}

// copy a staged 64 x D bf16 tile (pitch KP) to global rows
template <int D>
__device__ __forceinline__ void copy_out(uint16_t* __restrict__ dst, const uint16_t* s, int tid) {
  const int c = tid % Cfg<D>::CPR, r0 = tid / Cfg<D>::CPR;
#pragma unroll
  for (int it = 0; it < 64 / Cfg<D>::RPP; ++it) {
    const int r = r0 + Cfg<D>::RPP * it;
    *reinterpret_cast<u32x4*>(dst + (int64_t)r * D + 8 * c) = lds16(s + r * Cfg<D>::KP + 8 * c);
  }
}

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
  __shared__ __attribute__((aligned(16))) uint16_t sK[64 * C::KP];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * C::TP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const int h = blockIdx.y;
  const int natoms = N >> 6;
  const int row0 = xcd_atom(blockIdx.x, natoms) * 64;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  const int qb = block_of_row(bs, nbmax, row0);
  const int cnt = sel_count[(int64_t)h * nbmax + qb];
  const int32_t* list = sel_idx + ((int64_t)h * nbmax + qb) * nbmax;
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

  u32x4 kreg[C::NP][4], vreg[C::NP][4];
  int sidx = 0, kt = 0, kend = 0;
  if (cnt > 0) {
    const int j = list[0];
    kt = bs[j];
    kend = bs[j + 1];
    gload_quads<D>(Kh + (int64_t)kt * D, kreg, tid);
    gload_quads<D>(Vh + (int64_t)kt * D, vreg, tid);
  }
  while (sidx < cnt) {
    __syncthreads();
    lstore_rows<D>(sK, kreg, tid);
    lstore_trans<D>(sVt, vreg, tid);
    __syncthreads();
    int nkt = kt + 64, nsidx = sidx, nkend = kend;
    if (nkt >= kend) {
      ++nsidx;
      if (nsidx < cnt) {
        const int j = list[nsidx];
        nkt = bs[j];
        nkend = bs[j + 1];
      }
    }
    if (nsidx < cnt) {
      gload_quads<D>(Kh + (int64_t)nkt * D, kreg, tid);
      gload_quads<D>(Vh + (int64_t)nkt * D, vreg, tid);
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
    // online softmax (base 2, logits scaled by sm_scale * log2 e)
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(mrow, mx * scale2);
    const float alpha = __builtin_amdgcn_exp2f(mrow - mnew);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], scale2, -mnew));
        sacc[kb][r] = pv;
        psum += pv;
      }
    psum += __shfl_xor(psum, 32, 64);
    lrow = fmaf(lrow, alpha, psum);
    mrow = mnew;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
    // O^T += V^T P^T, with P as bf16 head + residual so O keeps fp32-level accuracy (the
    // backward's delta = dO . O cancels against dP and would expose bf16 rounding of P)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bf16x8 p_hi, p_lo;
      pack8_split(sacc[t >> 1], 8 * (t & 1), p_hi, p_lo);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const bf16x8 vt_op = as_bf16x8(lds16(sVt + toff(32 * db + l32, 16 * t + 8 * half)));
        oacc[db] = mfma(vt_op, p_hi, oacc[db]);
        oacc[db] = mfma(vt_op, p_lo, oacc[db]);
      }
    }
    kt = nkt;
    sidx = nsidx;
    kend = nkend;
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
  __shared__ __attribute__((aligned(16))) uint16_t sK[64 * C::KP];
  __shared__ __attribute__((aligned(16))) uint16_t sV[64 * C::KP];
  __shared__ __attribute__((aligned(16))) uint16_t sKt[D * C::TP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const int h = blockIdx.y;
  const int natoms = N >> 6;
  const int row0 = xcd_atom(blockIdx.x, natoms) * 64;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  const int qb = block_of_row(bs, nbmax, row0);
  const int cnt = sel_count[(int64_t)h * nbmax + qb];
  const int32_t* list = sel_idx + ((int64_t)h * nbmax + qb) * nbmax;
  const int64_t hoff = (int64_t)h * N * D;
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

  for (int sidx = 0; sidx < cnt; ++sidx) {
    const int j = list[sidx];
    for (int kt = bs[j]; kt < bs[j + 1]; kt += 64) {
      {
        u32x4 kreg[C::NP][4], vreg[C::NP][4];
        gload_quads<D>(K + hoff + (int64_t)kt * D, kreg, tid);
        gload_quads<D>(V + hoff + (int64_t)kt * D, vreg, tid);
        __syncthreads();
        lstore_rows<D>(sK, kreg, tid);
        lstore_trans<D>(sKt, kreg, tid);
        lstore_rows<D>(sV, vreg, tid);
        __syncthreads();
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
            const bf16x8 kt_op = as_bf16x8(lds16(sKt + toff(32 * db + l32, 16 * t + 8 * half)));
            dqacc[db] = mfma(kt_op, ds_hi, dqacc[db]);
            dqacc[db] = mfma(kt_op, ds_lo, dqacc[db]);
          }
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
  __shared__ __attribute__((aligned(16))) uint16_t sQ[64 * C::KP];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[64 * C::KP];
  __shared__ __attribute__((aligned(16))) uint16_t sQt[D * C::TP];
  __shared__ __attribute__((aligned(16))) uint16_t sdOt[D * C::TP];
  __shared__ __attribute__((aligned(16))) float sL[64];
  __shared__ __attribute__((aligned(16))) float sD[64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const int h = blockIdx.y;
  const int natoms = N >> 6;
  const int key0 = xcd_atom(blockIdx.x, natoms) * 64;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  const int kb_idx = block_of_row(bs, nbmax, key0);
  const uint32_t* mrow = mask_t + ((int64_t)h * nbmax + kb_idx) * nw;
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

  for (int wi = 0; wi < nw; ++wi) {
    uint32_t bits = mrow[wi];
    while (bits) {
      const int qbk = (wi << 5) + __ffs(bits) - 1;
      bits &= bits - 1;
      for (int rt = bs[qbk]; rt < bs[qbk + 1]; rt += 64) {
        {
          u32x4 qreg[C::NP][4], oreg[C::NP][4];
          gload_quads<D>(Q + hoff + (int64_t)rt * D, qreg, tid);
          gload_quads<D>(dO + hoff + (int64_t)rt * D, oreg, tid);
          float lv = 0.f, dv = 0.f;
          if (tid < 64) {
            lv = LSE[(int64_t)h * N + rt + tid] * kLog2e;
            dv = delta[(int64_t)h * N + rt + tid];
          }
          __syncthreads();
          lstore_rows<D>(sQ, qreg, tid);
          lstore_trans<D>(sQt, qreg, tid);
          lstore_rows<D>(sdO, oreg, tid);
          lstore_trans<D>(sdOt, oreg, tid);
          if (tid < 64) {
            sL[tid] = lv;
            sD[tid] = dv;
          }
          __syncthreads();
        }
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
              const int off = toff(32 * db + l32, 32 * rb + 16 * t + 8 * half);
              const bf16x8 dot_op = as_bf16x8(lds16(sdOt + off));
              const bf16x8 qt_op = as_bf16x8(lds16(sQt + off));
              dvacc[db] = mfma(pa_hi, dot_op, dvacc[db]);
              dvacc[db] = mfma(pa_lo, dot_op, dvacc[db]);
              dkacc[db] = mfma(da_hi, qt_op, dkacc[db]);
              dkacc[db] = mfma(da_lo, qt_op, dkacc[db]);
            }
          }
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
  if (g.d == 64) {
    hipLaunchKernelGGL(k_dq<64>, grid, dim3(128), 0, st, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                       (const uint16_t*)dout, lse, delta, dq, bs, cnt, idx, g.nbmax, g.hpg, (int)g.N,
                       scale2, sm_scale);
  } else {
    hipLaunchKernelGGL(k_dq<128>, grid, dim3(128), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (const uint16_t*)dout, lse, delta, dq, bs, cnt, idx, g.nbmax,
                       g.hpg, (int)g.N, scale2, sm_scale);
  }
  }
  prism_status s = check_launch("k_dq");
  if (s != PRISM_OK) return s;
  KernelTrace tr("k_dkdv", st);
  if (g.d == 64) {
    hipLaunchKernelGGL(k_dkdv<64>, grid, dim3(128), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (const uint16_t*)dout, lse, delta, dk, dv, bs,
                       mask_t, g.nbmax, nw, g.hpg, (int)g.N, scale2, sm_scale);
  } else {
    hipLaunchKernelGGL(k_dkdv<128>, grid, dim3(128), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (const uint16_t*)dout, lse, delta, dk, dv, bs,
                       mask_t, g.nbmax, nw, g.hpg, (int)g.N, scale2, sm_scale);
  }
  return check_launch("k_dkdv");
}

}  // namespace prism
