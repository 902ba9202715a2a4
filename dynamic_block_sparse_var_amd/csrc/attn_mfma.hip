// attn_mfma.hip -- bf16 block-sparse attention forward and backward on gfx950 matrix cores
// (RG M3: online-softmax attention solely across the selected key blocks S_i).
//
// Work decomposition.  Every block holds 64, 128 or 256 rows and starts on a multiple of 64,
// so the unit of work is a 64-row "atom" of one head: one workgroup of four wave64s per atom
// (dQ, dK/dV) or per pair of atoms of one zone (forward; the pair walks the union of its two
// lists, so a tile both selected is loaded once).  The other operand is streamed in 64-row
// tiles (the selected key blocks of a query atom, or the query blocks that selected a key
// atom), double-buffered in LDS: the direct global->LDS loads of tile i+1 are in flight while
// tile i is computed, one barrier per tile.  Within a tile, wave w takes 32 of the atom's rows
// (forward, dQ: query rows 32*(w&1)..; dK/dV: keys 32*(w&1)..) against 32 of the tile's rows
// (32*(w>>1)..), and the two waves that share the atom rows combine their partial results once
// at the end.  Atoms are assigned so that each of the 8 XCDs walks a contiguous range of atoms
// (neighbouring blocks tend to select the same key blocks, which may then still be in that
// XCD's L2); a launch order built by attn.hip moves the units with the longest walks to the
// front of that sequence, so that none of them starts near the end of the launch.
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
// Forward:  S^T = K Q^T (A = K tile, B = Q rows in registers or LDS), online softmax per query row
//           (a lane owns one row for 16 of the wave's 32 keys, lane ^ 32 the other 16; the
//           running max is only raised when a tile exceeds it by 2^16, so the O rescale is
//           rare), O^T += V^T P^T with P split into a bf16 head and residual.
// dQ:       S^T = K Q^T, dP^T = V dO^T, dS^T = P^T * (dP^T - delta), dQ^T += K^T dS^T.
// dK, dV:   key-major: for every query block whose list contains the key block (transposed
//           selection bitmap), S = Q K^T, dP = dO V^T, P, dS, dV += P^T dO, dK += dS^T Q.
// Products with P and dS use a bf16 head plus a bf16 residual of the fp32 value, so the
// results keep fp32-level accuracy.
#include <limits.h>
#include <math.h>

#include <type_traits>

#include "attn_common.h"

namespace prism {

namespace {

PRISM_DEVICE_SHAPES

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// log2 units the running max may lag behind: probabilities stay below 2^16 and row sums below
// 2^16 times the key count, far inside fp32 range
constexpr float kRescaleSlack = 16.f;

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

__device__ __forceinline__ u32x4 lds16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ u32x2 lds_tr(const uint16_t* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p)));
}

// ---- swizzled, unpadded 64 x D tiles filled by direct global -> LDS loads -----------------
// (layout, swizzle and addresses: index_math.h)

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

// Staging a 64-row tile: each of the 4 waves issues NI loads of 1 KB (global_load_lds_dwordx4,
// one 16-byte chunk per lane) from the byte offsets off[i] = dma_src_offset(w, lane, i).
// Completion is awaited with dma_wait() before the workgroup barrier.
template <int D>
__device__ __forceinline__ void dma_offsets(int w, int lane, uint32_t (&off)[Tile<D>::NI]) {
#pragma unroll
  for (int i = 0; i < Tile<D>::NI; ++i) off[i] = dma_src_offset<D>(w, lane, i);
}

template <int D>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ src, uint16_t* s, int w,
                                         const uint32_t (&off)[Tile<D>::NI]) {
  using TL = Tile<D>;
#pragma unroll
  for (int i = 0; i < TL::NI; ++i)
    __builtin_amdgcn_global_load_lds((gbl_void*)(reinterpret_cast<const char*>(src) + off[i]),
                                     (lds_void*)(reinterpret_cast<char*>(s) + (w * TL::NI + i) * 1024), 16, 0, 0);
}

__device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int D>
__device__ __forceinline__ void tr_addrs(int lane, uint32_t (&tr)[2]) {
  tr[0] = tr_addr<D>(lane, 0);
  tr[1] = tr_addr<D>(lane, 1);
}

__device__ __forceinline__ bf16x8 lds_b128(const uint16_t* s, uint32_t byte) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(s) + byte));
}


// Operands holding X[R0 + 8*(e/4) + 4*(lane/32) + e%4][32*db + lane%32], e = 0..7, of a
// swizzled tile X, for consecutive db starting at DB0 -- the lane's 8 k-slots when the product
// reduces over rows.  a[b] are the lane's absolute LDS addresses for the tile at smem byte 0,
// rows R0 = Rw and db = 0 (tr_table); column block db is reached by XOR-ing 64*db into the
// address, and OFF (an immediate) adds the tile's byte offset and 2*D*(R0 - Rw).  The reads are
// issued in one asm block that also waits for them: the compiler treats a transposing read as
// possibly aliasing the direct loads in flight into the other stage and would otherwise wait
// for those loads first.  Ordering against this stage's loads is given by dma_wait() and the
// barrier that precede every compute step.
template <int D>
__device__ __forceinline__ void tr_table(const uint16_t* smem, int lane, int Rw, uint32_t (&a)[2]) {
  uint32_t tr[2];
  tr_addrs<D>(lane, tr);
  const uint32_t sbase = (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) uint16_t*)smem);
#pragma unroll
  for (int b = 0; b < 2; ++b) a[b] = sbase + tr[b] + 2 * D * Rw;
}

__device__ __forceinline__ bf16x8 join_tr(u32x2 lo, u32x2 hi) {
  u32x4 v;
  v[0] = lo[0];
  v[1] = lo[1];
  v[2] = hi[0];
  v[3] = hi[1];
  return as_bf16x8(v);
}

template <int OFF, int DB0>
__device__ __forceinline__ void tr_ops(const uint32_t (&a)[2], bf16x8 (&op)[4]) {
  u32x2 r0, r1, r2, r3, r4, r5, r6, r7;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
      "ds_read_b64_tr_b16 %1, %9 offset:%16\n\t"
      "ds_read_b64_tr_b16 %2, %10 offset:%16\n\t"
      "ds_read_b64_tr_b16 %3, %11 offset:%16\n\t"
      "ds_read_b64_tr_b16 %4, %12 offset:%16\n\t"
      "ds_read_b64_tr_b16 %5, %13 offset:%16\n\t"
      "ds_read_b64_tr_b16 %6, %14 offset:%16\n\t"
      "ds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(a[0] ^ (64 * DB0)), "v"(a[1] ^ (64 * DB0)), "v"(a[0] ^ (64 * DB0 + 64)), "v"(a[1] ^ (64 * DB0 + 64)),
        "v"(a[0] ^ (64 * DB0 + 128)), "v"(a[1] ^ (64 * DB0 + 128)), "v"(a[0] ^ (64 * DB0 + 192)),
        "v"(a[1] ^ (64 * DB0 + 192)), "i"(OFF));
  op[0] = join_tr(r0, r1);
  op[1] = join_tr(r2, r3);
  op[2] = join_tr(r4, r5);
  op[3] = join_tr(r6, r7);
}

template <int OFF, int DB0>
__device__ __forceinline__ void tr_ops(const uint32_t (&a)[2], bf16x8 (&op)[2]) {
  u32x2 r0, r1, r2, r3;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%8\n\t"
      "ds_read_b64_tr_b16 %1, %5 offset:%8\n\t"
      "ds_read_b64_tr_b16 %2, %6 offset:%8\n\t"
      "ds_read_b64_tr_b16 %3, %7 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a[0] ^ (64 * DB0)), "v"(a[1] ^ (64 * DB0)), "v"(a[0] ^ (64 * DB0 + 64)), "v"(a[1] ^ (64 * DB0 + 64)),
        "i"(OFF));
  op[0] = join_tr(r0, r1);
  op[1] = join_tr(r2, r3);
}

// The tile walkers below fetch the bounds of up to 64 upcoming blocks at a time, one block per
// lane (vector loads), and take the current block's bounds from its lane with v_readlane, so
// walking a list costs no dependent memory round trip per block.

// Walks the 64-row tiles of the key blocks in a selection list (wave-uniform state).  The
// bounds of the next batch of 64 blocks, and the list entries of the batch after it, are
// loaded a batch ahead, so moving to a new batch waits for nothing.
struct ListTiles {
  const int32_t* list;
  const int32_t* bs;
  int cnt, base, k, kt, kend;
  int s_l, e_l;    // per lane: bounds of block list[base + lane]
  int ps_l, pe_l;  // per lane: bounds of block list[base + 64 + lane]
  int j_l;         // per lane: list[base + 128 + lane]
  __device__ int entry(int i) const { return (i < cnt) ? list[i] : 0; }
  __device__ void take() {
    kt = __builtin_amdgcn_readlane(s_l, k);
    kend = __builtin_amdgcn_readlane(e_l, k);
  }
  __device__ void begin(const int32_t* l, const int32_t* b, int c, int lane) {
    list = l;
    bs = b;
    cnt = c;
    base = k = 0;
    kt = kend = 0;
    if (cnt > 0) {
      const int j0 = entry(lane), j1 = entry(64 + lane);
      s_l = bs[j0];
      e_l = bs[j0 + 1];
      ps_l = bs[j1];
      pe_l = bs[j1 + 1];
      j_l = entry(128 + lane);
      take();
    }
  }
  __device__ bool valid() const { return base + k < cnt; }
  __device__ void next(int lane) {
    kt += 64;
    if (kt >= kend) {
      if (++k == 64) {
        base += 64;
        k = 0;
        if (base < cnt) {
          s_l = ps_l;
          e_l = pe_l;
          if (base + 64 < cnt) {
            ps_l = bs[j_l];
            pe_l = bs[j_l + 1];
            if (base + 128 < cnt) j_l = entry(base + 128 + lane);
          }
        }
      }
      if (base + k < cnt) take();
    }
  }
};

// Walks the 64-row tiles of the query blocks whose bit is set in a transposed-selection row
// (wave-uniform state).  64 words of the row are fetched at a time, one per lane, with a ballot
// of the non-zero ones, so finding the next set bit costs no memory round trip inside a batch
// and zero words are skipped at once.
struct MaskTiles {
  const uint32_t* mrow;
  const int32_t* bs;
  int nw, base, k, rt, rend;
  uint32_t bits;  // bits of word base + k not yet visited
  uint32_t w_l;   // per lane: word base + lane
  uint64_t nz;    // lanes whose word is non-zero
  __device__ void fetch(int lane) {
    const int i = base + lane;
    w_l = (i < nw) ? mrow[i] : 0u;
    nz = __ballot(w_l != 0u);
  }
  // moves to the first non-zero word among the lanes in rest, or past the row
  __device__ void seek(int lane, uint64_t rest) {
    while (rest == 0ull) {
      base += 64;
      if (base >= nw) return;
      fetch(lane);
      rest = nz;
    }
    k = __builtin_ctzll(rest);
    bits = __builtin_amdgcn_readlane(w_l, k);
  }
  __device__ void advance_block(int lane) {
    if (bits == 0u) {
      seek(lane, (k >= 63) ? 0ull : nz & (~0ull << (k + 1)));
      if (base >= nw) return;
    }
    const int bit = __builtin_ctz(bits);
    bits &= bits - 1;
    const int qb = ((base + k) << 5) + bit;
    PRISM_ASSERT(qb < nw * 32);
    rt = bs[qb];
    rend = bs[qb + 1];
  }
  __device__ void begin(const uint32_t* m, const int32_t* b, int n, int lane) {
    mrow = m;
    bs = b;
    nw = n;
    base = 0;
    k = -1;
    bits = 0u;
    rt = rend = 0;
    if (nw > 0) {
      fetch(lane);
      advance_block(lane);
    }
  }
  __device__ bool valid() const { return base < nw; }
  __device__ void next(int lane) {
    rt += 64;
    if (rt >= rend) advance_block(lane);
  }
};

// ------------------------------------------------------------------------------------------
// forward

// Walks the union of two selection lists (those of the two query atoms of a pair): the 64-row
// tiles of every key block in either list, in ascending order, each with the mask of the lists
// that hold it (bit 0: first, bit 1: second).  Both lists are read 64 entries at a time, one
// per lane, as ListTiles does; the merge itself is wave-uniform scalar work.
struct PairTiles {
  const int32_t* bs;
  const int32_t* la;
  const int32_t* lb;
  int ca, cb, basea, baseb, ka, kb;
  int kt, kend, mask;
  int sa_l, ea_l, sb_l, eb_l;  // per lane: bounds of blocks la[basea + lane], lb[baseb + lane]
  __device__ __forceinline__ void fetch_a(int lane) {
    const int i = basea + lane;
    const int j = (i < ca) ? la[i] : 0;
    sa_l = bs[j];
    ea_l = bs[j + 1];
  }
  __device__ __forceinline__ void fetch_b(int lane) {
    const int i = baseb + lane;
    const int j = (i < cb) ? lb[i] : 0;
    sb_l = bs[j];
    eb_l = bs[j + 1];
  }
  // the next block: the smaller head of the two lists (block rows ascend with the block index)
  __device__ __forceinline__ void pick() {
    const bool va = basea + ka < ca, vb = baseb + kb < cb;
    if (!va && !vb) {
      mask = 0;
      return;
    }
    const int sa = va ? __builtin_amdgcn_readlane(sa_l, ka) : INT_MAX;
    const int sb = vb ? __builtin_amdgcn_readlane(sb_l, kb) : INT_MAX;
    if (sa <= sb) {
      kt = sa;
      kend = __builtin_amdgcn_readlane(ea_l, ka);
    } else {
      kt = sb;
      kend = __builtin_amdgcn_readlane(eb_l, kb);
    }
    mask = (sa <= sb ? 1 : 0) | (sb <= sa ? 2 : 0);
  }
  __device__ __forceinline__ void begin(const int32_t* a, int na, const int32_t* b, int nb, const int32_t* bounds,
                                        int lane) {
    bs = bounds;
    la = a;
    lb = b;
    ca = na;
    cb = nb;
    basea = baseb = ka = kb = 0;
    kt = kend = 0;
    if (ca > 0) fetch_a(lane);
    if (cb > 0) fetch_b(lane);
    pick();
  }
  __device__ __forceinline__ bool valid() const { return mask != 0; }
  __device__ __forceinline__ void next(int lane) {
    kt += 64;
    if (kt < kend) return;
    if (mask & 1) {
      if (++ka == 64) {
        basea += 64;
        ka = 0;
        if (basea < ca) fetch_a(lane);
      }
    }
    if (mask & 2) {
      if (++kb == 64) {
        baseb += 64;
        kb = 0;
        if (baseb < cb) fetch_b(lane);
      }
    }
    pick();
  }
};

// The first rows of the two atoms of pair p (zone m = p / 4, slot s = p % 4).  In a zone of
// 128- or 256-row blocks the pair is atoms 2s and 2s + 1 of the zone, which lie in one block
// and share its list.  In a zone of eight 64-row blocks the blocks are matched greedily by the
// size of the intersection of their lists (largest first; among equal sizes the pair (a, c),
// a < c, that comes first in lexicographic order), counted on LDS bitmaps; slot s takes the
// s-th pair chosen.  The matching depends only on the lists, so the zone's four workgroups
// agree on it and every atom is in exactly one pair.  scratch: 8 * ceil(nbmax / 32) + 32 words
// of LDS, free again when this returns.
__device__ __forceinline__ void pair_atoms(const int32_t* bs, int nbmax, const int32_t* cnt_h, const int32_t* idx_h,
                                           int p, uint32_t* scratch, int& rowA, int& rowB) {
  const int tid = threadIdx.x;
  const int m = p >> 2, s = p & 3;
  const int j0 = block_of_row(bs, nbmax, 512 * m);
  if (bs[j0 + 1] - bs[j0] > 64) {
    rowA = 512 * m + 128 * s;
    rowB = rowA + 64;
    return;
  }
  const int nw = (nbmax + 31) >> 5;
  uint32_t* bm = scratch;
  int* inter = reinterpret_cast<int*>(scratch + 8 * nw);
  for (int i = tid; i < 8 * nw; i += blockDim.x) bm[i] = 0u;
  __syncthreads();
  for (int q = 0; q < 8; ++q) {
    const int c = cnt_h[j0 + q];
    const int32_t* l = idx_h + (int64_t)(j0 + q) * nbmax;
    for (int i = tid; i < c; i += blockDim.x) {
      const int j = l[i];
      atomicOr(&bm[q * nw + (j >> 5)], 1u << (j & 31));
    }
  }
  __syncthreads();
  // 28 block pairs x 8 threads: popcounts of the AND of two bitmaps
  {
    const int pi = tid >> 3, sub = tid & 7;
    int a = 0, n = pi;
    while (a < 7 && n >= 7 - a) {
      n -= 7 - a;
      ++a;
    }
    const int c = a + 1 + n;
    int cnt = 0;
    if (pi < 28)
      for (int wd = sub; wd < nw; wd += 8) cnt += __popc(bm[a * nw + wd] & bm[c * nw + wd]);
#pragma unroll
    for (int o = 4; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 8);
    if (pi < 28 && sub == 0) inter[pi] = cnt;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t used = 0u;
    int ra = 0, rc = 1;
    for (int k = 0; k <= s; ++k) {
      int best = -1, n = 0;
      for (int a2 = 0; a2 < 8; ++a2)
        for (int c2 = a2 + 1; c2 < 8; ++c2, ++n)
          if (!((used >> a2) & 1u) && !((used >> c2) & 1u) && inter[n] > best) {
            best = inter[n];
            ra = a2;
            rc = c2;
          }
      used |= (1u << ra) | (1u << rc);
    }
    inter[28] = bs[j0 + ra];
    inter[29] = bs[j0 + rc];
  }
  __syncthreads();
  rowA = __builtin_amdgcn_readfirstlane(inter[28]);
  rowB = __builtin_amdgcn_readfirstlane(inter[29]);
  __syncthreads();
}

// Forward over a pair of atoms of one zone (pair_atoms) walking the union of their lists, so a
// key tile both atoms selected is loaded once.  Workgroup = 4 waves; wave w owns rows 32*(w&1)..
// of both atoms and keys 32*(w>>1).. of every staged tile, and computes each tile for each atom
// that selected it, so every wave has work on every tile.  The first atom's Q rows are held in
// registers, the second's are staged once in LDS (80 KB per workgroup with the two K/V stages:
// two workgroups per CU).  The two waves sharing a row half keep separate online-softmax states
// per atom, merged once at the end.
template <int D>
__global__ __launch_bounds__(256, 2) void k_fwd(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                                                uint16_t* __restrict__ Olo, float* __restrict__ LSE,
                                                const int32_t* __restrict__ block_start,
                                                const int32_t* __restrict__ sel_count,
                                                const int32_t* __restrict__ sel_idx,
                                                const int32_t* __restrict__ order, int nbmax, int hpg, int N,
                                                float scale2, RowMap rm) {
  constexpr int T = 64 * D;
  constexpr int DS = D / 16, DB = D / 32, CH = D / 16;
  constexpr uint32_t SB = 4 * T;  // bytes of one stage (K tile, V tile)
  // two stages, then the second atom's Q rows
  __shared__ __attribute__((aligned(1024))) uint16_t smem[5 * T];
  const uint16_t* sQB = smem + 4 * T;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rh = w & 1, kh = w >> 1;
  // this workgroup's (head, pair): from the launch order if one is given, else head blockIdx.y
  // and the pairs of a head in xcd_atom order
  const int npairs = N >> 7;
  int h, pidx;
  if (order) {
    const int item = order[blockIdx.y * gridDim.x + blockIdx.x];
    h = item / npairs;
    pidx = item - h * npairs;
  } else {
    h = blockIdx.y;
    pidx = xcd_atom(blockIdx.x, npairs);
  }
  h = __builtin_amdgcn_readfirstlane(h);
  pidx = __builtin_amdgcn_readfirstlane(pidx);
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  int rowA, rowB;
  pair_atoms(bs, nbmax, sel_count + (int64_t)h * nbmax, sel_idx + (int64_t)h * nbmax * nbmax, pidx,
             reinterpret_cast<uint32_t*>(smem), rowA, rowB);
  PRISM_ASSERT(rowA >= 0 && rowB >= 0 && rowA + 64 <= N && rowB + 64 <= N && !(rowA & 63) && !(rowB & 63));
  const int qa = block_of_row(bs, nbmax, rowA), qb = block_of_row(bs, nbmax, rowB);
  const int64_t hoff = (int64_t)h * N * D;
  const uint16_t* Kh = K + hoff;
  const uint16_t* Vh = V + hoff;
  const int myrow = rowA + 32 * rh + l32;  // this lane's row of the first atom

  uint32_t doff[Tile<D>::NI], tav[2];
  dma_offsets<D>(w, lane, doff);
  dma_tile<D>(Q + hoff + (int64_t)rowB * D, smem + 4 * T, w, doff);
  bf16x8 qop[DS];
  {
    const uint16_t* qr = Q + hoff + (int64_t)myrow * D + (D / 2) * half;
#pragma unroll
    for (int s = 0; s < DS; ++s) qop[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qr + 8 * s));
  }
  f32x16 oa[DB], ob[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    oa[db] = zero16();
    ob[db] = zero16();
  }
  float ma = -INFINITY, la = 0.f, mb = -INFINITY, lb = 0.f;

  PairTiles it;
  {
    const int64_t ra = (int64_t)h * nbmax + qa, rb = (int64_t)h * nbmax + qb;
    it.begin(sel_idx + ra * nbmax, sel_count[ra], sel_idx + rb * nbmax, sel_count[rb], bs, lane);
  }
  tr_table<D>(smem, lane, 32 * kh, tav);
  // per-lane read addresses of the stage being computed (moved to the other stage per tile)
  uint32_t rowa = row_addr<D>(32 * kh + l32) ^ ((CH * half) << 4);
  const uint32_t rowq = row_addr<D>(32 * rh + l32) ^ ((CH * half) << 4);
  auto stage = [&](uint32_t soff) __attribute__((always_inline)) {
    PRISM_ASSERT(it.kt >= 0 && it.kt + 64 <= N);
    uint16_t* s = smem + soff / 2;
    dma_tile<D>(Kh + (int64_t)it.kt * D, s, w, doff);
    dma_tile<D>(Vh + (int64_t)it.kt * D, s + T, w, doff);
  };
  // one atom's rows against the wave's 32 keys of the staged tile; FROM_LDS: Q rows from sQB
  auto compute = [&](auto fromc, f32x16(&oacc)[DB], float& mrow, float& lrow) __attribute__((always_inline)) {
    constexpr bool FROM_LDS = decltype(fromc)::value;
    const uint16_t* sK = smem;
    f32x16 sacc = zero16();
    // K operands four at a time, so one LDS wait covers four products
#pragma unroll
    for (int b = 0; b < DS; b += 4) {
      bf16x8 ka[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) ka[st] = lds_b128(sK, rowa ^ ((b + st) << 4));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8 qv = FROM_LDS ? lds_b128(sQB, rowq ^ ((b + st) << 4)) : qop[b + st];
        sacc = mfma(ka[st], qv, sacc);
      }
    }
    float mx = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx *= scale2;
    if (__any(mx > mrow + kRescaleSlack)) {
      const float mnew = fmaxf(mrow, fmaxf(mx, __shfl_xor(mx, 32, 64)));
      const float alpha = __builtin_amdgcn_exp2f(mrow - mnew);
      lrow *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      mrow = mnew;
    }
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale2, -mrow));
      sacc[r] = pv;
      psum += pv;
    }
    lrow += psum;
    auto pv = [&](auto ttc) __attribute__((always_inline)) {
      constexpr int tt = decltype(ttc)::value;
      bf16x8 p_hi, p_lo, vt[DB];
      pack8_split(sacc, 8 * tt, p_hi, p_lo);
      tr_ops<2 * T + 32 * D * tt, 0>(tav, vt);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        oacc[db] = mfma(vt[db], p_hi, oacc[db]);
        oacc[db] = mfma(vt[db], p_lo, oacc[db]);
      }
    };
    __builtin_amdgcn_s_setprio(1);
    pv(std::integral_constant<int, 0>{});
    pv(std::integral_constant<int, 1>{});
    __builtin_amdgcn_s_setprio(0);
  };
  if (it.valid()) {
    uint32_t soff = 0;
    stage(0);
    while (true) {
      dma_wait();
      __syncthreads();
      const int cur = it.mask;
      it.next(lane);
      const bool more = it.valid();
      if (more) stage(soff ^ SB);
      if (cur & 1) compute(std::false_type{}, oa, ma, la);
      if (cur & 2) compute(std::true_type{}, ob, mb, lb);
      if (!more) break;
      soff ^= SB;
      rowa ^= SB;
      const uint32_t step = soff ? SB : (uint32_t)(-(int32_t)SB);
      tav[0] += step;
      tav[1] += step;
    }
  } else {
    dma_wait();
  }
  la += __shfl_xor(la, 32, 64);
  lb += __shfl_xor(lb, 32, 64);
  // merge the key halves of both atoms: the kh = 1 wave of each row half hands (O, m, l) over
  // through LDS
  __syncthreads();
  float* xo = reinterpret_cast<float*>(smem);                 // [atom][rh][DB * 16][64 lanes]
  float* xm = reinterpret_cast<float*>(smem) + 4 * DB * 16 * 64;  // [atom][rh][m | l][32 rows]
  if (kh == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        xo[(((0 * 2 + rh) * DB + db) * 16 + r) * 64 + lane] = oa[db][r];
        xo[(((1 * 2 + rh) * DB + db) * 16 + r) * 64 + lane] = ob[db][r];
      }
    if (half == 0) {
      xm[(0 * 2 + rh) * 64 + l32] = ma;
      xm[(0 * 2 + rh) * 64 + 32 + l32] = la;
      xm[(1 * 2 + rh) * 64 + l32] = mb;
      xm[(1 * 2 + rh) * 64 + 32 + l32] = lb;
    }
  }
  __syncthreads();
  if (kh == 0) {
    auto finish = [&](int at, const f32x16(&oacc)[DB], float mrow, float lrow) __attribute__((always_inline)) {
      const int row = (at ? rowB : rowA) + 32 * rh + l32;
      const float m1 = xm[(at * 2 + rh) * 64 + l32], l1 = xm[(at * 2 + rh) * 64 + 32 + l32];
      const float m = fmaxf(mrow, m1);
      const float a0 = (mrow == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mrow - m);
      const float a1 = (m1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
      const float l = lrow * a0 + l1 * a1;
      const float inv = (l > 0.f) ? 1.f / l : 0.f;
      if (half == 0) LSE[(int64_t)h * N + row] = (l > 0.f) ? (m + log2f(l)) * kLn2 : -INFINITY;
      const int64_t orw = out_row(rm, c_shapes, h / hpg, h, gridDim.y, N, row) * D + 4 * half;
      uint16_t* orow = O + orw;
      uint16_t* rrow = Olo ? Olo + orw : nullptr;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float ov[4], rv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * jj + e;
            ov[e] = (oacc[db][r] * a0 + xo[(((at * 2 + rh) * DB + db) * 16 + r) * 64 + lane] * a1) * inv;
            rv[e] = ov[e] - bf16_to_f32(f32_to_bf16(ov[e]));
          }
          u32x2 pk;
          pk[0] = pack_bf16x2(ov[0], ov[1]);
          pk[1] = pack_bf16x2(ov[2], ov[3]);
          *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * jj) = pk;
          if (rrow) {
            pk[0] = pack_bf16x2(rv[0], rv[1]);
            pk[1] = pack_bf16x2(rv[2], rv[3]);
            *reinterpret_cast<u32x2*>(rrow + 32 * db + 8 * jj) = pk;
          }
        }
    };
    finish(0, oa, ma, la);
    finish(1, ob, mb, lb);
  }
}

// ------------------------------------------------------------------------------------------
// backward, query-major: dQ

// Same decomposition as the forward: wave w owns query rows 32*(w&1).. and keys 32*(w>>1).. of
// every tile; the two partial dQ of a row half are summed at the end.
template <int D>
__global__ __launch_bounds__(256, 2) void k_dq(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                               const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                                               const float* __restrict__ LSE2, const float* __restrict__ delta,
                                               float* __restrict__ dQ, const int32_t* __restrict__ block_start,
                                               const int32_t* __restrict__ sel_count,
                                               const int32_t* __restrict__ sel_idx,
                                               const int32_t* __restrict__ order, int nbmax, int hpg, int N,
                                               float scale2, float sm_scale, RowMap rm) {
  constexpr int T = 64 * D;
  constexpr int DS = D / 16, DB = D / 32, CH = D / 16;
  constexpr uint32_t SB = 4 * T;  // bytes of one stage (K tile, V tile)
  __shared__ __attribute__((aligned(1024))) uint16_t smem[4 * T];  // two stages
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rh = w & 1, kh = w >> 1;
  // this workgroup's item of the launch order: (head, atom) = divmod(item, natoms)
  const int natoms = N >> 6;
  const int item = order[blockIdx.y * gridDim.x + blockIdx.x];
  const int h = item / natoms;
  const int row0 = (item - h * natoms) * 64;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  PRISM_ASSERT(h < gridDim.y && row0 >= 0 && row0 + 64 <= N);
  const int qb = block_of_row(bs, nbmax, row0);
  const int64_t hoff = (int64_t)h * N * D;
  const uint16_t* Kh = K + hoff;
  const uint16_t* Vh = V + hoff;
  const int myrow = row0 + 32 * rh + l32;

  bf16x8 qop[DS], doop[DS];
  {
    const uint16_t* qr = Q + hoff + (int64_t)myrow * D + (D / 2) * half;
    const uint16_t* dr = dO + hoff + (int64_t)myrow * D + (D / 2) * half;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      qop[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qr + 8 * s));
      doop[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(dr + 8 * s));
    }
  }
  const float lse2 = LSE2[(int64_t)h * N + myrow];
  const float dl = delta[(int64_t)h * N + myrow];
  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqacc[db] = zero16();

  ListTiles it;
  it.begin(sel_idx + ((int64_t)h * nbmax + qb) * nbmax, bs, sel_count[(int64_t)h * nbmax + qb], lane);
  uint32_t doff[Tile<D>::NI], tak[2];
  dma_offsets<D>(w, lane, doff);
  tr_table<D>(smem, lane, 32 * kh, tak);
  // per-lane read addresses of the stage being computed (moved to the other stage per tile)
  uint32_t rowa = row_addr<D>(32 * kh + l32) ^ ((CH * half) << 4);
  auto stage = [&](uint32_t soff) __attribute__((always_inline)) {
    PRISM_ASSERT(it.kt >= 0 && it.kt + 64 <= N);
    uint16_t* s = smem + soff / 2;
    dma_tile<D>(Kh + (int64_t)it.kt * D, s, w, doff);
    dma_tile<D>(Vh + (int64_t)it.kt * D, s + T, w, doff);
  };
  auto compute = [&]() __attribute__((always_inline)) {
    const uint16_t* sK = smem;
    const uint16_t* sV = smem + T;
    // S^T = K Q^T, dP^T = V dO^T for this wave's 32 keys x 32 rows
    f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
    for (int st = 0; st < DS; ++st) {
      sacc = mfma(lds_b128(sK, rowa ^ (st << 4)), qop[st], sacc);
      dpacc = mfma(lds_b128(sV, rowa ^ (st << 4)), doop[st], dpacc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale2, -lse2));
      sacc[r] = pv * (dpacc[r] - dl);
    }
    // dQ^T += K^T dS^T, dS as bf16 head + residual
    auto dsk = [&](auto ttc) __attribute__((always_inline)) {
      constexpr int tt = decltype(ttc)::value;
      bf16x8 ds_hi, ds_lo, kt[DB];
      pack8_split(sacc, 8 * tt, ds_hi, ds_lo);
      tr_ops<32 * D * tt, 0>(tak, kt);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dqacc[db] = mfma(kt[db], ds_hi, dqacc[db]);
        dqacc[db] = mfma(kt[db], ds_lo, dqacc[db]);
      }
    };
    dsk(std::integral_constant<int, 0>{});
    dsk(std::integral_constant<int, 1>{});
  };
  if (it.valid()) {
    uint32_t soff = 0;
    stage(0);
    while (true) {
      dma_wait();
      __syncthreads();
      it.next(lane);
      const bool more = it.valid();
      if (more) stage(soff ^ SB);
      compute();
      if (!more) break;
      soff ^= SB;
      rowa ^= SB;
      const uint32_t step = soff ? SB : (uint32_t)(-(int32_t)SB);
      tak[0] += step;
      tak[1] += step;
    }
  }
  // sum the key halves: the kh = 1 wave of each row half hands its partial over through LDS
  __syncthreads();
  float* xo = reinterpret_cast<float*>(smem);  // [rh][DB * 16][64 lanes]
  if (kh == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[((rh * DB + db) * 16 + r) * 64 + lane] = dqacc[db][r];
  }
  __syncthreads();
  if (kh == 0) {
    // the lane holds dQ[myrow][32db + 8jj + 4half + e].  The wave's 32 x D block goes out as whole
    // rows (32 lanes x 16 bytes per row and store): it is staged in the wave's own LDS region
    // (read out above first), 16-byte chunk c of row r at chunk slot c ^ (r % CPR)
    constexpr int CPR = D / 4;  // 16-byte chunks per fp32 row
    float* xs = xo + rh * DB * 16 * 64;
    float acc[DB][16];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = (dqacc[db][r] + xs[(db * 16 + r) * 64 + lane]) * sm_scale;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // every lane's partner values are read
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int c = 8 * db + 2 * jj + half;
        *reinterpret_cast<float4*>(xs + l32 * D + 4 * (c ^ (l32 & (CPR - 1)))) =
            make_float4(acc[db][4 * jj], acc[db][4 * jj + 1], acc[db][4 * jj + 2], acc[db][4 * jj + 3]);
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    constexpr int RPI = 64 / CPR;  // rows per store instruction
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = RPI * i + lane / CPR, c = lane % CPR;
      const float4 x = *reinterpret_cast<const float4*>(xs + r * D + 4 * (c ^ (r & (CPR - 1))));
      const int row = row0 + 32 * rh + r;
      *reinterpret_cast<float4*>(dQ + out_row(rm, c_shapes, h / hpg, h, gridDim.y, N, row) * D + 4 * c) = x;
    }
  }
}

// ------------------------------------------------------------------------------------------
// backward, key-major: dK, dV

// Workgroup = 4 waves on one 64-key atom.  Wave w owns keys 32*(w&1).. of the atom and, of every
// staged 64-row query tile (the tiles of the query blocks whose lists hold this key block), query
// rows 32*(w>>1)..; the two partial dK, dV of a key half are summed at the end.  A stage holds
// the Q and dO tiles plus the tile's lse2 and delta rows.
template <int D>
__global__ __launch_bounds__(256, 2) void k_dkdv(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                 const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                                                 const float* __restrict__ LSE2, const float* __restrict__ delta,
                                                 float* __restrict__ dK, float* __restrict__ dV,
                                                 const int32_t* __restrict__ block_start,
                                                 const uint32_t* __restrict__ mask_t,
                                                 const int32_t* __restrict__ order, int nbmax, int nw, int hpg,
                                                 int N, float scale2, float sm_scale, RowMap rm) {
  constexpr int T = 64 * D;
  constexpr int DS = D / 16, DB = D / 32, CH = D / 16;
  constexpr uint32_t SB = 4 * T;  // bytes of one stage's tiles (Q, dO)
  // two stages of (Q, dO) tiles, then [stage][lse2 | delta][256] floats
  __shared__ __attribute__((aligned(1024))) uint16_t smem[4 * T + 2048];
  float* sld = reinterpret_cast<float*>(smem + 4 * T);
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = w & 1, qh = w >> 1;
  // this workgroup's item of the launch order: (head, key atom) = divmod(item, natoms)
  const int natoms = N >> 6;
  const int item = order[blockIdx.y * gridDim.x + blockIdx.x];
  const int h = item / natoms;
  const int key0 = (item - h * natoms) * 64;
  const int32_t* bs = block_start + (int64_t)(h / hpg) * (nbmax + 1);
  PRISM_ASSERT(h < gridDim.y && key0 >= 0 && key0 + 64 <= N);
  const int kb_idx = block_of_row(bs, nbmax, key0);
  const int64_t hoff = (int64_t)h * N * D;
  const int mykey = key0 + 32 * kh + l32;

  bf16x8 kop[DS], vop[DS];
  {
    const uint16_t* kr = K + hoff + (int64_t)mykey * D + (D / 2) * half;
    const uint16_t* vr = V + hoff + (int64_t)mykey * D + (D / 2) * half;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      kop[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(kr + 8 * s));
      vop[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(vr + 8 * s));
    }
  }
  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dkacc[db] = zero16();
    dvacc[db] = zero16();
  }

  MaskTiles it;
  it.begin(mask_t + ((int64_t)h * nbmax + kb_idx) * nw, bs, nw, lane);
  uint32_t taq[2];
  tr_table<D>(smem, lane, 32 * qh, taq);
  // per-lane read addresses of the stage being computed (moved to the other stage per tile)
  uint32_t rowa = row_addr<D>(32 * qh + l32) ^ ((CH * half) << 4);
  // byte address of lse2[32qh + 4half] in the stage's row-statistics block (delta at +256)
  uint32_t lda = 2 * SB + 4 * (32 * qh + 4 * half);  // lse2 rows; delta at +1024 bytes
  const float* L2h = LSE2 + (int64_t)h * N;
  const float* Dh = delta + (int64_t)h * N;
  // lse2 (wave 0) and delta (wave 1) of a tile's 64 rows: one 1 KB direct load each, lanes
  // 0-15 fetching the 256 bytes (the other lanes repeat them)
  const float* ldsrc = (w == 0) ? L2h : Dh;
  auto stage = [&](uint32_t soff, int stg) __attribute__((always_inline)) {
    // the load offsets are recomputed here rather than kept live through the loop: this
    // kernel is at its register limit, and a spill reload inside the loop would make the
    // compiler wait for the loads just issued
    int ln = lane;
    asm volatile("" : "+v"(ln));
    uint32_t doff[Tile<D>::NI];
    dma_offsets<D>(w, ln, doff);
    PRISM_ASSERT(it.rt >= 0 && it.rt + 64 <= N);
    uint16_t* s = smem + soff / 2;
    if (w < 2)
      __builtin_amdgcn_global_load_lds((gbl_void*)(ldsrc + it.rt + 4 * (ln & 15)),
                                       (lds_void*)(sld + 512 * stg + 256 * w), 16, 0, 0);
    dma_tile<D>(Q + hoff + (int64_t)it.rt * D, s, w, doff);
    dma_tile<D>(dO + hoff + (int64_t)it.rt * D, s + T, w, doff);
  };
  auto compute = [&]() __attribute__((always_inline)) {
    const uint16_t* sQ = smem;
    const uint16_t* sdO = smem + T;

    // S = Q K^T and dP = dO V^T for this wave's 32 query rows x 32 keys
    f32x16 sacc = zero16(), dpacc = zero16();
    // operands two steps at a time, so one LDS wait covers four products (more would spill)
#pragma unroll
    for (int b = 0; b < DS; b += 2) {
      bf16x8 qa[2], da[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        qa[st] = lds_b128(sQ, rowa ^ ((b + st) << 4));
        da[st] = lds_b128(sdO, rowa ^ ((b + st) << 4));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        sacc = mfma(qa[st], kop[b + st], sacc);
        dpacc = mfma(da[st], vop[b + st], dpacc);
      }
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const u32x4 L4 = __builtin_bit_cast(u32x4, lds_b128(smem, lda + 32 * jj));
      const u32x4 D4 = __builtin_bit_cast(u32x4, lds_b128(smem, lda + 1024 + 32 * jj));
      const float Lv[4] = {__uint_as_float(L4[0]), __uint_as_float(L4[1]), __uint_as_float(L4[2]),
                           __uint_as_float(L4[3])};
      const float Dv[4] = {__uint_as_float(D4[0]), __uint_as_float(D4[1]), __uint_as_float(D4[2]),
                           __uint_as_float(D4[3])};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * jj + e;
        const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale2, -Lv[e]));
        sacc[r] = pv;
        dpacc[r] = pv * (dpacc[r] - Dv[e]);
      }
    }
    // dV += P^T dO, then dK += dS^T Q (P and dS as bf16 head + residual); the phases are kept
    // apart so that only one split operand set is live at a time
    __builtin_amdgcn_sched_barrier(0);
    // the dV and dK products run at raised wave priority (as the forward's PV; measured: -1.5 %)
    __builtin_amdgcn_s_setprio(1);
    auto pdo = [&](auto tc) __attribute__((always_inline)) {
      constexpr int t = decltype(tc)::value;
      bf16x8 pa_hi, pa_lo, dot[2];
      pack8_split(sacc, 8 * t, pa_hi, pa_lo);
      auto half_db = [&](auto dpc) __attribute__((always_inline)) {
        constexpr int dp = decltype(dpc)::value;
        tr_ops<2 * T + 32 * D * t, 2 * dp>(taq, dot);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          dvacc[2 * dp + j] = mfma(pa_hi, dot[j], dvacc[2 * dp + j]);
          dvacc[2 * dp + j] = mfma(pa_lo, dot[j], dvacc[2 * dp + j]);
        }
      };
      half_db(std::integral_constant<int, 0>{});
      if constexpr (DB == 4) half_db(std::integral_constant<int, 1>{});
    };
    pdo(std::integral_constant<int, 0>{});
    pdo(std::integral_constant<int, 1>{});
    __builtin_amdgcn_sched_barrier(0);
    auto dsq = [&](auto tc) __attribute__((always_inline)) {
      constexpr int t = decltype(tc)::value;
      bf16x8 da_hi, da_lo, qt[2];
      pack8_split(dpacc, 8 * t, da_hi, da_lo);
      auto half_db = [&](auto dpc) __attribute__((always_inline)) {
        constexpr int dp = decltype(dpc)::value;
        tr_ops<32 * D * t, 2 * dp>(taq, qt);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          dkacc[2 * dp + j] = mfma(da_hi, qt[j], dkacc[2 * dp + j]);
          dkacc[2 * dp + j] = mfma(da_lo, qt[j], dkacc[2 * dp + j]);
        }
      };
      half_db(std::integral_constant<int, 0>{});
      if constexpr (DB == 4) half_db(std::integral_constant<int, 1>{});
    };
    dsq(std::integral_constant<int, 0>{});
    dsq(std::integral_constant<int, 1>{});
    __builtin_amdgcn_s_setprio(0);
  };
  if (it.valid()) {
    uint32_t soff = 0;
    int stg = 0;
    stage(0, 0);
    while (true) {
      dma_wait();
      __syncthreads();
      it.next(lane);
      const bool more = it.valid();
      if (more) stage(soff ^ SB, stg ^ 1);
      compute();
      if (!more) break;
      soff ^= SB;
      stg ^= 1;
      rowa ^= SB;
      const uint32_t step = soff ? SB : (uint32_t)(-(int32_t)SB);
      taq[0] += step;
      taq[1] += step;
      lda ^= 2048;
    }
  }
  // sum the query halves: the qh = 1 wave of each key half hands its partials over through LDS
  __syncthreads();
  float* xo = reinterpret_cast<float*>(smem);  // [kh][dK | dV][DB * 16][64 lanes]
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        xo[(((2 * kh + 0) * DB + db) * 16 + r) * 64 + lane] = dkacc[db][r];
        xo[(((2 * kh + 1) * DB + db) * 16 + r) * 64 + lane] = dvacc[db][r];
      }
  }
  __syncthreads();
  if (qh == 0) {
    // fp32 outputs: accumulators hold [key = 8jj + 4half + e][d = 32db + l32]; 32 lanes store
    // 128 contiguous bytes of one key row per instruction; block or token order
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 32 * kh + 8 * (r >> 2) + 4 * half + (r & 3);
      const int64_t krow = out_row(rm, c_shapes, h / hpg, h, gridDim.y, N, key) * D + l32;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int64_t off = krow + 32 * db;
        dK[off] = (dkacc[db][r] + xo[(((2 * kh + 0) * DB + db) * 16 + r) * 64 + lane]) * sm_scale;
        dV[off] = dvacc[db][r] + xo[(((2 * kh + 1) * DB + db) * 16 + r) * 64 + lane];
      }
    }
  }
}

}  // namespace

prism_status launch_mfma_fwd(const Geom& g, const int32_t* bs, const int32_t* cnt, const int32_t* idx, float sm_scale,
                             const void* q, const void* k, const void* v, void* o, void* o_lo, float* lse,
                             const int32_t* order, const RowMap& out, hipStream_t st) {
  dim3 grid((unsigned)(g.N / 128), g.heads);  // one workgroup per pair of atoms
  const float scale2 = sm_scale * kLog2e;
  KernelTrace tr("k_fwd", st);
  if (g.d == 64)
    hipLaunchKernelGGL(k_fwd<64>, grid, dim3(256), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (uint16_t*)o, (uint16_t*)o_lo, lse, bs, cnt, idx, order, g.nbmax,
                       g.hpg, (int)g.N, scale2, out);
  else
    hipLaunchKernelGGL(k_fwd<128>, grid, dim3(256), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (uint16_t*)o, (uint16_t*)o_lo, lse, bs, cnt, idx, order, g.nbmax,
                       g.hpg, (int)g.N, scale2, out);
  return check_launch("k_fwd");
}

prism_status launch_mfma_bwd(const Geom& g, const int32_t* bs, const int32_t* cnt, const int32_t* idx, float sm_scale,
                             const void* q, const void* k, const void* v, const void* dout, const float* lse2,
                             const float* delta, const uint32_t* mask_t, int nw, const int32_t* order_q,
                             const int32_t* order_k, float* dq, float* dk, float* dv, const RowMap& out,
                             hipStream_t st) {
  dim3 grid((unsigned)(g.N / 64), g.heads);
  const float scale2 = sm_scale * kLog2e;
  {
    KernelTrace tr("k_dq", st);
    if (g.d == 64)
      hipLaunchKernelGGL(k_dq<64>, grid, dim3(256), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                         (const uint16_t*)v, (const uint16_t*)dout, lse2, delta, dq, bs, cnt, idx, order_q,
                         g.nbmax, g.hpg, (int)g.N, scale2, sm_scale, out);
    else
      hipLaunchKernelGGL(k_dq<128>, grid, dim3(256), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                         (const uint16_t*)v, (const uint16_t*)dout, lse2, delta, dq, bs, cnt, idx, order_q,
                         g.nbmax, g.hpg, (int)g.N, scale2, sm_scale, out);
  }
  prism_status s = check_launch("k_dq");
  if (s != PRISM_OK) return s;
  KernelTrace tr("k_dkdv", st);
  if (g.d == 64)
    hipLaunchKernelGGL(k_dkdv<64>, grid, dim3(256), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (const uint16_t*)dout, lse2, delta, dk, dv, bs, mask_t, order_k,
                       g.nbmax, nw, g.hpg, (int)g.N, scale2, sm_scale, out);
  else
    hipLaunchKernelGGL(k_dkdv<128>, grid, dim3(256), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (const uint16_t*)dout, lse2, delta, dk, dv, bs, mask_t, order_k,
                       g.nbmax, nw, g.hpg, (int)g.N, scale2, sm_scale, out);
  return check_launch("k_dkdv");
}

}  // namespace prism
