// index_math.h -- the integer index arithmetic the kernels share: block order of a zone, block
// lookup, the XCD-contiguous unit order, and the addressing of the swizzled 64-row LDS tiles.
// Plain host + device functions, so that the same code is checked exhaustively on the CPU
// (tests/test_index_math.py compiles tests/index_check.cpp against this header with a host
// compiler under AddressSanitizer / UndefinedBehaviorSanitizer).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define PRISM_HD __host__ __device__ __forceinline__
#else
#define PRISM_HD inline
#endif

// Index assertions of the bounds-checked build (-DPRISM_DEBUG, `python -m
// dynamic_block_sparse_var_amd.build --debug`): each kernel checks that the rows, tiles and
// list entries it is about to touch lie inside their tensors.  Compiled out otherwise.
#if defined(PRISM_DEBUG)
#include <assert.h>
#define PRISM_ASSERT(cond) assert(cond)
#else
#define PRISM_ASSERT(cond) ((void)0)
#endif

namespace prism {

// Largest j in [0, nbmax) with bs[j] <= row (bs ascending, bs[j] = N past the last block).
PRISM_HD int block_of_row(const int32_t* bs, int nbmax, int row) {
  int lo = 0, hi = nbmax - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (bs[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Token of a block-order row.  Position p (0..511) of zone m's block-order range, the zone's
// blocks having edges (bT, bH, bW) in {2, 4, 8}: blocks in raster order over the zone's block
// grid, tokens in raster order inside a block.  Returns n = (t*H + h)*W + w.
PRISM_HD int ilog2_edge(int x) { return x == 2 ? 1 : x == 4 ? 2 : 3; }
PRISM_HD int64_t zone_pos_token(int m, int p, int bT, int bH, int bW, int H, int W, int ZH, int ZW) {
  const int lT = ilog2_edge(bT), lH = ilog2_edge(bH), lW = ilog2_edge(bW);
  const int lB = lT + lH + lW, lnW = 3 - lW, lnH = 3 - lH;
  const int beta = p >> lB, iota = p & ((1 << lB) - 1);
  const int bw = beta & ((1 << lnW) - 1), bh = (beta >> lnW) & ((1 << lnH) - 1), bt = beta >> (lnW + lnH);
  const int iw = iota & (bW - 1), ih = (iota >> lW) & (bH - 1), it = iota >> (lW + lH);
  const int zt = m / (ZH * ZW), zh = (m / ZW) % ZH, zw = m % ZW;
  return ((int64_t)(zt * 8 + (bt << lT) + it) * H + zh * 8 + (bh << lH) + ih) * W + zw * 8 + (bw << lW) + iw;
}

// Units (atoms or pairs) of one head in launch order, spread so that each XCD (workgroup id
// mod 8) walks a contiguous range: launch position x of a head's natoms units takes unit
// xcd_atom(x).
PRISM_HD int xcd_atom(int x, int natoms) {
  return ((natoms & 7) == 0) ? (x & 7) * (natoms >> 3) + (x >> 3) : x;
}

// ---- swizzled, unpadded 64 x D LDS tiles (bf16 rows of 2*D bytes) ------------------------
// Row r occupies 2*D contiguous bytes; its 16-byte chunk c sits in chunk slot c ^ swz(r).  The
// swizzle gives distinct slots to 16 consecutive rows at one chunk (the ds_read_b128 operand
// reads) and to 4 consecutive rows x 4 consecutive chunks (the ds_read_b64_tr_b16 reads).
template <int D>
PRISM_HD int swz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

template <int D>
struct Tile {
  static constexpr int CPR = D / 8;         // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;      // rows per 1 KB load
  static constexpr int NI = 16 / RPI;       // 1 KB loads per wave per tile (4 waves)
  static constexpr int ELEMS = 64 * D;
};

// Staging a tile: wave w's i-th 1 KB direct load puts lane l's 16 bytes at LDS byte
// (w*NI + i)*1024 + 16*l of the tile, so the lane fetches the chunk whose swizzled slot that
// is; this is its byte offset from the start of the 64 source rows.
template <int D>
PRISM_HD uint32_t dma_src_offset(int w, int lane, int i) {
  using TL = Tile<D>;
  const int r = (w * TL::NI + i) * TL::RPI + lane / TL::CPR;
  return (uint32_t)(r * 2 * D + (((lane % TL::CPR) ^ swz<D>(r)) << 4));
}

// Byte address of row r's chunk 0 slot; chunk c of row r is at row_addr(r) ^ (c << 4).
template <int D>
PRISM_HD uint32_t row_addr(int r) {
  return (uint32_t)(r * 2 * D + (swz<D>(r) << 4));
}

// The lane's byte address, for rows R0 = 0 and columns D0 = 0, of transposing read b (0, 1):
// 4 bf16 of row 4*(lane/32) + (lane%16)/4 + 8b at columns 16*((lane/16)%2) + 4*(lane%4).
// Reads at rows R0.. (R0 % 16 == 0) and columns D0.. (D0 % 32 == 0) are at
// (tr ^ (2 * D0)) + 2 * D * R0.
template <int D>
PRISM_HD uint32_t tr_addr(int lane, int b) {
  const int j = lane & 15;
  const int col = 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const int row = 4 * (lane >> 5) + (j >> 2) + 8 * b;
  return (uint32_t)(row * 2 * D + (((col >> 3) ^ swz<D>(row)) << 4) + (col & 7) * 2);
}

}  // namespace prism
