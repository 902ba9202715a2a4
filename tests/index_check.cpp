// Exhaustive CPU checks of the kernels' index arithmetic (dynamic_block_sparse_var_amd/csrc/
// index_math.h), built with a host compiler under AddressSanitizer + UndefinedBehaviorSanitizer
// by tests/test_index_math.py.
//
//   index_check tiles            LDS tile addressing for head_dim 64 and 128
//   index_check units            xcd_atom is a bijection; block_of_row on random layouts
//   index_check layout T H W s0 s1 ... (one shape index per zone, edges from stdin as 16 x 3
//                                 ints): prints pos[n] (block-order row of token n) for the
//                                 caller to compare with the oracle's block layout
//
// Every failed check prints a line starting with FAIL and the program exits with status 1.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "index_math.h"

using namespace prism;

static int failures = 0;
#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      if (failures < 20) {                \
        printf("FAIL %s: ", #cond);       \
        printf(__VA_ARGS__);              \
        printf("\n");                     \
      }                                   \
      ++failures;                         \
    }                                     \
  } while (0)

template <int D>
static void check_tiles() {
  using TL = Tile<D>;
  const int tile_bytes = 64 * 2 * D, slots = tile_bytes / 16;
  // staging: every 16-byte slot of the tile written exactly once, with the chunk whose
  // swizzled slot it is, fetched from inside the 64 source rows
  std::vector<int> written(slots, 0);
  for (int w = 0; w < 4; ++w)
    for (int i = 0; i < TL::NI; ++i)
      for (int lane = 0; lane < 64; ++lane) {
        const uint32_t src = dma_src_offset<D>(w, lane, i);
        const uint32_t dst = (uint32_t)((w * TL::NI + i) * 1024 + 16 * lane);
        CHECK(src % 16 == 0 && src < (uint32_t)tile_bytes, "D=%d w=%d i=%d lane=%d src=%u", D, w, i, lane, src);
        CHECK(dst < (uint32_t)tile_bytes, "D=%d dst=%u", D, dst);
        const int r = (int)(src / (2 * D)), c = (int)((src % (2 * D)) / 16);
        CHECK((row_addr<D>(r) ^ (uint32_t)(c << 4)) == dst, "D=%d row %d chunk %d lands at %u, read at %u", D, r, c,
              dst, row_addr<D>(r) ^ (uint32_t)(c << 4));
        if (dst < (uint32_t)tile_bytes) written[dst / 16]++;
      }
  for (int sl = 0; sl < slots; ++sl) CHECK(written[sl] == 1, "D=%d slot %d written %d times", D, sl, written[sl]);
  // the b128 operand reads: chunk c of row r inside the tile; 16 consecutive rows at one chunk
  // take 16 distinct slots of their rows
  for (int r = 0; r < 64; ++r)
    for (int c = 0; c < TL::CPR; ++c) {
      const uint32_t a = row_addr<D>(r) ^ (uint32_t)(c << 4);
      CHECK(a >= (uint32_t)(r * 2 * D) && a + 16 <= (uint32_t)((r + 1) * 2 * D), "D=%d r=%d c=%d a=%u", D, r, c, a);
    }
  for (int r0 = 0; r0 < 64; r0 += 16)
    for (int c = 0; c < TL::CPR; ++c) {
      int seen[16] = {0};
      for (int r = r0; r < r0 + 16; ++r) {
        const int slot = (int)(((row_addr<D>(r) ^ (uint32_t)(c << 4)) % (2 * D)) / 16) % 16;
        seen[slot]++;
      }
      for (int q = 0; q < 16; ++q)
        CHECK(seen[q] <= (TL::CPR >= 16 ? 1 : 2), "D=%d rows %d..%d chunk %d: slot %d used %d times", D, r0,
              r0 + 15, c, q, seen[q]);
    }
  // the transposing reads: for every row base R0 (multiple of 16) and column block D0 (multiple
  // of 32) the 8-byte read of lane l, read b, is element (row, col..col+3) of the tile, inside
  // its row, and the 4 rows x 4 chunks of one 16-lane group take distinct slots
  for (int R0 = 0; R0 < 64; R0 += 16)
    for (int D0 = 0; D0 < D; D0 += 32)
      for (int lane = 0; lane < 64; ++lane)
        for (int b = 0; b < 2; ++b) {
          const uint32_t a = (tr_addr<D>(lane, b) ^ (uint32_t)(2 * D0)) + (uint32_t)(2 * D * R0);
          const int j = lane & 15;
          const int col = D0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
          const int row = R0 + 4 * (lane >> 5) + (j >> 2) + 8 * b;
          const uint32_t want = (row_addr<D>(row) ^ (uint32_t)((col >> 3) << 4)) + (uint32_t)((col & 7) * 2);
          CHECK(a == want, "D=%d R0=%d D0=%d lane=%d b=%d: %u, element at %u", D, R0, D0, lane, b, a, want);
          CHECK(a + 8 <= (uint32_t)tile_bytes, "D=%d tr read past the tile: %u", D, a);
        }
  // each half-wave's transposing read covers 4 rows x 4 chunks; for head_dim 128 (16 chunk
  // slots per row) those 16 (row, chunk) pairs take 16 distinct slots
  if (D == 128)
    for (int b = 0; b < 2; ++b)
      for (int h = 0; h < 2; ++h) {
        int seen[16] = {0};
        for (int lane = 32 * h; lane < 32 * h + 32; lane += 2) seen[(tr_addr<D>(lane, b) % (2 * D)) / 16]++;
        for (int q = 0; q < 16; ++q)
          CHECK(seen[q] == 1, "D=%d tr half %d read %d: slot %d used %d times", D, h, b, q, seen[q]);
      }
  printf("tiles D=%d checked\n", D);
}

static void check_units() {
  for (int n = 1; n <= 4096; ++n) {
    std::vector<int> seen(n, 0);
    for (int x = 0; x < n; ++x) {
      const int a = xcd_atom(x, n);
      CHECK(a >= 0 && a < n, "xcd_atom(%d, %d) = %d", x, n, a);
      if (a >= 0 && a < n) seen[a]++;
    }
    for (int a = 0; a < n; ++a) CHECK(seen[a] == 1, "xcd_atom: unit %d of %d taken %d times", a, n, seen[a]);
  }
  // block_of_row on random layouts of 64/128/256-row blocks, entries past the last block = N
  srand(12345);
  for (int t = 0; t < 200; ++t) {
    const int zones = 1 + rand() % 64, nbmax = 8 * zones, N = 512 * zones;
    std::vector<int32_t> bs(nbmax + 1, N);
    int j = 0;
    for (int m = 0; m < zones; ++m) {
      const int B = 64 << (rand() % 3);
      for (int q = 0; q < 512 / B; ++q) bs[j++] = 512 * m + q * B;
    }
    for (int row = 0; row < N; ++row) {
      const int k = block_of_row(bs.data(), nbmax, row);
      CHECK(k >= 0 && k < j && bs[k] <= row && row < (k + 1 < j ? bs[k + 1] : N), "block_of_row(%d) = %d", row, k);
    }
  }
  printf("units checked\n");
}

static void layout(int argc, char** argv) {
  const int T = atoi(argv[2]), H = atoi(argv[3]), W = atoi(argv[4]);
  const int ZT = T / 8, ZH = H / 8, ZW = W / 8, Z = ZT * ZH * ZW;
  if (argc != 5 + Z) {
    printf("FAIL usage: %d shape indices needed\n", Z);
    ++failures;
    return;
  }
  int edges[16][3];
  for (int i = 0; i < 16; ++i)
    if (scanf("%d %d %d", &edges[i][0], &edges[i][1], &edges[i][2]) != 3) {
      printf("FAIL edges\n");
      ++failures;
      return;
    }
  const int64_t N = (int64_t)T * H * W;
  std::vector<int64_t> pos(N, -1);
  for (int m = 0; m < Z; ++m) {
    const int s = atoi(argv[5 + m]);
    for (int p = 0; p < 512; ++p) {
      const int64_t n = zone_pos_token(m, p, edges[s][0], edges[s][1], edges[s][2], H, W, ZH, ZW);
      CHECK(n >= 0 && n < N, "zone %d pos %d -> token %lld", m, p, (long long)n);
      if (n < 0 || n >= N) continue;
      // the token lies in zone m
      const int t = (int)(n / ((int64_t)H * W)), h = (int)((n / W) % H), w = (int)(n % W);
      CHECK(((t / 8) * ZH + h / 8) * ZW + w / 8 == m, "zone %d pos %d -> token outside the zone", m, p);
      CHECK(pos[n] == -1, "token %lld reached twice", (long long)n);
      pos[n] = 512LL * m + p;
    }
  }
  for (int64_t n = 0; n < N; ++n) printf("%lld\n", (long long)pos[n]);
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "tiles") == 0) {
    check_tiles<64>();
    check_tiles<128>();
  } else if (argc >= 2 && strcmp(argv[1], "units") == 0) {
    check_units();
  } else if (argc >= 5 && strcmp(argv[1], "layout") == 0) {
    layout(argc, argv);
  } else {
    printf("FAIL usage\n");
    return 2;
  }
  if (failures) {
    printf("FAIL %d checks\n", failures);
    return 1;
  }
  return 0;
}
