// Host check of the LDS tile layout used by the gfx950 kernels (lds_layout.h).
//
// Emulates, for D = 64 and 128:
//   * the direct global->LDS tile load (wave-wide load kb: lane L's 16 bytes land
//     at LDS bytes 1024 kb + 16 L),
//   * the row reads (16-byte loads at the reader's offsets),
//   * the transpose reads (ds_read_b64_tr_b16: in each 16-lane group lane i gives
//     the address of 4 consecutive bf16 of row i / 4 of a 4 x 16 block, columns
//     4 (i mod 4) .. +3; lane j receives column j of the block, rows 0..3),
// on a tile whose element (row, col) holds 1000 row + col, and checks that every
// lane receives the MFMA operand values its comment promises.  Then checks that
// every read instruction is free of bank conflicts on a 64-bank LDS: each group
// of 16 lanes of a 16-byte read, and each group of 32 lanes of an 8-byte read,
// touches distinct bank groups.  Prints "OK" and exits 0 when all hold.
#include <cstdio>
#include <cstring>
#include <set>
#include <vector>

#include "lds_layout.h"

using namespace bdattn;

static int failures = 0;
#define CHECK(cond, ...)                     \
  do {                                       \
    if (!(cond)) {                           \
      if (failures < 20) {                   \
        std::printf("FAIL: " __VA_ARGS__);   \
        std::printf("\n");                   \
      }                                      \
      ++failures;                            \
    }                                        \
  } while (0)

template <int D>
static void check_layout() {
  using T = TileShape<D>;
  // global tile, element (row, col) = 1000 row + col
  std::vector<int> glob(T::ROWS * D);
  for (int r = 0; r < T::ROWS; ++r)
    for (int c = 0; c < D; ++c) glob[r * D + c] = 1000 * r + c;
  // LDS as an array of elements (2 bytes each); -1 = never written
  std::vector<int> lds(T::BYTES / 2, -1);
  std::set<std::pair<int, int>> fetched;
  for (int kb = 0; kb < T::LOADS; ++kb)
    for (int lane = 0; lane < 64; ++lane) {
      int row, chunk;
      tile_load_src<D>(kb, lane, &row, &chunk);
      CHECK(row >= 0 && row < T::ROWS && chunk >= 0 && chunk < T::CPR, "D=%d load source out of tile", D);
      CHECK(fetched.insert({row, chunk}).second, "D=%d chunk (%d,%d) fetched twice", D, row, chunk);
      const int dst = (1024 * kb + 16 * lane) / 2;
      for (int e = 0; e < 8; ++e) lds[dst + e] = glob[row * D + 8 * chunk + e];
      // the layout formula agrees with where the load put it
      CHECK(tile_off<D>(row, chunk) == 1024 * kb + 16 * lane, "D=%d tile_off mismatch", D);
    }
  CHECK((int)fetched.size() == T::ROWS * T::CPR, "D=%d tile not fully loaded", D);

  // row reads
  for (int tb = 0; tb < 2; ++tb)
    for (int c = 0; c < T::NC; ++c) {
      int addr[64];
      for (int lane = 0; lane < 64; ++lane) {
        int off[T::NC];
        row_read_offsets<D>(lane, off);
        addr[lane] = off[c] + tb * 32 * T::ROWB;
        const int row = 32 * tb + (lane & 31), col0 = 16 * c + 8 * (lane >> 5);
        for (int e = 0; e < 8; ++e)
          CHECK(lds[addr[lane] / 2 + e] == 1000 * row + col0 + e, "D=%d row read lane %d tb %d c %d elem %d: got %d",
                D, lane, tb, c, e, lds[addr[lane] / 2 + e]);
      }
      for (int grp = 0; grp < 64; grp += 16) {
        std::set<int> banks;
        for (int l = grp; l < grp + 16; ++l) banks.insert((addr[l] % 256) / 16);
        CHECK(banks.size() == 16, "D=%d row read tb %d c %d lanes %d..: %zu bank groups", D, tb, c, grp, banks.size());
      }
    }

  // transpose reads
  for (int c16 = 0; c16 < T::ROWS / 16; ++c16)
    for (int mt = 0; mt < T::ND; ++mt) {
      int addr[2][64];
      for (int lane = 0; lane < 64; ++lane) {
        int off[T::ND];
        tr_read_offsets<D>(lane, off);
        addr[0][lane] = 16 * c16 * T::ROWB + off[mt];
        addr[1][lane] = 16 * c16 * T::ROWB + off[mt ^ T::TR_BX] + 8 * T::ROWB;
      }
      for (int lane = 0; lane < 64; ++lane) {
        const int grp = lane & ~15, jj = lane & 15, g = lane >> 5;
        const int m = 32 * mt + (lane & 31);
        for (int h = 0; h < 2; ++h)
          for (int k = 0; k < 4; ++k) {
            // lane jj receives column jj of the 4 x 16 block, row k: supplied by lane 4k + jj / 4
            const int src = grp + 4 * k + jj / 4;
            const int got = lds[addr[h][src] / 2 + (jj & 3)];
            const int row = 16 * c16 + 8 * h + 4 * g + k;
            CHECK(got == 1000 * row + m, "D=%d tr read lane %d c16 %d mt %d half %d k %d: got %d want %d", D, lane,
                  c16, mt, h, k, got, 1000 * row + m);
          }
      }
      for (int h = 0; h < 2; ++h)
        for (int grp = 0; grp < 64; grp += 32) {
          std::set<int> banks;
          for (int l = grp; l < grp + 32; ++l) banks.insert((addr[h][l] % 256) / 8);
          CHECK(banks.size() == 32, "D=%d tr read c16 %d mt %d half %d lanes %d..: %zu bank pairs", D, c16, mt, h, grp,
                banks.size());
        }
    }
}

int main() {
  check_layout<64>();
  check_layout<128>();
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("OK\n");
  return 0;
}
