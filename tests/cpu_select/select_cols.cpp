// Host build of the library's per-lane channel-wise selection
// (select_lane.hpp, lane_select_columns): reads 64-row tiles of 128 fp16
// values (uint16, little endian) and a keep per tile from stdin, runs the
// selection for the 64 channel pairs as the 64 lanes of a wave would, and
// writes the tile's row bitmaps (four 32-bit words per row, bit j of word w <=>
// channel 32w + j kept) to stdout.
#include <stdint.h>
#include <stdio.h>

#include "../../unstructured_sparse_kv_amd/csrc/select_lane.hpp"

int main() {
  static uint16_t tile[64][128];
  int32_t keep;
  while (fread(&keep, 4, 1, stdin) == 1 && fread(tile, 2, 64 * 128, stdin) == 64 * 128) {
    uint32_t bm[64][4] = {};
    for (int l = 0; l < 64; ++l) {
      uint32_t y[64], lo[2], hi[2];
      for (int r = 0; r < 64; ++r) y[r] = tile[r][2 * l] | ((uint32_t)tile[r][2 * l + 1] << 16);
      mustafar::lane_select_columns(y, (uint32_t)keep / 2u, lo, hi);
      for (int r = 0; r < 64; ++r) {
        if ((lo[r / 32] >> (r % 32)) & 1u) bm[r][(2 * l) / 32] |= 1u << ((2 * l) % 32);
        if ((hi[r / 32] >> (r % 32)) & 1u) bm[r][(2 * l + 1) / 32] |= 1u << ((2 * l + 1) % 32);
      }
    }
    fwrite(bm, 4, 64 * 4, stdout);
  }
  return 0;
}
