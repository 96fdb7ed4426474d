// Host build of the library's per-lane selection (select_lane.hpp): reads rows
// of 128 fp16 values (uint16, little endian) and a keep per row from stdin,
// writes the four 32-bit mask words of each row to stdout.
#include <stdint.h>
#include <stdio.h>

#include "../../unstructured_sparse_kv_amd/csrc/select_lane.hpp"

int main() {
  uint16_t row[128];
  int32_t keep;
  while (fread(&keep, 4, 1, stdin) == 1 && fread(row, 2, 128, stdin) == 128) {
    uint32_t x[64], bm[4];
    for (int j = 0; j < 64; ++j) x[j] = row[2 * j] | ((uint32_t)row[2 * j + 1] << 16);
    mustafar::lane_select_row(x, (uint32_t)keep, bm);
    fwrite(bm, 4, 4, stdout);
  }
  return 0;
}
