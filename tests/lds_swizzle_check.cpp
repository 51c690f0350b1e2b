// Host-side check of the LDS tile layout of the 16-bit kernels (swz and
// tile_off in fa_device.h) for every supported head dimension.  A tile of
// 64 rows x D 16-bit elements is filled by direct global->LDS copies: 16-byte
// slot s holds row s / CPR, chunk (s % CPR) ^ swz(row).  Checked:
//   - that map and tile_off are inverse bijections between slots and
//     (row, chunk);
//   - row reads: the 16 rows of an aligned 16-row group, one chunk column,
//     fall in 16 different bank groups (64 banks of 4 bytes = 16 groups of
//     one 16-byte slot);
//   - transpose reads: 4 aligned rows x an aligned group of 4 chunks fall in
//     16 different bank groups.
// Built with hipcc, run on the CPU; prints "ok" or the first failing case.
#include <cstdio>
#include <vector>

#include "fa_device.h"

template <int D>
bool check() {
  constexpr int CPR = D / 8, ROWS = 64;
  std::vector<int> hit(ROWS * CPR, 0);
  for (int s = 0; s < ROWS * CPR; ++s) {
    const int r = s / CPR, c = (s % CPR) ^ fa::swz<CPR>(r);
    if (c < 0 || c >= CPR || fa::tile_off<D>(r, c * 8) != s * 8 || hit[r * CPR + c]++) {
      std::printf("FAIL D=%d slot %d -> row %d chunk %d\n", D, s, r, c);
      return false;
    }
  }
  for (int r0 = 0; r0 < ROWS; r0 += 16)
    for (int c = 0; c < CPR; ++c) {
      unsigned seen = 0;
      for (int r = r0; r < r0 + 16; ++r) seen |= 1u << ((fa::tile_off<D>(r, c * 8) / 8) % 16);
      if (seen != 0xffffu) {
        std::printf("FAIL D=%d row read rows %d.. chunk %d\n", D, r0, c);
        return false;
      }
    }
  for (int r0 = 0; r0 < ROWS; r0 += 4)
    for (int c0 = 0; c0 < CPR; c0 += 4) {
      unsigned seen = 0;
      for (int r = r0; r < r0 + 4; ++r)
        for (int c = c0; c < c0 + 4; ++c) seen |= 1u << ((fa::tile_off<D>(r, c * 8) / 8) % 16);
      if (seen != 0xffffu) {
        std::printf("FAIL D=%d transpose read rows %d.. chunks %d..\n", D, r0, c0);
        return false;
      }
    }
  return true;
}

int main() {
  if (!(check<32>() && check<64>() && check<96>() && check<128>())) return 1;
  std::printf("ok\n");
  return 0;
}
