// Host-side check of the row clamp used by the direct global->LDS tile
// copies (clamped_chunk_offset in fa_device.h): for every tile start, tile
// row, matrix height and row stride (packed rows, and the wider strides of
// row-interleaved [B][N][H][d] views), the row actually read must be
// min(row0 + r, nrows - 1), inside [0, nrows).  Built with hipcc, run on
// the CPU; prints "ok" or the first failing case.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "fa_device.h"

int main() {
  const int dims[2] = {64, 128};
  const int stride_mul[3] = {1, 3, 16};  // rs = D, 3 D, 16 D
  std::vector<uint16_t> mat((size_t)(400 + 256) * 128 * 16);
  for (int D : dims)
    for (int mul : stride_mul)
      for (int nrows = 1; nrows <= 400; ++nrows)
        for (int row0 = 0; row0 < nrows + 192; row0 += 64) {
          if (row0 >= nrows + 128) break;  // a listed tile starts inside the last 128-row block
          const int64_t rs = (int64_t)D * mul;
          // the copy forms its address exactly so: tile base + per-lane offset
          const uint16_t* base = mat.data() + (int64_t)row0 * rs;
          for (int r = 0; r < 64; ++r)
            for (int c = 0; c < D; c += 8) {
              const uint32_t off = (uint32_t)(r * rs + c);
              const uint16_t* src = base + fa::clamped_chunk_offset(off, r, rs, row0, nrows);
              const long elem = (long)(src - mat.data());  // element index the copy reads
              const long row = elem / rs, col = elem % rs;
              const long want = row0 + r < nrows ? row0 + r : nrows - 1;
              if (elem < 0 || row != want || col != c || row >= nrows) {
                std::printf("FAIL D=%d rs=%ld nrows=%d row0=%d r=%d c=%d -> row %ld col %ld\n",
                            D, (long)rs, nrows, row0, r, c, row, col);
                return 1;
              }
            }
        }
  std::printf("ok\n");
  return 0;
}
