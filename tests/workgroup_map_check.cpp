// Host-side check of the workgroup -> (tile rank, head) map of the kernels
// (map_workgroup / snake in fa_device.h): for every grid shape and snake
// period tried, the map must be a permutation of [0, ntiles) x [0, nheads),
// keep every tile of a head on one XCD (workgroup id mod 8) when the head
// count is a multiple of 8, and balance the summed rank over the compute
// units that take workgroups period apart.  Built with hipcc, run on the
// CPU; prints "ok" or the first failing case.
#include <cstdio>
#include <vector>

#include "fa_device.h"

int main() {
  const int heads[] = {1, 2, 3, 7, 8, 16, 24, 40};
  const int periods[] = {0, 1, 2, 3, 5, 32, 256};
  for (int nheads : heads)
    for (int ntiles = 1; ntiles <= 140; ++ntiles)
      for (int period : periods) {
        const int grid = ntiles * nheads;
        std::vector<int> seen(grid, 0);
        for (int id = 0; id < grid; ++id) {
          int rank = -1, head = -1;
          fa::map_workgroup(id, ntiles, nheads, period, &rank, &head);
          if (rank < 0 || rank >= ntiles || head < 0 || head >= nheads ||
              seen[rank * nheads + head]++ ||
              ((nheads & 7) == 0 && (head & 7) != (id & 7))) {
            std::printf("FAIL nheads=%d ntiles=%d period=%d id=%d -> rank %d head %d\n", nheads,
                        ntiles, period, id, rank, head);
            return 1;
          }
        }
      }
  // balance: 16 heads, 64 tiles, 32 CUs per XCD each taking 4 workgroups;
  // a CU's summed rank must be within 2 of the mean (plain order: spread 60)
  {
    const int nheads = 16, ntiles = 64, period = 32, hpx = 2;
    std::vector<long> cu_sum(8 * period, 0);
    for (int id = 0; id < ntiles * nheads; ++id) {
      int rank, head;
      fa::map_workgroup(id, ntiles, nheads, period, &rank, &head);
      cu_sum[(id & 7) * period + ((id >> 3) % period)] += rank;
    }
    const long mean = (long)ntiles * nheads * (ntiles - 1) / 2 / (8 * period);
    for (long s : cu_sum)
      if (s < mean - 2 || s > mean + 2) {
        std::printf("FAIL balance: cu sum %ld, mean %ld\n", s, mean);
        return 1;
      }
    (void)hpx;
  }
  std::printf("ok\n");
  return 0;
}
