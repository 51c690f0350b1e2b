// Host-side check of the kernels' Philox4x32-10 (philox4x32_10 in
// fa_device.h) against the known-answer vectors published with the
// generator (Random123 distribution, Salmon et al., SC 2011).  Built with
// hipcc, run on the CPU; prints "ok" or the first failing case.
#include <cstdint>
#include <cstdio>

#include "fa_device.h"

int main() {
  struct Case {
    uint32_t c[4], k[2], want[4];
  } cases[] = {
      {{0, 0, 0, 0}, {0, 0}, {0x6627E8D5u, 0xE169C58Du, 0xBC57AC4Cu, 0x9B00DBD8u}},
      {{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu}, {0xFFFFFFFFu, 0xFFFFFFFFu},
       {0x408F276Du, 0x41C83B0Eu, 0xA20BC7C6u, 0x6D5451FDu}},
      {{0x243F6A88u, 0x85A308D3u, 0x13198A2Eu, 0x03707344u}, {0xA4093822u, 0x299F31D0u},
       {0xD16CFE09u, 0x94FDCCEBu, 0x5001E420u, 0x24126EA1u}},
  };
  for (const Case& t : cases) {
    uint32_t w[4];
    fa::philox4x32_10(t.c[0], t.c[1], t.c[2], t.c[3], t.k[0], t.k[1], w);
    for (int j = 0; j < 4; ++j)
      if (w[j] != t.want[j]) {
        std::printf("FAIL counter %08x: word %d = %08x, want %08x\n", t.c[0], j, w[j], t.want[j]);
        return 1;
      }
  }
  std::printf("ok\n");
  return 0;
}
