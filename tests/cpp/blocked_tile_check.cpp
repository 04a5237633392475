// Host check of the grouped GEMMs' work-item order (blocked_tile in device_common.h): for
// every expert shape, block height and item index the mapping lands inside the expert's
// M x N tiles, and it hits every tile exactly once.  Prints "ok <cases>" or the first failure.
#include <cstdio>
#include <vector>

#include "device_common.h"

int main() {
  long cases = 0;
  for (int mb : {0, 1, 2, 4, 8, 16, 32})
    for (int mt = 1; mt <= 80; ++mt)
      for (int NT = 1; NT <= 40; ++NT) {
        std::vector<int> seen(mt * NT, 0);
        for (int l = 0; l < mt * NT; ++l) {
          int nt = -1, m = -1;
          moe::blocked_tile(l, mt, NT, mb, nt, m);
          if (nt < 0 || nt >= NT || m < 0 || m >= mt) {
            std::printf("out of range: mb=%d mt=%d NT=%d item %d -> (%d, %d)\n", mb, mt, NT, l, nt, m);
            return 1;
          }
          ++seen[nt * mt + m];
        }
        for (int v : seen)
          if (v != 1) {
            std::printf("not a bijection: mb=%d mt=%d NT=%d\n", mb, mt, NT);
            return 1;
          }
        ++cases;
      }
  std::printf("ok %ld\n", cases);
  return 0;
}
