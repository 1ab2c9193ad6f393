// Host-side check of the symmetric product kernel's workgroup -> tile map
// (symk::sym_tile): for every grid of T x T tiles up to T = 64, the T^2
// workgroups cover each diagonal tile and each 256 x 128 half of the tiles
// above the diagonal exactly once, and for T a multiple of 4 each XCD's
// workgroups touch at most 2 T / 4 row blocks of 256 (the block partition).
// Compiled with hipcc; runs on the host only.
#include "gemm_sym.h"

#include <cstdio>
#include <set>
#include <vector>

int main() {
  int failures = 0;
  for (int t = 1; t <= 64; ++t) {
    const int nwg = t * t;
    std::set<long> seen;
    std::vector<std::set<int>> rows(8);
    for (int b = 0; b < nwg; ++b) {
      const ortho::symk::SymTile w = ortho::symk::sym_tile(t, nwg, b);
      const bool ok = w.tm >= 0 && w.tm < t && w.tn >= w.tm && w.tn < t && (w.half == 0 || w.half == 1) &&
                      !(w.tm == w.tn && w.half != 0);
      if (!ok || !seen.insert((long)w.tm * 4096 + w.tn * 2 + w.half).second) {
        printf("T=%d workgroup %d: tile (%d, %d, %d) %s\n", t, b, w.tm, w.tn, w.half,
               ok ? "repeated" : "out of range");
        ++failures;
        break;
      }
      rows[b & 7].insert(w.tm);
      rows[b & 7].insert(w.tn);
    }
    if ((int)seen.size() != nwg && failures == 0) {
      printf("T=%d: %zu of %d units covered\n", t, seen.size(), nwg);
      ++failures;
    }
    if (t % 4 == 0)
      for (int x = 0; x < 8; ++x)
        if ((int)rows[x].size() > t / 2) {
          printf("T=%d: XCD %d touches %zu row blocks (more than %d)\n", t, x, rows[x].size(), t / 2);
          ++failures;
        }
  }
  printf("%d failures\n", failures);
  return failures != 0;
}
