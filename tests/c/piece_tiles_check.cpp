// Host check of the per-sample query-tile map in positions.h
// (fill_piece_tiles, piece_tile): over seeded random packings of 1..256
// samples, every local row of the share lies in exactly one tile, each tile
// lies inside one piece (one sample's chunk r or 2 cp - 1 - r, length / (2 cp)
// rows) and holds at most `rows` rows.  Prints "piece tiles ok <cases>".
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <vector>

using std::max;  // the header's device code calls min and max unqualified
using std::min;

#include "positions.h"

namespace {
uint64_t state = 0x9e3779b97f4a7c15ull;
uint32_t next_u32() {  // xorshift64*
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (uint32_t)((state * 0x2545f4914f6cdd1dull) >> 32);
}

int fail(const char *what, int c, int lt) {
  std::printf("case %d tile %d: %s\n", c, lt, what);
  return 1;
}
}  // namespace

int main() {
  const int cps[] = {1, 2, 3, 4, 8};
  const int rows_opts[] = {128, 64, 32};
  int cases = 0;
  for (int c = 0; c < 600; ++c) {
    const int cp = cps[next_u32() % 5], rows = rows_opts[next_u32() % 3];
    usp::Samples s{};
    s.per_sample = 1;
    s.nseq = 1 + (int)(next_u32() % usp::kMaxSeqs);
    s.cu[0] = 0;
    for (int n = 0; n < s.nseq; ++n) {
      // piece lengths m of 1 .. 300, with 1, rows and rows + 1 made common
      const uint32_t r = next_u32() % 8;
      const int m = r == 0 ? 1 : r == 1 ? rows : r == 2 ? rows + 1 : 1 + (int)(next_u32() % 300);
      s.cu[n + 1] = s.cu[n] + 2 * cp * m;
    }
    const int L = s.cu[s.nseq] / cp;
    std::vector<int32_t> tiles(usp::kMaxSeqs + 1);
    const int nt = usp::fill_piece_tiles(s, cp, rows, tiles.data());
    std::vector<int> seen(L, 0);
    for (int lt = 0; lt < nt; ++lt) {
      int q0 = -1, qe = -1;
      usp::piece_tile(s, tiles.data(), cp, rows, lt, q0, qe);
      if (!(0 <= q0 && q0 < qe && qe <= L && qe - q0 <= rows)) return fail("out of bounds", c, lt);
      // the piece holding q0: sample n's rows start at cu[n] / cp, two pieces of m
      int n = 0;
      while (s.cu[n + 1] / cp <= q0) ++n;
      const int b = s.cu[n] / cp, m = (s.cu[n + 1] - s.cu[n]) / (2 * cp);
      const int pstart = q0 < b + m ? b : b + m;
      if (qe > pstart + m) return fail("tile crosses a piece", c, lt);
      for (int i = q0; i < qe; ++i) ++seen[i];
    }
    for (int i = 0; i < L; ++i)
      if (seen[i] != 1) return fail("row not covered exactly once", c, i);
    ++cases;
  }
  std::printf("piece tiles ok %d\n", cases);
  return 0;
}
