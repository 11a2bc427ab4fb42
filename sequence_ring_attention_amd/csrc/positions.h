// Global positions of the rows of a ring rank's share, for both splits of
// the sequence into shares ([USP review] section 三, Algorithm 2):
//   * whole stream: the sequence is cut into 2 cp chunks of c tokens and
//     rank r holds chunks r and 2 cp - 1 - r, so local row i sits at
//     r c + i (i < c) or (2 cp - 1 - r) c + i - c;
//   * per sample: every packed sample n (boundaries cu[n], cu[n + 1], length
//     a multiple of 2 cp) is cut into 2 cp chunks of m_n tokens and rank r
//     holds chunks r and 2 cp - 1 - r of every sample, in sample order; the
//     rows of sample n start at local row cu[n] / cp.
// Positions increase with the local row in both, which is what lets the
// kernels bound tiles by their first and last rows and turn "position <= p"
// into a prefix length (count_le).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace usp {

constexpr int kMaxSeqs = 256;

__host__ __device__ inline int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Packed samples and the split, passed by value with the kernel arguments.
struct Samples {
  int32_t nseq;        // 0: one sequence, no sample mask
  int32_t per_sample;  // 1: per-sample split (needs nseq >= 1)
  int32_t cu[kMaxSeqs + 1];
};

struct ShareMap {
  int c, cp, L;
  const Samples *sm;  // points into the kernel arguments
  bool ps;            // per-sample split

  // A kernel built for the whole-stream split only passes per_sample_ok =
  // false, which removes the per-sample branches at compile time.
  __host__ __device__ ShareMap(int c_, int cp_, int L_, const Samples &s, bool per_sample_ok = true)
      : c(c_), cp(cp_), L(L_), sm(&s), ps(per_sample_ok && s.per_sample) {}

  __host__ __device__ bool packed() const { return sm->nseq > 0; }

  // Sample n holding global position p: cu[n] <= p < cu[n + 1].
  __host__ __device__ int sample_of(int p) const {
    int lo = 0, hi = sm->nseq;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sm->cu[mid] <= p) lo = mid; else hi = mid;
    }
    return lo;
  }

  // Global position of local row i of `rank`'s share.
  __host__ __device__ int pos(int rank, int i) const {
    if (!ps) return i < c ? rank * c + i : (2 * cp - 1 - rank) * c + (i - c);
    const int n = sample_of(i * cp);  // the sample's rows start at local row cu[n] / cp
    const int b = sm->cu[n], m = (sm->cu[n + 1] - b) / (2 * cp), o = i - b / cp;
    return b + (o < m ? rank * m + o : (2 * cp - 1 - rank) * m + (o - m));
  }

  // Number of local rows of `rank`'s share at positions <= p (a prefix).
  __host__ __device__ int count_le(int rank, int p) const {
    if (!ps) {
      const int a = clampi(p - rank * c + 1, 0, c);
      const int b = clampi(p - (2 * cp - 1 - rank) * c + 1, 0, c);
      return a + b;
    }
    if (p < 0) return 0;
    if (p >= cp * L) return L;
    const int n = sample_of(p);
    const int b = sm->cu[n], m = (sm->cu[n + 1] - b) / (2 * cp), q = p - b;
    return b / cp + clampi(q - rank * m + 1, 0, m) + clampi(q - (2 * cp - 1 - rank) * m + 1, 0, m);
  }

  // count_le(rank, p) for s0 - 1 <= p < s1, where [s0, s1) is a sample: the
  // per-sample split then needs no search (the samples before it put s0 / cp
  // rows in every share).
  __host__ __device__ int count_le_in(int rank, int p, int s0, int s1) const {
    if (!ps) return count_le(rank, p);
    const int m = (s1 - s0) / (2 * cp), q = p - s0;
    return s0 / cp + clampi(q - rank * m + 1, 0, m) + clampi(q - (2 * cp - 1 - rank) * m + 1, 0, m);
  }

  // First position of the sample holding p, and the first position after it.
  __host__ __device__ int seg_start(int p) const { return sm->cu[sample_of(p)]; }
  __host__ __device__ int seg_end(int p) const { return sm->cu[sample_of(p) + 1]; }
};

// Query tiles of a per-sample share cut at its pieces: the share holds two
// pieces per sample (its chunks r and 2 cp - 1 - r, m = length / (2 cp)
// rows each), and each piece is cut into tiles of at most `rows` rows, so a
// tile's rows lie in one sample and one chunk.  tiles[n] = the tiles before
// sample n; returns their total.  Host side, at launch.
inline int fill_piece_tiles(const Samples &s, int cp, int rows, int32_t *tiles) {
  tiles[0] = 0;
  for (int n = 0; n < s.nseq; ++n) {
    const int m = (s.cu[n + 1] - s.cu[n]) / (2 * cp);
    tiles[n + 1] = tiles[n] + 2 * ((m + rows - 1) / rows);
  }
  return tiles[s.nseq];
}

// Rows [q0, qend) of tile lt under the cut above (0 <= lt < tiles[nseq]).
// Host-callable too, for the CPU test of the map.
__host__ __device__ inline void piece_tile(const Samples &s, const int32_t *tiles, int cp, int rows, int lt, int &q0,
                                           int &qend) {
  int lo = 0, hi = s.nseq;  // the sample n with tiles[n] <= lt < tiles[n + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tiles[mid] <= lt) lo = mid; else hi = mid;
  }
  const int s0 = s.cu[lo], m = (s.cu[lo + 1] - s0) / (2 * cp);
  const int tp = (m + rows - 1) / rows, k = lt - tiles[lo], piece = k >= tp ? 1 : 0;
  const int pstart = s0 / cp + piece * m;
  q0 = pstart + (k - piece * tp) * rows;
  qend = q0 + rows < pstart + m ? q0 + rows : pstart + m;
}

}  // namespace usp
