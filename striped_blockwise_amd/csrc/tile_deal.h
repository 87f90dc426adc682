// Integer arithmetic that decides which key tiles the attention kernels visit and how they deal
// them to wavefronts: the per-round mask class, the ring schedule, the tiles a row range visits
// in a round, and the two ways of spreading one row group's tiles over several wavefronts (key
// splits, and the paired mode).  Plain C++ with no HIP dependence, so that the kernels and a
// host-side check compile the very same functions.
#pragma once

#include "ra.h"

#if defined(__HIPCC__) || defined(__HIP__)
#define RA_HD __host__ __device__ __forceinline__
#else
#define RA_HD inline
#endif

namespace ra {

// Per-(query device, K/V block) mask class.  From the causal matrix (query position < key
// position is masked; Striped Attention review, "核心公式") and the GetMask procedures
// ("GetMask 函数"), in local indices y (query row of block p) and x (key row of block k):
//   FULL   every pair visible   (non-causal; contiguous block from an earlier device)
//   INCL   visible iff x <= y   (contiguous own block; striped block from device k <= p)
//   STRICT visible iff x <  y   (striped block from device k > p)
//   SKIP   nothing visible      (contiguous block from a later device)
enum Mode : int { MODE_FULL = 0, MODE_INCL = 1, MODE_STRICT = 2, MODE_SKIP = 3 };

RA_HD int round_mode(int layout, int causal, int p, int k) {
  if (!causal) return MODE_FULL;
  if (layout == RA_CONTIGUOUS) return k < p ? MODE_FULL : (k == p ? MODE_INCL : MODE_SKIP);
  return k <= p ? MODE_INCL : MODE_STRICT;
}

// Ring schedule (Ring Attention review, step 2): blocks move from rank i to rank i+1 each
// round, so in round r device p holds the block that started on device (p - r) mod P.
RA_HD int ring_block(int p, int r, int P) {
  int k = (p - r) % P;
  return k < 0 ? k + P : k;
}

// Tiles of tk keys (out of ntk_all = ceil(c / tk)) that query rows up to `last` visit in a round
// of class `mode`: all (FULL), none (SKIP), else up to the last tile holding a key visible to
// row `last` (key <= row for INCL, key < row for STRICT).  Tiles are visited from 0 upwards.
RA_HD int visited_tiles(int mode, int last, int ntk_all, int tk) {
  if (mode == MODE_FULL) return ntk_all;
  if (mode == MODE_SKIP) return 0;
  const int lim = last - (mode == MODE_STRICT ? 1 : 0);
  if (lim < 0) return 0;
  const int t = lim / tk + 1;
  return t < ntk_all ? t : ntk_all;
}

// visited_tiles summed over the rounds r_begin .. r_begin + r_count - 1 of device p.
RA_HD int rounds_tiles(int layout, int causal, int p, int P, int r_begin, int r_count, int last,
                       int ntk_all, int tk) {
  int n = 0;
  for (int rr = 0; rr < r_count; ++rr)
    n += visited_tiles(round_mode(layout, causal, p, ring_block(p, r_begin + rr, P)), last, ntk_all, tk);
  return n;
}

// Key-stationary side (the dK/dV kernel): the first tile of ts query rows that holds a row
// seeing some key at or after key row x0 (all tiles for FULL; SKIP rounds are never visited).
RA_HD int first_query_tile(int mode, int x0, int ts) {
  return mode == MODE_FULL ? 0 : (x0 + (mode == MODE_STRICT ? 1 : 0)) / ts;
}

// Key splits: split s of ns takes tiles s, s + ns, s + 2 ns, ... of a round's n tiles.
RA_HD int split_count(int n, int s, int ns) { return n > s ? (n - s + ns - 1) / ns : 0; }
RA_HD int split_tile(int j, int s, int ns) { return j * ns + s; }

// Paired mode: a workgroup of nw wavefronts serves row groups a and b, with na and nb tiles over
// all its rounds.  Group a gets the number of wavefronts k (1 <= k < nw) for which the longer of
// the two per-wavefront shares, ceil(na / k) and ceil(nb / (nw - k)), is shortest; ties go to
// the more even split.  A workgroup whose two groups are one (a == b) gives it all nw.
RA_HD int paired_split(int na, int nb, int nw, bool same_group) {
  if (same_group) return nw;
  int ka = nw, best = 1 << 30;
  for (int k = 1; k < nw; ++k) {
    const int sa = (na + k - 1) / k, sb = (nb + nw - k - 1) / (nw - k);
    const int worst = sa > sb ? sa : sb;
    const int dk = 2 * k - nw < 0 ? nw - 2 * k : 2 * k - nw;
    const int dbest = 2 * ka - nw < 0 ? nw - 2 * ka : 2 * ka - nw;
    if (worst < best || (worst == best && dk < dbest)) {
      best = worst;
      ka = k;
    }
  }
  return ka;
}

// Paired mode, one round: the group's tiles are numbered on through its rounds (pbase of them
// came in earlier rounds) and dealt to its k wavefronts in turn; wavefront idx takes the round's
// tiles t0, t0 + k, ... below ntk, cnt of them.
RA_HD void paired_deal(int idx, int k, int pbase, int ntk, int& t0, int& cnt) {
  t0 = ((idx - pbase) % k + k) % k;
  cnt = t0 < ntk ? (ntk - t0 + k - 1) / k : 0;
}

// Paired query tiles (the dQ kernel under triangular masks): unit u of a stream's
// pair_count(nqt) units takes the query tiles u and nqt - 1 - u (the same tile twice for the
// middle unit of an odd count), so that every tile is taken exactly once.
RA_HD int pair_count(int nqt) { return (nqt + 1) / 2; }
RA_HD int pair_second(int u, int nqt) { return nqt - 1 - u; }

}  // namespace ra
