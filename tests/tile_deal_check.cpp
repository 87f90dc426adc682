// Host-side check of the kernels' tile dealing (csrc/tile_deal.h, compiled here by g++ exactly
// as the HIP kernels include it).  For every workgroup shape the attention kernels launch, and
// for ranges of block sizes, device counts, layouts and masks, it replays which key tiles each
// wavefront issues a DMA for and computes, and checks that
//   * every issued tile starts inside the block (x0 < c), so no DMA reads past a block;
//   * in every round, each tile a row group needs is computed by exactly one wavefront
//     (key splits: one split; paired mode: one wavefront of the group);
//   * the visited range is exact: it covers every visible (query, key) pair of the rows, and its
//     last tile holds a visible pair (or the round visits nothing when no pair is visible).
// Usage: tile_deal_check [c_max] ; prints "ok <cases>" and exits 0, or the first failure.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "tile_deal.h"

using namespace ra;

static long g_cases = 0;

#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      std::printf("FAIL %s:%d: ", __FILE__, __LINE__);     \
      std::printf(__VA_ARGS__);                            \
      std::printf("\n");                                   \
      std::exit(1);                                        \
    }                                                      \
  } while (0)

// Is key x (local) visible to query row y (local) under a mode?
static bool visible(int mode, int y, int x) {
  switch (mode) {
    case MODE_FULL: return true;
    case MODE_INCL: return x <= y;
    case MODE_STRICT: return x < y;
    default: return false;
  }
}

// The visited range of rows [y0, y_last] must cover every visible pair and be no longer than
// the last tile with a visible pair.
static void check_range(int mode, int y0, int y_last, int c, int tk, int ntk, const char* what) {
  const int ntk_all = (c + tk - 1) / tk;
  CHECK(ntk >= 0 && ntk <= ntk_all, "%s: ntk %d of %d", what, ntk, ntk_all);
  int need = 0;                                  // 1 + last tile holding a visible pair
  for (int y = y0; y <= y_last; ++y) {
    // the largest visible key of row y
    int xmax = -1;
    if (mode == MODE_FULL) xmax = c - 1;
    else if (mode == MODE_INCL) xmax = y;
    else if (mode == MODE_STRICT) xmax = y - 1;
    if (xmax > c - 1) xmax = c - 1;
    if (xmax >= 0) {
      CHECK(visible(mode, y, xmax) && (xmax + 1 >= c || !visible(mode, y, xmax + 1)), "%s: last key of row %d",
            what, y);
      need = need > xmax / tk + 1 ? need : xmax / tk + 1;
    }
  }
  CHECK(ntk == need, "%s: mode %d rows [%d, %d] c %d tk %d: visits %d tiles, needs %d", what, mode, y0, y_last,
        c, tk, ntk, need);
}

// Key-split shapes (the forward's 12 x 1, 2 x 4, 2 x 2 and 4 x 1 x 3 stages; the dQ kernel's 8 x 1,
// 2 x 4 and 4 x 2): NR row groups of 32 rows, NS splits.
static void check_split(int NR, int NS, int layout, int causal, int P, int c, int p, int r_begin, int r_count,
                        int tk) {
  const int TQ = NR * 32;
  const int nqt = (c + TQ - 1) / TQ;
  const int ntk_all = (c + tk - 1) / tk;
  std::vector<int> hits(ntk_all);
  for (int qt = 0; qt < nqt; ++qt) {
    const int q_wg_last = (c < (qt + 1) * TQ ? c : (qt + 1) * TQ) - 1;
    for (int rr = 0; rr < r_count; ++rr) {
      const int k = ring_block(p, r_begin + rr, P);
      CHECK(k >= 0 && k < P, "ring_block(%d, %d, %d) = %d", p, r_begin + rr, P, k);
      const int mode = round_mode(layout, causal, p, k);
      const int ntk = visited_tiles(mode, q_wg_last, ntk_all, tk);
      check_range(mode, qt * TQ, q_wg_last, c, tk, ntk, "split workgroup");
      std::fill(hits.begin(), hits.end(), 0);
      for (int s = 0; s < NS; ++s) {
        const int my_n = NS == 1 ? ntk : split_count(ntk, s, NS);
#ifdef REPLAY_UNGUARDED_FIRST_ISSUE
        // the former issue rule: every split of a workgroup that iterates issued its first tile,
        // owned or not (a planted mistake: the check must reject it)
        if (NR > 1 && ntk > 0 && my_n == 0)
          CHECK((long)split_tile(0, s, NS) * tk < c, "split %d: DMA at row %d past the block (c %d)", s,
                split_tile(0, s, NS) * tk, c);
#endif
        for (int j = 0; j < my_n; ++j) {          // exactly the tiles the kernel issues and computes
          const int t = split_tile(j, s, NS);
          CHECK(t >= 0 && t < ntk, "split %d of %d: tile %d outside [0, %d)", s, NS, t, ntk);
          CHECK((long)t * tk < c, "split %d: DMA at row %d past the block (c %d)", s, t * tk, c);
          ++hits[t];
        }
      }
      for (int t = 0; t < ntk; ++t)
        CHECK(hits[t] == 1, "NR %d NS %d c %d P %d p %d round %d: tile %d computed %d times", NR, NS, c, P, p,
              r_begin + rr, t, hits[t]);
      ++g_cases;
    }
  }
}

// Paired mode (the forward's small triangular launches): workgroup qt takes row groups qt and
// G - 1 - qt of 32 rows and deals their tiles over NW wavefronts.
static void check_paired(int NW, int layout, int causal, int P, int c, int p, int r_begin, int r_count, int tk) {
  const int QW = 32;
  const int G = (c + QW - 1) / QW;
  const int nqt = (c + 2 * QW - 1) / (2 * QW);
  const int ntk_all = (c + tk - 1) / tk;
  std::vector<int> group_seen(G, 0);
  std::vector<int> hits(ntk_all);
  for (int qt = 0; qt < nqt; ++qt) {
    const int rga = qt, rgb = G - 1 - qt;
    CHECK(rgb >= rga, "paired: workgroup %d of %d takes groups %d and %d", qt, nqt, rga, rgb);
    auto last_of = [&](int rg) { return (c < rg * QW + QW ? c : rg * QW + QW) - 1; };
    const int na = rounds_tiles(layout, causal, p, P, r_begin, r_count, last_of(rga), ntk_all, tk);
    const int nb = rounds_tiles(layout, causal, p, P, r_begin, r_count, last_of(rgb), ntk_all, tk);
    const int ka = paired_split(na, nb, NW, rga == rgb);
    if (rga == rgb) CHECK(ka == NW, "paired: one group gets every wavefront");
    else CHECK(ka >= 1 && ka <= NW - 1, "paired: %d wavefronts for group a of %d", ka, NW);
    ++group_seen[rga];
    if (rgb != rga) ++group_seen[rgb];
    for (int grp = 0; grp < (rga == rgb ? 1 : 2); ++grp) {
      const int rg = grp == 0 ? rga : rgb;
      const int kk = grp == 0 ? ka : NW - ka;
      const int last = last_of(rg);
      int pbase = 0, total = 0;
      for (int rr = 0; rr < r_count; ++rr) {
        const int mode = round_mode(layout, causal, p, ring_block(p, r_begin + rr, P));
        const int ntk = visited_tiles(mode, last, ntk_all, tk);
        check_range(mode, rg * QW, last, c, tk, ntk, "paired group");
        std::fill(hits.begin(), hits.end(), 0);
        for (int idx = 0; idx < kk; ++idx) {
          int t0, cnt;
          paired_deal(idx, kk, pbase, ntk, t0, cnt);
          for (int i = 0; i < cnt; ++i) {
            const int t = t0 + i * kk;
            CHECK(t >= 0 && t < ntk, "paired: tile %d outside [0, %d)", t, ntk);
            CHECK((long)t * tk < c, "paired: DMA at row %d past the block (c %d)", t * tk, c);
            ++hits[t];
          }
        }
        for (int t = 0; t < ntk; ++t)
          CHECK(hits[t] == 1, "paired c %d P %d p %d round %d group %d: tile %d computed %d times", c, P, p,
                r_begin + rr, rg, t, hits[t]);
        pbase += ntk;
        total += ntk;
        ++g_cases;
      }
      CHECK(total == (grp == 0 ? na : nb), "paired: group tile total %d vs counted %d", total, grp == 0 ? na : nb);
    }
  }
  for (int rg = 0; rg < G; ++rg) CHECK(group_seen[rg] == 1, "paired: row group %d served %d times", rg, group_seen[rg]);
}

// dK/dV kernel: key rows [x0, x_last] of one workgroup visit query tiles first_query_tile .. end;
// every query tile before that has no row that sees any of the keys, and the first one has one.
static void check_key_side(int layout, int causal, int P, int c, int kblk, int p, int wg_rows, int ts) {
  const int mode = round_mode(layout, causal, p, kblk);
  if (mode == MODE_SKIP) return;
  const int ntq = (c + ts - 1) / ts;
  for (int x0 = 0; x0 < c; x0 += wg_rows) {
    const int t0 = first_query_tile(mode, x0, ts);
    // the smallest query row that sees some key >= x0 (keys only become visible to later rows)
    int y_first = -1;
    for (int y = 0; y < c && y_first < 0; ++y)
      if (visible(mode, y, x0)) y_first = y;
    // no query sees these keys: whatever is visited holds no visible pair (the per-wave tile
    // class skips it) and lies inside the block (t0 >= 0, tiles below ntq)
    CHECK(t0 >= 0 && (y_first < 0 || t0 < ntq), "key side: first tile %d of %d", t0, ntq);
    if (y_first >= 0)
      CHECK(t0 == y_first / ts, "key side: mode %d keys from %d: first tile %d, needs %d", mode, x0, t0, y_first / ts);
    ++g_cases;
  }
}

// dQ kernel, paired query tiles: every tile of a stream is taken by exactly one unit.
static void check_query_pairs(int nqt) {
  std::vector<int> seen(nqt, 0);
  for (int u = 0; u < pair_count(nqt); ++u) {
    const int a = u, b = pair_second(u, nqt);
    CHECK(b >= a && b < nqt, "query pairs: unit %d of %d takes tiles %d and %d", u, nqt, a, b);
    ++seen[a];
    if (b != a) ++seen[b];
  }
  for (int t = 0; t < nqt; ++t) CHECK(seen[t] == 1, "query pairs: tile %d of %d taken %d times", t, nqt, seen[t]);
  ++g_cases;
}

int main(int argc, char** argv) {
  const int c_max = argc > 1 ? std::atoi(argv[1]) : 700;
  const int Ps[] = {1, 2, 3, 4, 8, 64};
  const int layouts[] = {RA_CONTIGUOUS, RA_STRIPED};
  // forward shapes: (NR, NS) with 32-key tiles; dQ shapes; the paired mode with 8 wavefronts
  const int fwd_split[][2] = {{12, 1}, {2, 4}, {2, 2}, {4, 1}};
  const int dq_split[][2] = {{8, 1}, {2, 4}, {4, 2}};
  for (int c = 1; c <= c_max; ++c) {
    for (int P : Ps) {
      for (int layout : layouts) {
        for (int causal = 0; causal <= 1; ++causal) {
          const int p_list[] = {0, P / 2, P - 1};
          for (int p : p_list) {
            for (const auto& sh : fwd_split) check_split(sh[0], sh[1], layout, causal, P, c, p, 0, P, 32);
            for (const auto& sh : dq_split) check_split(sh[0], sh[1], layout, causal, P, c, p, 0, P, 32);
            check_paired(8, layout, causal, P, c, p, 0, P, 32);
            for (int kb = 0; kb < P && kb < 8; ++kb) check_key_side(layout, causal, P, c, kb, p, 128, 32);
            // a single round (ra_round / ra_backward_round), every round of the ring
            if (c <= 130)
              for (int r = 0; r < P && r < 8; ++r) {
                check_split(2, 4, layout, causal, P, c, p, r, 1, 32);
                check_paired(8, layout, causal, P, c, p, r, 1, 32);
              }
          }
        }
      }
    }
  }
  for (int nqt = 1; nqt <= 1000; ++nqt) check_query_pairs(nqt);
  // the full-size shares: c = 32768 (P = 8 and 32), every device of P = 8
  for (int layout : layouts)
    for (int p = 0; p < 8; ++p) {
      check_split(12, 1, layout, 1, 8, 32768, p, 0, 8, 32);
      check_split(8, 1, layout, 1, 8, 32768, p, 0, 8, 32);
    }
  check_split(12, 1, RA_STRIPED, 1, 32, 32768, 31, 0, 32, 32);
  std::printf("ok %ld\n", g_cases);
  return 0;
}
