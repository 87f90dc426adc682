// bf16 blockwise attention on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), head dim 128.
//
// What one workgroup computes: NR row groups of QW query rows of device p's Q block, against the
// K/V blocks of the ring rounds it is given (Ring Attention review, step 2: round r brings the
// block of device (p - r) mod P), folding each round in with the online softmax (step 3).  Each
// row group's key tiles are spread over NS wavefronts (key splits) whose partial states are
// merged at the end, so a workgroup has NR NS wavefronts: 12 x 1 for grids with at least two
// such workgroups per CU, and split shapes for smaller grids (see launch_attn_bf16).
// Masks follow the GetMask procedures of the Striped Attention review ("GetMask 函数"), applied
// per tile: a tile with no visible pair is skipped ("分块与分瓦片"), a tile with every pair
// visible runs unmasked, and only tiles that straddle the diagonal pay for an element mask.
//
// Data flow per TK-key tile:
//   HBM -> LDS by DMA (buffer_load ... lds, 16 B per lane), K and V both row-major with a
//   per-row XOR swizzle of their 16-byte chunks; no registers or VALU work on the way in.  A
//   block's rows are consecutive in HBM, or P rows apart when a striped block is read straight
//   from a token-order tensor (row y of block k is token y P + k).  Two or three LDS stages per
//   key split: the next tiles' loads are in flight while this tile computes.
//   S^T = K Q^T on MFMA: A = 32 K rows from LDS, B = the wavefront's Q columns in registers.
//   In this orientation each lane owns one query, so the row max / row sum are in-lane
//   reductions plus one v_permlane32_swap with the other half of the wavefront.
//   P = exp2(S * scale * log2e - m) in fp32, rounded to bf16 (round-to-nearest-even).
//   O^T += V^T P^T on MFMA: A = V^T, read from the row-major V tile with ds_read_b64_tr_b16
//   (which transposes 4x4 blocks of 16-bit elements across lanes), B = P straight from the
//   score registers (the contraction index is permuted identically on both operands).
// The running max is only raised when a tile's max exceeds it by more than 8 (in log2 units),
// so the rescale of O (64-128 multiplies per lane) is rare; the result is exact either way
// because O, l and the reference max always stay consistent.  The tile max itself is only
// computed when P against the current reference comes out large (a lane's partial row sum
// above 2^12) or a row has no reference yet; otherwise that first P is kept.
#include <type_traits>

#include "bf16_tile.h"
#include "ra_internal.h"

namespace ra {
namespace {

using namespace bf16t;

#ifndef RA_BF16_NW
#define RA_BF16_NW 12           // wavefronts per workgroup (one workgroup fills a CU at 3 waves per SIMD)
#endif
#ifndef RA_BF16_XMAP
#define RA_BF16_XMAP 1          // 1: XCD-major block order (one (head, device) stream per XCD)
#endif
constexpr float TAU = 8.0f;     // lazy-rescale threshold, log2 units
#ifndef RA_BF16_LAZYMAX
#define RA_BF16_LAZYMAX 1       // 1: skip the tile max unless P against the current reference gets large
#endif
constexpr bool LAZYMAX = RA_BF16_LAZYMAX != 0;
constexpr float LAZY_LIM = 4096.0f;   // 2^(TAU + 4)

#ifndef RA_BF16_QB
#define RA_BF16_QB 1            // 32-query column blocks per wavefront
#endif
#ifndef RA_BF16_TK
#define RA_BF16_TK 32           // keys per tile
#endif
#ifndef RA_BF16_OCC
#define RA_BF16_OCC 2           // target wavefronts per SIMD
#endif
#ifndef RA_BF16_VPRE
#define RA_BF16_VPRE 3          // V^T fragments: 0 read next to each MFMA, 1 all read before the P V MFMAs,
                                // 2 all before the softmax, 3 the first 16 keys' before the softmax
#endif
#ifndef RA_BF16_PRIO
#define RA_BF16_PRIO 1          // 1: fixed issue priority wave % 3 (distinct on each SIMD)
#endif

// LDS layout of a K or V tile: row = key, 256 B = 16 chunks of 16 B with a per-row XOR mask on
// the chunk index.  K tiles are only read row-wise (MFMA A operand), V tiles only transposed
// (ds_read_b64_tr_b16), so each gets the mask that is conflict-free for its own read pattern.

// Workgroup shape: NR row groups of QW queries times NS key splits, NW = NR NS wavefronts.  The
// NR wavefronts of a split share its K/V tiles (one DMA, one LDS copy); split s takes tiles s,
// s + NS, s + 2 NS, ... of every round, so a row group's sweep over its keys is spread over NS
// wavefronts, whose partial softmax states are merged through LDS at the end (the same rule as
// the log-sum-exp merge of "Computing Attention Weights in Sequence Parallelism": rescale both
// to the larger reference, add numerators and denominators).  NST LDS stages per split: NST - 1
// tiles in flight while one computes.
//
// NST = 1 is the paired mode, for launches small enough to be resident at once.  Workgroup i of
// a stream takes the row groups i and G - 1 - i (G = row groups of the block) and divides its
// NR NS wavefronts between them so that the longer of the two groups' per-wavefront shares of
// key tiles is as short as it can be (under the causal masks the early rows see few keys and
// the late rows many).  Every wavefront then streams its share of
// its group's tiles through a private K buffer and V buffer, one tile each (K refilled once
// S is formed, V once P V is done), and each group's partial states are merged at the end.  The
// longest sweep of a wavefront then follows the pair's work, not the heaviest row group's.
template <int QB, int TK, bool STATS, int NR, int NS, int NST>
struct Attn {
  static constexpr int NW = NR * NS;              // wavefronts per workgroup
  static constexpr int QW = 32 * QB;              // query rows per wavefront
  static constexpr int TQ = NR * QW;              // query rows per workgroup
  static constexpr int KB = TK / 32;              // 32-key MFMA blocks per tile
  static constexpr int KS = TK / 16;              // 16-key MFMA k-steps per tile (P V)
  static constexpr int TILE = TK * ROWB;          // bytes of one K or V tile
  static constexpr int SPLIT_BYTES = 2 * NST * TILE;              // K stages, then V stages
  static constexpr int SLOT = QB * (64 * 64 * 4 + 2 * 64 * 4);    // one wavefront's O, m, l
  static constexpr bool PAIRED = NST == 1;
  static constexpr int STAGE_BYTES = PAIRED ? NW * SPLIT_BYTES : NS * SPLIT_BYTES;
  static constexpr int MERGE_BYTES = PAIRED ? NW * SLOT : (NS - 1) * NR * SLOT;
  static constexpr int LDS_BYTES = STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES;
  static_assert(NST >= 1 && NST <= 3, "one (paired), two or three stages");
  static_assert(!PAIRED || (NR == 2 && QB == 1), "paired mode: two row groups of 32 queries");

  // Per-lane constant parts of the LDS addresses (split base included).
  int k_base[8];       // K operand: row l32, chunk (2 dk + hh)
  int v_base[4][2];    // V^T operand: transposed reads, [d-block][first/second 4 keys]

  __device__ __forceinline__ void init_offsets(int lane, int split_base) {
#pragma unroll
    for (int dk = 0; dk < 8; ++dk) k_base[dk] = split_base + a_rowwise_off<SWZ_K>(lane, dk);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) v_base[db][sec] = split_base + a_tr_off<SWZ_V>(lane, db, sec);
  }
};

template <int QB, int TK, bool STATS, int NR, int NS, int NST>
__global__ __launch_bounds__(NR * NS * 64, RA_BF16_OCC) void k_attn_bf16(AttnArgs a) {
  using A = Attn<QB, TK, STATS, NR, NS, NST>;
  constexpr int NW = A::NW, QW = A::QW, TQ = A::TQ, KB = A::KB, KS = A::KS, TILE = A::TILE;
  __shared__ __attribute__((aligned(1024))) char smem[A::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = NS == 1 ? wave_u : wave_u % NR;   // row group
  const int s = NS == 1 ? 0 : wave_u / NR;        // key split
  constexpr bool PAIRED = A::PAIRED;
  constexpr int DNR = PAIRED ? 1 : NR;            // wavefronts sharing one tile's DMA
  const int split_base = (PAIRED ? wave_u : s) * A::SPLIT_BYTES;
  char* const sb = smem + split_base;             // this split's stages
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int c = a.c;
  // The three wavefronts that share a SIMD get distinct fixed issue priorities (wave % 3 differs
  // for w, w + 4, w + 8 as well as for three consecutive waves), so that after each tile's
  // barrier they do not contend symmetrically for the matrix core but run staggered; measured
  // 1.2% faster than equal priorities.
  if (RA_BF16_PRIO && NW % 3 == 0) {
    const int pr = wave_u % 3;
    if (pr == 1) __builtin_amdgcn_s_setprio(1);
    else if (pr == 2) __builtin_amdgcn_s_setprio(2);
  }

  // Block -> (stream = (device, head), q-tile).  Blocks are dispatched round-robin over the 8
  // XCDs (block i on XCD i % 8), each with its own L2.  XCD-major order gives XCD x the streams
  // x, x+8, x+16, ... one after another, all q-tiles of a stream together, so the workgroups
  // resident on an XCD read the same K/V blocks at about the same time.  Within a stream the
  // q-tiles with the most causal work go first.
  const int nqt = (c + TQ - 1) / TQ;
  int stream, qt;
  if (RA_BF16_XMAP && a.xcd_major) {
    const int x = blockIdx.x & 7;
    const int sq = blockIdx.x >> 3;
    stream = (sq / nqt) * 8 + x;
    qt = nqt - 1 - sq % nqt;
  } else {
    stream = blockIdx.x % (a.BH * a.n_dev);
    qt = nqt - 1 - blockIdx.x / (a.BH * a.n_dev);
  }
  const int bh = stream % a.BH;
  const int dev = stream / a.BH;
  const int p = a.p_begin + dev;
  const int q_wg0 = qt * TQ;
  // paired mode: this wavefront's index within its group, the group's wavefront count and the
  // group's first row
  int pw_idx = 0, pw_k = 1, prow = 0;
  if constexpr (PAIRED) {
    const int G = (c + QW - 1) / QW;
    const int rga = qt, rgb = G - 1 - qt;
    const int ntk_all0 = (c + TK - 1) / TK;
    auto group_tiles = [&](int rg) -> int {
      return rounds_tiles(a.layout, a.causal, p, a.P, a.r_begin, a.r_count, min(c, rg * QW + QW) - 1, ntk_all0, TK);
    };
    // wavefronts of group a: the split whose longest share is shortest (ties: the more even one)
    const int ka = rgb != rga ? paired_split(group_tiles(rga), group_tiles(rgb), NW, false) : NW;
    const bool in_a = wave_u < ka;
    pw_idx = in_a ? wave_u : wave_u - ka;
    pw_k = in_a ? ka : NW - ka;
    prow = (in_a ? rga : rgb) * QW;
  }
  const int q_wg_last = PAIRED ? min(c, prow + QW) - 1 : min(c, q_wg0 + TQ) - 1;
  const int qw0 = PAIRED ? prow : q_wg0 + g * QW;
  const int qw_last = min(c, qw0 + QW) - 1;  // < qw0 when the wave has no rows
  const bool wave_live = qw0 < c;

  A off;
  off.init_offsets(lane, split_base);
  unsigned kdma[DmaShape<DNR, TK>::PER_WAVE], vdma[DmaShape<DNR, TK>::PER_WAVE];
  dma_init<DNR, TK>(kdma, SWZ_K, PAIRED ? 0 : g, lane, a.row_step);
  dma_init<DNR, TK>(vdma, SWZ_V, PAIRED ? 0 : g, lane, a.row_step);

  // ---- Q columns (B operand): lane holds row qw0 + 32 qb + l32, head dims 16 dk + 8 hh .. +7
  const __bf16* qp = (const __bf16*)a.q + bh * a.q_bh_stride + dev * a.q_dev_stride;
  const int64_t rstride = (int64_t)a.row_step * D;   // elements between rows of a block
  bf16x8 qf[QB][8];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw0 + qb * 32 + l32;
#pragma unroll
    for (int dk = 0; dk < 8; ++dk)
      qf[qb][dk] = row < c ? *reinterpret_cast<const bf16x8*>(qp + row * rstride + dk * 16 + hh * 8)
                           : bf16x8{};
  }

  f32x16 o[QB][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < 4; ++db) o[qb][db] = f32x16{};
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { m[qb] = -INFINITY; l[qb] = 0.f; }
  const float cs = a.scale * LOG2E;
  // When the V^T fragments are read (see RA_BF16_VPRE).  Reading the first 16 keys' fragments
  // before the softmax lets their LDS latency pass under the exp work; all of them would need
  // more registers than the 3-waves-per-SIMD budget leaves.  The counting variant, which holds
  // more registers and is never timed, keeps the reads next to the MFMAs.  The paired mode
  // reads them all after the softmax, so that the single V buffer's next fill has the S and
  // softmax phases to land in.
  constexpr int VPRE = STATS ? 0 : (PAIRED ? 1 : RA_BF16_VPRE);
  // Small workgroups read V^T without the compiler's wait for every LDS DMA in flight (their own
  // waits cover the tile); measured faster for them and slower for the 12-wave workgroups.
  constexpr bool TR_NOWAIT = NW <= 8;

  // S^T tile of one wavefront: [qb][32-key block]
  f32x16 sA[QB][KB];

  // S^T = K Q^T for one tile.  All K fragments of a 32-key block are requested from LDS before
  // the first MFMA that needs one (the scheduling barrier keeps the compiler from interleaving
  // each read with its MFMA), so the LDS latency is paid once per block, not once per MFMA.
  auto compute_s = [&](const char* ks_, f32x16 (&s)[QB][KB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      bf16x8 kf[8];
#pragma unroll
      for (int dk = 0; dk < 8; ++dk)
        kf[dk] = *reinterpret_cast<const bf16x8*>(ks_ + off.k_base[dk] + kb * 32 * ROWB);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb][kb] = f32x16{};
#pragma unroll
      for (int dk = 0; dk < 8; ++dk)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[dk], qf[qb][dk], s[qb][kb], 0, 0, 0);
    }
  };

  // softmax of tile s (scores already masked) -> P (bf16, B-operand order), updates m, l, o
  auto softmax_pv = [&](f32x16 (&s)[QB][KB], const char* vs_) __attribute__((always_inline)) {
    bf16x8 va[KS][4];
    auto read_v = [&](int ks0, int ks1) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = ks0; ks < ks1; ++ks)
#pragma unroll
        for (int db = 0; db < 4; ++db)
          va[ks][db] = TR_NOWAIT ? read_a_tr_nowait(vs_ + ks * 16 * ROWB, off.v_base[db][0], off.v_base[db][1])
                                 : read_a_tr(vs_ + ks * 16 * ROWB, off.v_base[db][0], off.v_base[db][1]);
      __builtin_amdgcn_sched_barrier(0);
    };
    if (VPRE == 2) read_v(0, KS);
    if (VPRE == 3) read_v(0, 1);
    // Row max and lazy rescale: the reference m of a row is raised only when the tile's max
    // exceeds it by more than TAU (log2 units).
    auto grow_max = [&]() __attribute__((always_inline)) {
      bool any_grow = false;
      float mt[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = s[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int rg = 0; rg < 16; ++rg) mx = fmaxf(mx, s[qb][kb][rg]);
        mt[qb] = pair_max(mx) * cs;
        any_grow |= mt[qb] > m[qb] + TAU;
      }
      if (__builtin_amdgcn_ballot_w64(any_grow)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const bool grow = mt[qb] > m[qb] + TAU;
          const float m_new = grow ? mt[qb] : m[qb];
          const float alpha = grow ? __builtin_amdgcn_exp2f(m[qb] - m_new) : 1.0f;
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < 4; ++db) o[qb][db] *= alpha;
          m[qb] = m_new;
        }
      }
    };
    // P = exp2(S * cs - ref) -> bf16, and this lane's row sums of the unrounded values
    bf16x8 pf[QB][KS];
    float rsum[QB];
    auto make_p = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float ref = m[qb] == -INFINITY ? 0.f : m[qb];
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            bf16x8 pk;
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const float p0 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][half * 8 + e], cs, -ref));
              const float p1 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][half * 8 + e + 1], cs, -ref));
              const bf16x2 pp = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
              rs += p0 + p1;
              pk[e] = pp[0];
              pk[e + 1] = pp[1];
            }
            pf[qb][2 * kb + half] = pk;
          }
        rsum[qb] = rs;
      }
    };
    if (LAZYMAX) {
      // Without the tile max: P against the current reference, and the max path only when a
      // row has no reference yet or a lane's sum shows a value above 2^(TAU + 4) (each of the
      // lane's 16 values is at most its sum).  Either way O, l and m stay consistent.
      bool first = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) first |= m[qb] == -INFINITY;
      bool need_max = __builtin_amdgcn_ballot_w64(first) != 0;
      if (!need_max) {
        make_p();
        bool big = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) big |= !(rsum[qb] <= LAZY_LIM);
        need_max = __builtin_amdgcn_ballot_w64(big) != 0;
      }
      if (need_max) {
        grow_max();
        make_p();
      }
    } else {
      grow_max();
      make_p();
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l[qb] += rsum[qb];
    // O^T += V^T P^T
    if (VPRE == 1) read_v(0, KS);
    if (VPRE == 3) read_v(1, KS);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        if (VPRE == 0)
          va[ks][db] = TR_NOWAIT ? read_a_tr_nowait(vs_ + ks * 16 * ROWB, off.v_base[db][0], off.v_base[db][1])
                                 : read_a_tr(vs_ + ks * 16 * ROWB, off.v_base[db][0], off.v_base[db][1]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks][db], pf[qb][ks], o[qb][db], 0, 0, 0);
      }
    }
  };

  const int ntk_all = (c + TK - 1) / TK;
  int pbase = 0;                                  // paired mode: tiles of the group in earlier rounds
  // tiles of [0, n) that split s takes (s, s + NS, ...)
  auto my_tiles = [&](int n) -> int { return NS == 1 ? n : split_count(n, s, NS); };
  // Loads per tile and wavefront (K and V) for the partial wait of a three-stage pipeline; every
  // wavefront of a split then issues the same number.
  constexpr int LPT = 2 * DmaShape<NR, TK>::PER_WAVE;
  static_assert(NST == 2 || DmaShape<NR, TK>::SEGS % NR == 0, "uneven DMA shares");
  for (int rr = 0; rr < a.r_count; ++rr) {
    const int r = a.r_begin + rr;
    const int k = ring_block(p, r, a.P);
    const int mode = round_mode(a.layout, a.causal, p, k);
    const int delta = mode == MODE_STRICT ? 1 : 0;
    // tiles this workgroup visits: up to the last one with a visible pair for its rows
    const int ntk = visited_tiles(mode, q_wg_last, ntk_all, TK);

    const int64_t kvo = bh * a.kv_bh_stride + (int64_t)(k - a.kv_base) * a.kv_blk_stride;
    const char* kblk = (const char*)((const __bf16*)a.k + kvo);
    const char* vblk = (const char*)((const __bf16*)a.v + kvo);

    uint64_t st_full = 0, st_diag = 0, st_pairs_uniform = 0;
    uint32_t st_pairs_lane = 0;

    // per-wave tile class: 0 skip; 1 every pair visible; 2 diagonal (element mask, pairs counted
    // per element); 3 every in-range pair visible but the tile runs past the block end (mask only
    // the keys past the end)
    auto tile_class = [&](int t) -> int {
      const int x0 = t * TK;
      const int x_last = min(c, x0 + TK) - 1;
      if (!wave_live || (mode != MODE_FULL && x0 > qw_last - delta)) return 0;
      const bool full = mode == MODE_FULL || x_last <= qw0 - delta;
      if (STATS) {
        if (full) { ++st_full; st_pairs_uniform += (uint64_t)(qw_last - qw0 + 1) * (x_last - x0 + 1); }
        else ++st_diag;
      }
      return full ? (x0 + TK <= c ? 1 : 3) : 2;
    };
    auto apply_mask = [&](f32x16 (&s)[QB][KB], int t, bool count) __attribute__((always_inline)) {
      const int x0 = t * TK;
      const bool full_mode = mode == MODE_FULL;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int y = qw0 + qb * 32 + l32;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int rg = 0; rg < 16; ++rg) {
            const int x = x0 + 32 * kb + acc_row(rg, hh);
            const bool vis = x < c && (full_mode || x <= y - delta);
            if (STATS && count) st_pairs_lane += (vis && y < c) ? 1u : 0u;
            s[qb][kb][rg] = vis ? s[qb][kb][rg] : -INFINITY;
          }
      }
    };

    if constexpr (PAIRED) {
      // The group's tiles, numbered on from the earlier rounds, go to its pw_k wavefronts in
      // turn: this wavefront takes t0, t0 + pw_k, ...  One K and one V buffer of its own: K(t+1)
      // is fetched once S of t is formed, V(t+1) once P V of t is done.  K and V DMAs of a tile
      // are issued in that order and complete in order, so waiting until at most VL loads are
      // outstanding means the older of the two has landed.
      constexpr int VL = DmaShape<1, TK>::PER_WAVE;
      int t0, cnt;
      paired_deal(pw_idx, pw_k, pbase, ntk, t0, cnt);
      pbase += ntk;
      if (cnt > 0) {
        dma_issue<1, TK>(kdma, kblk, sb, t0 * TK, c, a.row_step, 0);
        dma_issue<1, TK>(vdma, vblk, sb + TILE, t0 * TK, c, a.row_step, 0);
        for (int i = 0; i < cnt; ++i) {
          const int t = t0 + i * pw_k;
          const bool more = i + 1 < cnt;
          vm_wait<VL>();                              // K(t) landed
          const int cls = tile_class(t);
          if (cls) compute_s(smem, sA);
          lgkm_wait0();                               // K reads returned: the buffer may refill
          if (more) dma_issue<1, TK>(kdma, kblk, sb, (t + pw_k) * TK, c, a.row_step, 0);
          if (more) vm_wait<VL>();                    // V(t) landed (K(t + pw_k) in flight)
          else vm_wait<0>();
          if (cls) {
            if (cls >= 2) apply_mask(sA, t, cls == 2);
            softmax_pv(sA, smem + TILE);
          }
          lgkm_wait0();                               // V reads returned
          if (more) dma_issue<1, TK>(vdma, vblk, sb + TILE, (t + pw_k) * TK, c, a.row_step, 0);
        }
      }
    } else if constexpr (NS == 1 && NST == 2) {
      // One split, two stages: tile t lives in stage t & 1; its DMA was issued one iteration
      // earlier.  The loop is unrolled by two so that the stage offsets are compile-time
      // immediates.
      if (ntk > 0) {
        dma_issue<NR, TK>(kdma, kblk, smem, 0, c, a.row_step, g);
        dma_issue<NR, TK>(vdma, vblk, smem + 2 * TILE, 0, c, a.row_step, g);
        auto iter = [&](int t, auto stage_c) __attribute__((always_inline)) {
          constexpr int S = decltype(stage_c)::value;
          vm_wait<0>();                               // tile t landed; with NR > 1 the barrier
          if (NR > 1) __syncthreads();                // makes it whole and frees the other stage
          if (t + 1 < ntk) {
            dma_issue<NR, TK>(kdma, kblk, smem + (1 - S) * TILE, (t + 1) * TK, c, a.row_step, g);
            dma_issue<NR, TK>(vdma, vblk, smem + (3 - S) * TILE, (t + 1) * TK, c, a.row_step, g);
          }
          const int cls = tile_class(t);
          if (cls) {
            compute_s(smem + S * TILE, sA);
            if (cls >= 2) apply_mask(sA, t, cls == 2);
            softmax_pv(sA, smem + (2 + S) * TILE);
          }
        };
        int t = 0;
        for (; t + 1 < ntk; t += 2) {
          iter(t, std::integral_constant<int, 0>{});
          iter(t + 1, std::integral_constant<int, 1>{});
        }
        if (t < ntk) iter(t, std::integral_constant<int, 0>{});
        if (NR > 1) __syncthreads();                  // LDS stages free for the next round
      }
    } else {
      // This split's tiles: j = 0 .. my_n - 1 is tile j NS + s.  Wavefronts that share tiles
      // (NR > 1) run the same iteration count in lock-step; a lone wavefront runs its own.
      const int my_n = my_tiles(ntk);
      const int nit = NR > 1 ? (ntk + NS - 1) / NS : my_n;
      if (nit > 0) {
        // my tile j lives in stage j % NST; its DMA was issued NST - 1 iterations earlier.  The
        // loop is unrolled by NST so that the stage offsets are compile-time immediates.
        auto issue = [&](int j, int stage) __attribute__((always_inline)) {
          const int x0 = split_tile(j, s, NS) * TK;
          dma_issue<NR, TK>(kdma, kblk, sb + stage * TILE, x0, c, a.row_step, g);
          dma_issue<NR, TK>(vdma, vblk, sb + (NST + stage) * TILE, x0, c, a.row_step, g);
        };
        // only tiles this split owns: with NR > 1 a split may have none in a round that the
        // others still iterate over, and its first tile would start past the end of the block
        if (my_n > 0) issue(0, 0);
        if (NST == 3 && my_n > 1) issue(1, 1);
        auto iter = [&](int j, auto stage_c) __attribute__((always_inline)) {
          constexpr int S = decltype(stage_c)::value;
          // my tile j landed (with three stages tile j + 1 may stay in flight); with NR > 1 the
          // barrier makes the whole tile visible and frees the stage read one iteration ago
          if (NST == 3 && j + 1 < my_n) vm_wait<LPT>();
          else vm_wait<0>();
          if (NR > 1) __syncthreads();
          if (j + NST - 1 < my_n) issue(j + NST - 1, (S + NST - 1) % NST);
          if (NR == 1 || j < my_n) {
            const int t = split_tile(j, s, NS);
            const int cls = tile_class(t);
            if (cls) {
              compute_s(smem + S * TILE, sA);
              if (cls >= 2) apply_mask(sA, t, cls == 2);
              softmax_pv(sA, smem + (NST + S) * TILE);
            }
          }
        };
        int j = 0;
        for (; j + NST <= nit; j += NST) {
          iter(j, std::integral_constant<int, 0>{});
          iter(j + 1, std::integral_constant<int, 1>{});
          if constexpr (NST == 3) iter(j + 2, std::integral_constant<int, 2>{});
        }
        if (j < nit) iter(j, std::integral_constant<int, 0>{});
        if (NST == 3 && j + 1 < nit) iter(j + 1, std::integral_constant<int, 1>{});
        if (NR > 1) __syncthreads();                  // LDS stages free for the next round
      }
    }

    if (STATS && wave_live) {
      unsigned long long pairs = st_pairs_lane;
      for (int off2 = 32; off2 > 0; off2 >>= 1) pairs += __shfl_xor(pairs, off2);
      if (lane == 0) {
        ra_round_stats_t* st = a.stats_single ? a.stats : a.stats + ((int64_t)p * a.P + r);
        atomicAdd((unsigned long long*)&st->unmasked_pairs, (unsigned long long)(pairs + st_pairs_uniform));
        atomicAdd((unsigned long long*)&st->tiles_full, (unsigned long long)st_full);
        atomicAdd((unsigned long long*)&st->tiles_diag, (unsigned long long)st_diag);
        // skipped tiles of a row group: all of them less those its wavefronts visited (in the
        // paired mode the group's first wavefront adds the group's tiles, every one subtracts
        // its own; the unsigned sum wraps to the group's count)
        const uint64_t own = PAIRED ? (pw_idx == 0 ? (uint64_t)ntk_all : 0) : (uint64_t)my_tiles(ntk_all);
        atomicAdd((unsigned long long*)&st->tiles_skipped, (unsigned long long)(own - st_full - st_diag));
      }
    }
  }

  // ---- key splits: splits 1 .. NS-1 hand (m, l, O) to split 0 of their row group through LDS;
  // split 0 folds them in with the blockwise softmax merge (both sides rescaled to the larger
  // reference; a side that saw no key has m = -inf and contributes nothing).
  if constexpr (PAIRED) {
    // every wavefront parks (m, l, O) in its slot; the first wavefront of each group folds in
    // the others of the group with the same merge rule
    __syncthreads();                                  // every wavefront is done with its buffers
    {
      char* const slot = smem + wave_u * A::SLOT;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          reinterpret_cast<float4*>(slot)[(db * 4 + q4) * 64 + lane] =
              make_float4(o[0][db][4 * q4], o[0][db][4 * q4 + 1], o[0][db][4 * q4 + 2], o[0][db][4 * q4 + 3]);
      float* ml = reinterpret_cast<float*>(slot + 64 * 64 * 4);
      ml[lane] = m[0];
      ml[64 + lane] = l[0];
    }
    __syncthreads();
    if (pw_idx != 0) return;
#pragma unroll 1
    for (int j = 1; j < pw_k; ++j) {
      const char* const slot = smem + (wave_u + j) * A::SLOT;
      const float* ml = reinterpret_cast<const float*>(slot + 64 * 64 * 4);
      const float m2 = ml[lane], l2 = ml[64 + lane];
      const float mn = fmaxf(m[0], m2);
      const float al = m[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[0] - mn);
      const float be = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
      l[0] = al * l[0] + be * l2;
      m[0] = mn;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 w = reinterpret_cast<const float4*>(slot)[(db * 4 + q4) * 64 + lane];
          o[0][db][4 * q4] = al * o[0][db][4 * q4] + be * w.x;
          o[0][db][4 * q4 + 1] = al * o[0][db][4 * q4 + 1] + be * w.y;
          o[0][db][4 * q4 + 2] = al * o[0][db][4 * q4 + 2] + be * w.z;
          o[0][db][4 * q4 + 3] = al * o[0][db][4 * q4 + 3] + be * w.w;
        }
    }
  }
  if constexpr (NS > 1 && !PAIRED) {
    __syncthreads();                                  // every split is done with its stages
    if (s > 0) {
      char* const slot = smem + ((s - 1) * NR + g) * A::SLOT;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            reinterpret_cast<float4*>(slot)[((qb * 4 + db) * 4 + q4) * 64 + lane] =
                make_float4(o[qb][db][4 * q4], o[qb][db][4 * q4 + 1], o[qb][db][4 * q4 + 2], o[qb][db][4 * q4 + 3]);
        float* ml = reinterpret_cast<float*>(slot + QB * 64 * 64 * 4);
        ml[qb * 128 + lane] = m[qb];
        ml[qb * 128 + 64 + lane] = l[qb];
      }
    }
    __syncthreads();
    if (s > 0) return;
#pragma unroll 1
    for (int s2 = 1; s2 < NS; ++s2) {
      const char* const slot = smem + ((s2 - 1) * NR + g) * A::SLOT;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float* ml = reinterpret_cast<const float*>(slot + QB * 64 * 64 * 4);
        const float m2 = ml[qb * 128 + lane], l2 = ml[qb * 128 + 64 + lane];
        const float mn = fmaxf(m[qb], m2);
        const float al = m[qb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[qb] - mn);
        const float be = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
        l[qb] = al * l[qb] + be * l2;
        m[qb] = mn;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const float4 w = reinterpret_cast<const float4*>(slot)[((qb * 4 + db) * 4 + q4) * 64 + lane];
            o[qb][db][4 * q4] = al * o[qb][db][4 * q4] + be * w.x;
            o[qb][db][4 * q4 + 1] = al * o[qb][db][4 * q4 + 1] + be * w.y;
            o[qb][db][4 * q4 + 2] = al * o[qb][db][4 * q4 + 2] + be * w.z;
            o[qb][db][4 * q4 + 3] = al * o[qb][db][4 * q4 + 3] + be * w.w;
          }
      }
    }
  }

  // ---- finalize: O = acc / l, LSE = ln(2) * (m + log2 l); rows with no key: 0 and -inf (a NaN
  // normaliser, from NaN inputs, counts as live so that the NaN reaches O and LSE)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = pair_sum(l[qb]);
    const bool live = !(lt <= 0.f);
    const float inv = live ? 1.f / lt : 0.f;
    const int y = qw0 + qb * 32 + l32;
    if (y < c) {
      const int64_t oel = bh * a.o_bh_stride + dev * a.o_dev_stride + y * rstride;
      if (a.o_f32) {
        float* op = (float*)a.o + oel;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 w = make_float4(o[qb][db][4 * g] * inv, o[qb][db][4 * g + 1] * inv,
                                         o[qb][db][4 * g + 2] * inv, o[qb][db][4 * g + 3] * inv);
            *reinterpret_cast<float4*>(op + 32 * db + 8 * g + 4 * hh) = w;
          }
      } else {
        __bf16* op = (__bf16*)a.o + oel;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const bf16x2 w0 = __builtin_convertvector(f32x2{o[qb][db][4 * g] * inv, o[qb][db][4 * g + 1] * inv}, bf16x2);
            const bf16x2 w1 = __builtin_convertvector(f32x2{o[qb][db][4 * g + 2] * inv, o[qb][db][4 * g + 3] * inv}, bf16x2);
            u32x2 w = {__builtin_bit_cast(uint32_t, w0), __builtin_bit_cast(uint32_t, w1)};
            *reinterpret_cast<u32x2*>(op + 32 * db + 8 * g + 4 * hh) = w;
          }
      }
      if (a.lse && hh == 0)
        a.lse[bh * a.lse_bh_stride + dev * a.lse_dev_stride + (int64_t)y * a.row_step] = live ? (m[qb] + __log2f(lt)) * LN2 : -INFINITY;
    }
  }
}

constexpr int QB_SEL = RA_BF16_QB;
constexpr int TK_SEL = RA_BF16_TK;

}  // namespace

bool attn_bf16_supported(int64_t d) { return d == D; }
void attn_bf16_tile(int* tq, int* tk) { *tq = 32 * QB_SEL; *tk = TK_SEL; }

namespace {

template <int NR, int NS, int NST>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t s) {
  constexpr int NW = NR * NS;
  constexpr int TQ = NR * 32 * QB_SEL;
  const int64_t blocks = (int64_t)((a.c + TQ - 1) / TQ) * a.BH * a.n_dev;
  if (blocks * NW * 64 >= (1ll << 32)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks);
  AttnArgs b = a;
  b.xcd_major = ((int64_t)a.BH * a.n_dev) % 8 == 0 ? 1 : 0;
  if (a.stats)
    hipLaunchKernelGGL((k_attn_bf16<QB_SEL, TK_SEL, true, NR, NS, NST>), grid, dim3(NW * 64), 0, s, b);
  else
    hipLaunchKernelGGL((k_attn_bf16<QB_SEL, TK_SEL, false, NR, NS, NST>), grid, dim3(NW * 64), 0, s, b);
  return hipGetLastError();
}

// True when no round of the launch shows a row group every key: causal, and no contiguous round
// with k < p (that is, with r mod P in 1..p for a launched device p).  Row groups then have work
// that grows with their position in the block, which the paired workgroups balance.
bool triangular_rounds(const AttnArgs& a) {
  if (!a.causal) return false;
  if (a.layout != RA_CONTIGUOUS) return true;
  const int p_max = a.p_begin + a.n_dev - 1;
  for (int i = 0; i < a.r_count && i < a.P; ++i) {
    const int res = (a.r_begin + i) % a.P;
    if (res >= 1 && res <= p_max) return false;
  }
  return true;
}

}  // namespace

// Workgroup shape by grid size.  Wide workgroups (one per CU, 384 queries sharing each K/V tile)
// when the grid has at least two of them per CU.  Below that, a round lasts about as long as the
// longest sweep of one wavefront over its key tiles, and the smaller the grid the more that sweep
// is split over wavefronts: with G = 32-row groups of the whole launch and C compute units,
//   G <= 2 C and every round triangular (see triangular_rounds): the paired mode (8 wavefronts
//               for two row groups, 132 KB LDS, the whole launch resident at once),
//   G <= 4 C:   2 row groups x 4 key splits (8 wavefronts, 128 KB LDS, one workgroup per CU),
//   G <= 12 C:  2 row groups x 2 key splits (4 wavefronts, 64 KB LDS, two per CU),
//   otherwise:  4 row groups, one split, three LDS stages (4 wavefronts, 48 KB LDS).
// Apart from the paired mode, which only pays when the row groups' work differs, the shape
// depends on the grid, not on the mask.
hipError_t launch_attn_bf16(const AttnArgs& a, int d, hipStream_t s) {
  if (d != D) return hipErrorInvalidValue;
  const int64_t cus = cu_count();
  constexpr int TQW = RA_BF16_NW * 32 * QB_SEL;
  const int64_t wide = (int64_t)((a.c + TQW - 1) / TQW) * a.BH * a.n_dev;
  if (wide >= 2 * cus) return launch_cfg<RA_BF16_NW, 1, 2>(a, s);
  const int64_t groups = (int64_t)((a.c + 32 * QB_SEL - 1) / (32 * QB_SEL)) * a.BH * a.n_dev;
  if (groups <= 2 * cus && triangular_rounds(a)) return launch_cfg<2, 4, 1>(a, s);
  if (groups <= 4 * cus) return launch_cfg<2, 4, 2>(a, s);
  if (groups <= 12 * cus) return launch_cfg<2, 2, 2>(a, s);
  return launch_cfg<4, 1, 3>(a, s);
}

}  // namespace ra
