// bf16 backward of blockwise attention on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), head
// dim 128.
//
// The pages give only the forward; its gradients follow from O = softmax(S + C) V with
// S = Q K^T * scale (Striped Attention review, "核心公式"; Ring Attention review, step 3).  With
// the forward's log-sum-exp L of each query row, a (query block, K/V block) pair has the exact
// probabilities P = exp(S + C - L) on its own, so the ring's rounds are independent and each
// pair contributes
//     dV += P^T dO,   dP = dO V^T,   dS = P * (dP - D),   dQ += scale dS K,   dK += scale dS^T Q,
// with D = rowsum(O * dO).  The same GetMask classes as the forward decide which pairs count
// (Striped Attention review, "GetMask 函数") and which tiles are skipped or run unmasked.
//
// Two kernels, neither with atomics, so every gradient is a deterministic sum:
//   dQ kernel   query rows stationary (32 per wavefront), the K/V tiles of the given rounds
//               streamed through LDS as in the forward:
//                 S^T = K Q^T, dP^T = V dO^T (A = K / V rows from LDS, B = Q / dO in registers),
//                 dS^T = P^T * (dP^T - D) in registers (one query per lane),
//                 dQ^T += K^T dS^T (A = K read transposed from the same LDS tile).
//   dK/dV kernel key rows stationary (32 per wavefront), the query tiles of every device that
//               meets the block streamed through LDS (Q, dO, L, D):
//                 S = Q K^T, dP = dO V^T (A = Q / dO rows from LDS, B = K / V in registers),
//                 dS = P * (dP - D) in registers (one key per lane),
//                 dV^T += dO^T P, dK^T += Q^T dS (A = dO / Q read transposed).
// A tile read both row-wise and transposed uses the t_swz chunk mask, conflict-free for both.
// Every row-indexed tensor is addressed with the same row step: consecutive rows of a block, or
// rows P apart for a striped block of a token-order tensor (row y of block k is token y P + k).
// Rows past the end of a block arrive in LDS as zeros: a zero query row with L = D = 0 gives
// P = 1 and dS = 0 and adds nothing; zero key rows are masked in the dQ kernel and only reach
// their own (unwritten) dK/dV columns in the dK/dV kernel.
#include <type_traits>

#include "bf16_tile.h"
#include "ra_internal.h"

namespace ra {
namespace {

using namespace bf16t;

#ifndef RA_BWD_DQ_NW
#define RA_BWD_DQ_NW 8           // dQ kernel: wavefronts per workgroup (one workgroup per CU)
#endif
#ifndef RA_BWD_DQ_PAIR
#define RA_BWD_DQ_PAIR 1         // dQ kernel: paired query tiles for wide launches with triangular rounds
#endif
#ifndef RA_BWD_DKV_NW
#define RA_BWD_DKV_NW 4          // dK/dV kernel: wavefronts per workgroup (two per CU)
#endif
constexpr int WR = 32;           // stationary rows per wavefront
constexpr int TS = 32;           // streamed rows per tile
constexpr int TILE = TS * ROWB;  // bytes of one streamed tile (8 KB)
// dQ kernel: clamp for L = -inf (a row that sees no key), so that P stays 0 on its masked keys.
// The dK/dV kernel needs none: its accumulator starts at -L / scale (+inf for such a row) and
// the element mask sets every masked pair to -inf, which such a row's pairs all are.
constexpr float NEG_BIG = -1e30f;
#ifndef RA_BWD_DKV_NOWAIT
#define RA_BWD_DKV_NOWAIT 1      // dK/dV kernel: LDS reads without the compiler's wait for the next tile's DMA
#endif

// Block -> (stream, tile).  Blocks are dispatched round-robin over the 8 XCDs; with xcd_major
// XCD x takes streams x, x+8, ... one after another, all tiles of a stream together, so the
// workgroups on one XCD share the streamed blocks in its L2.  `reverse` puts the last tile
// first (dQ: late query rows see the most keys; dK/dV: early key rows meet the most queries).
__device__ __forceinline__ void map_block(int xcd_major, int nstream, int ntile, bool reverse,
                                          int& stream, int& tile) {
  if (xcd_major) {
    const int x = blockIdx.x & 7;
    const int sq = blockIdx.x >> 3;
    stream = (sq / ntile) * 8 + x;
    tile = sq % ntile;
  } else {
    stream = blockIdx.x % nstream;
    tile = blockIdx.x / nstream;
  }
  if (reverse) tile = ntile - 1 - tile;
}

__device__ __forceinline__ bf16x8 load_row8(const __bf16* p, bool ok) {
  return ok ? *reinterpret_cast<const bf16x8*>(p) : bf16x8{};
}

// Packs f(r) for r = 8 ks .. 8 ks + 7 into bf16 (round to nearest even): the B operand of
// contraction step ks.
template <typename F>
__device__ __forceinline__ bf16x8 pack8(F&& f, int ks) {
  bf16x8 out;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const bf16x2 pp = __builtin_convertvector(f32x2{f(8 * ks + e), f(8 * ks + e + 1)}, bf16x2);
    out[e] = pp[0];
    out[e + 1] = pp[1];
  }
  return out;
}

// Writes (or adds) acc * mul for the lane's stationary row: rows d = 32 db + acc_row(r, h).
__device__ __forceinline__ void store_rows(float* row, const f32x16 (&acc)[4], float mul, int hh, bool add) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float4* dst = reinterpret_cast<float4*>(row + 32 * db + 8 * g + 4 * hh);
      float4 w = make_float4(acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul, acc[db][4 * g + 2] * mul,
                             acc[db][4 * g + 3] * mul);
      if (add) {
        const float4 o = *dst;
        w.x += o.x; w.y += o.y; w.z += o.z; w.w += o.w;
      }
      *dst = w;
    }
}

// ------------------------------------------------------------------------------- dQ kernel
// NR row groups of WR query rows times NS key splits (NR NS wavefronts).  With NS > 1, split s
// of a row group takes the K/V tiles s, s + NS, ... of every round into LDS stages of its own
// (shared by its NR wavefronts), and the splits' dQ partial sums are added up through LDS at the
// end: grids too small to fill the chip then spread each row group's sweep over its keys.
//
// PAIR (NS == 1, launches whose rounds are all causal-triangular): workgroup i of a stream takes
// the query tiles i and nqt - 1 - i and, round by round, sweeps the round's K/V block for the
// first tile and then for the second, adding each (round, tile) partial into dq as it goes.
// Under triangular masks the two tiles see few and many keys, so every paired workgroup does
// about the same work in every round: the workgroups resident at one time stay in the same
// round and read the same K/V block, instead of drifting over all P blocks (whose union does
// not fit the caches).  The query tile's Q, dO, L and D are reloaded for each sweep.
template <int NR, int NS, bool PAIR>
__global__ __launch_bounds__(NR * NS * 64, 2) void k_bwd_dq_bf16(BwdArgs a) {
  static_assert(!PAIR || NS == 1, "paired query tiles: one key split");
  constexpr int WG_ROWS = NR * WR;      // stationary rows per workgroup
  constexpr int SPLIT_BYTES = 4 * TILE;                       // K0 K1 V0 V1 of one split
  constexpr int SLOT = 64 * 64 * 4;                           // one wavefront's dQ partial
  constexpr int LDS_BYTES = NS * SPLIT_BYTES > (NS - 1) * NR * SLOT ? NS * SPLIT_BYTES : (NS - 1) * NR * SLOT;
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = NS == 1 ? wave_u : wave_u % NR;   // row group
  const int s = NS == 1 ? 0 : wave_u / NR;        // key split
  const int split_base = s * SPLIT_BYTES;
  char* const sb = smem + split_base;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int c = a.c;

  const int nqt = (c + WG_ROWS - 1) / WG_ROWS;
  int stream, unit;
  // unpaired: heaviest query tile first (late rows see the most keys); paired: equal units
  map_block(a.xcd_major, a.BH * a.n_dev, PAIR ? pair_count(nqt) : nqt, !PAIR, stream, unit);
  const int bh = stream % a.BH;
  const int dev = stream / a.BH;
  const int p = a.p_begin + dev;

  int k_row[8], v_row[8], k_tr[4][2];
#pragma unroll
  for (int dk = 0; dk < 8; ++dk) {
    k_row[dk] = split_base + a_rowwise_off<SWZ_T>(lane, dk);
    v_row[dk] = split_base + a_rowwise_off<SWZ_K>(lane, dk);
  }
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) k_tr[db][sec] = split_base + a_tr_off<SWZ_T>(lane, db, sec);
  unsigned kdma[DmaShape<NR, TS>::PER_WAVE], vdma[DmaShape<NR, TS>::PER_WAVE];
  dma_init<NR, TS>(kdma, SWZ_T, g, lane, a.row_step);
  dma_init<NR, TS>(vdma, SWZ_K, g, lane, a.row_step);
  // Split workgroups read K^T without the compiler's wait for every LDS DMA in flight (their
  // own waits cover the tile), as the forward's small shapes do.
  constexpr bool TR_NOWAIT = NS > 1;
  const int64_t rstride = (int64_t)a.row_step * D;   // elements between rows of a block
  const float cs = a.scale * LOG2E;

  // The current query tile: its rows, and this lane's row of Q and dO (B operands, head dims
  // 16 dk + 8 hh .. +7), -L log2(e) and D.
  int qt = 0, q_wg_last = -1, qw0 = 0, qw_last = -1, y = 0;
  bool wave_live = false;
  bf16x8 qf[8], df[8];
  float nl = 0.f, dl = 0.f;
  auto set_tile = [&](int t) {
    qt = t;
    q_wg_last = min(c, qt * WG_ROWS + WG_ROWS) - 1;
    qw0 = qt * WG_ROWS + g * WR;
    qw_last = min(c, qw0 + WR) - 1;
    wave_live = qw0 < c;
    y = qw0 + l32;
  };
  auto load_tile = [&]() {
    const __bf16* qp = (const __bf16*)a.q + bh * a.q_bh_stride + dev * a.q_dev_stride + y * rstride + hh * 8;
    const __bf16* dop = (const __bf16*)a.dout + bh * a.do_bh_stride + dev * a.do_dev_stride + y * rstride + hh * 8;
#pragma unroll
    for (int dk = 0; dk < 8; ++dk) {
      qf[dk] = load_row8(qp + dk * 16, y < c);
      df[dk] = load_row8(dop + dk * 16, y < c);
    }
    nl = 0.f;
    dl = 0.f;
    if (y < c) {
      const int64_t ro = bh * a.row_bh_stride + dev * a.row_dev_stride + (int64_t)y * a.row_step;
      nl = -fmaxf(a.lse[ro], NEG_BIG) * LOG2E;
      dl = a.delta[ro];
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};

  const int ntk_all = (c + TS - 1) / TS;
  // Key tiles that the current query tile visits in ring round r_begin + rr.
  auto round_tiles = [&](int rr) {
    return visited_tiles(round_mode(a.layout, a.causal, p, ring_block(p, a.r_begin + rr, a.P)), q_wg_last,
                         ntk_all, TS);
  };
  // The current query tile against the K/V block of round r_begin + rr, added into acc.
  auto sweep_round = [&](int rr) __attribute__((always_inline)) {
    const int r = a.r_begin + rr;
    const int k = ring_block(p, r, a.P);
    const int mode = round_mode(a.layout, a.causal, p, k);
    const int delta = mode == MODE_STRICT ? 1 : 0;
    const int ntk = visited_tiles(mode, q_wg_last, ntk_all, TS);
    if (ntk == 0) return;

    const int64_t kvo = bh * a.kv_bh_stride + (int64_t)(k - a.kv_base) * a.kv_blk_stride;
    const char* kblk = (const char*)((const __bf16*)a.k + kvo);
    const char* vblk = (const char*)((const __bf16*)a.v + kvo);

    // 0: no visible pair for this wave; 1: all visible; 2: element mask (diagonal, or the
    // tile runs past the end of the block)
    auto tile_class = [&](int t) -> int {
      const int x0 = t * TS;
      if (!wave_live || (mode != MODE_FULL && x0 > qw_last - delta)) return 0;
      const bool full = (mode == MODE_FULL || x0 + TS - 1 <= qw0 - delta) && x0 + TS <= c;
      return full ? 1 : 2;
    };

    auto compute = [&](const char* ks_, const char* vs_, int t, bool masked) __attribute__((always_inline)) {
      f32x16 s = f32x16{}, dp = f32x16{};
      {
        bf16x8 kf[8];
#pragma unroll
        for (int dk = 0; dk < 8; ++dk) kf[dk] = *reinterpret_cast<const bf16x8*>(ks_ + k_row[dk]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dk = 0; dk < 8; ++dk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[dk], qf[dk], s, 0, 0, 0);
      }
      {
        bf16x8 vf[8];
#pragma unroll
        for (int dk = 0; dk < 8; ++dk) vf[dk] = *reinterpret_cast<const bf16x8*>(vs_ + v_row[dk]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dk = 0; dk < 8; ++dk) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dk], df[dk], dp, 0, 0, 0);
      }
      if (masked) {
        const int x0 = t * TS;
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) {
          const int x = x0 + acc_row(rg, hh);
          const bool vis = x < c && (mode == MODE_FULL || x <= y - delta);
          s[rg] = vis ? s[rg] : -INFINITY;
        }
      }
      auto ds = [&](int rg) __attribute__((always_inline)) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(s[rg], cs, nl));
        return pr * (dp[rg] - dl);
      };
      const bf16x8 ds0 = pack8(ds, 0);
      const bf16x8 ds1 = pack8(ds, 1);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 k0 = TR_NOWAIT ? read_a_tr_nowait(ks_, k_tr[db][0], k_tr[db][1])
                                    : read_a_tr(ks_, k_tr[db][0], k_tr[db][1]);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, ds0, acc[db], 0, 0, 0);
        const bf16x8 k1 = TR_NOWAIT ? read_a_tr_nowait(ks_ + 16 * ROWB, k_tr[db][0], k_tr[db][1])
                                    : read_a_tr(ks_ + 16 * ROWB, k_tr[db][0], k_tr[db][1]);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, ds1, acc[db], 0, 0, 0);
      }
    };

    if constexpr (NS == 1) {
      dma_issue<NR, TS>(kdma, kblk, smem, 0, c, a.row_step, g);
      dma_issue<NR, TS>(vdma, vblk, smem + 2 * TILE, 0, c, a.row_step, g);
      auto iter = [&](int t, auto stage_c) __attribute__((always_inline)) {
        constexpr int S = decltype(stage_c)::value;
        wait_dma_and_barrier();                       // tile t landed; the other stage is free
        if (t + 1 < ntk) {
          dma_issue<NR, TS>(kdma, kblk, smem + (1 - S) * TILE, (t + 1) * TS, c, a.row_step, g);
          dma_issue<NR, TS>(vdma, vblk, smem + (3 - S) * TILE, (t + 1) * TS, c, a.row_step, g);
        }
        const int cls = tile_class(t);
        if (cls) compute(smem + S * TILE, smem + (2 + S) * TILE, t, cls == 2);
      };
      int t = 0;
      for (; t + 1 < ntk; t += 2) {
        iter(t, std::integral_constant<int, 0>{});
        iter(t + 1, std::integral_constant<int, 1>{});
      }
      if (t < ntk) iter(t, std::integral_constant<int, 0>{});
      __syncthreads();                                // LDS stages free for the next round
    } else {
      // This split's tiles: j = 0 .. my_n - 1 is tile j NS + s, in stage j & 1.  Wavefronts that
      // share tiles (NR > 1) run the workgroup's iteration count in lock-step; a lone wavefront
      // runs its own.  Only owned tiles are fetched: a split may own none in a round.
      const int my_n = split_count(ntk, s, NS);
      const int nit = NR > 1 ? (ntk + NS - 1) / NS : my_n;
      auto issue = [&](int j, int stage) __attribute__((always_inline)) {
        const int x0 = split_tile(j, s, NS) * TS;
        dma_issue<NR, TS>(kdma, kblk, sb + stage * TILE, x0, c, a.row_step, g);
        dma_issue<NR, TS>(vdma, vblk, sb + (2 + stage) * TILE, x0, c, a.row_step, g);
      };
      if (my_n > 0) issue(0, 0);
      auto iter = [&](int j, auto stage_c) __attribute__((always_inline)) {
        constexpr int S = decltype(stage_c)::value;
        vm_wait<0>();                                 // my tile j landed; with NR > 1 the
        if (NR > 1) __syncthreads();                  // barrier also frees the other stage
        if (j + 1 < my_n) issue(j + 1, 1 - S);
        if (NR == 1 || j < my_n) {
          const int t = split_tile(j, s, NS);
          const int cls = tile_class(t);
          if (cls) compute(smem + S * TILE, smem + (2 + S) * TILE, t, cls == 2);
        }
      };
      int j = 0;
      for (; j + 1 < nit; j += 2) {
        iter(j, std::integral_constant<int, 0>{});
        iter(j + 1, std::integral_constant<int, 1>{});
      }
      if (j < nit) iter(j, std::integral_constant<int, 0>{});
      if (NR > 1) __syncthreads();                    // LDS stages free for the next round
    }
  };

  if constexpr (PAIR) {
    // Per round: the first query tile's sweep, then the second's; each (round, tile) partial
    // is scaled and added into dq (the first one written, unless accumulating).
    const int pair[2] = {unit, pair_second(unit, nqt)};
    const int nseg = pair[1] != pair[0] ? 2 : 1;
    for (int rr = 0; rr < a.r_count; ++rr) {
      for (int sg = 0; sg < nseg; ++sg) {
        set_tile(pair[sg]);
        const bool first = rr == 0 && a.accumulate == 0;
        const bool work = round_tiles(rr) > 0;
        if (!work && !first) continue;
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
        if (work) {                                     // (no key in the first round: zeros)
          load_tile();
          sweep_round(rr);
        }
        if (y < c)
          store_rows(a.dq + bh * a.dq_bh_stride + dev * a.dq_dev_stride + y * rstride, acc, a.scale, hh, !first);
      }
    }
    return;
  }

  set_tile(unit);
  load_tile();
  for (int rr = 0; rr < a.r_count; ++rr) sweep_round(rr);

  // Key splits: splits 1 .. NS-1 hand their dQ partial sums to split 0 of their row group
  // through LDS; split 0 adds them up and stores.
  if constexpr (NS > 1) {
    __syncthreads();                                  // every split is done with its stages
    if (s > 0) {
      float4* const slot = reinterpret_cast<float4*>(smem + ((s - 1) * NR + g) * SLOT);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          slot[(db * 4 + q4) * 64 + lane] =
              make_float4(acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2], acc[db][4 * q4 + 3]);
    }
    __syncthreads();
    if (s > 0) return;
#pragma unroll 1
    for (int s2 = 1; s2 < NS; ++s2) {
      const float4* const slot = reinterpret_cast<const float4*>(smem + ((s2 - 1) * NR + g) * SLOT);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 w = slot[(db * 4 + q4) * 64 + lane];
          acc[db][4 * q4] += w.x;
          acc[db][4 * q4 + 1] += w.y;
          acc[db][4 * q4 + 2] += w.z;
          acc[db][4 * q4 + 3] += w.w;
        }
    }
  }

  if (y < c)
    store_rows(a.dq + bh * a.dq_bh_stride + dev * a.dq_dev_stride + y * rstride, acc, a.scale, hh, a.accumulate != 0);
}

// ---------------------------------------------------------------------------- dK/dV kernel
// LDS per stage: Q tile, dO tile, then 32 floats of L and 32 of D.
constexpr int RS_BYTES = 2 * TS * 4;

__global__ __launch_bounds__(RA_BWD_DKV_NW * 64, 2) void k_bwd_dkv_bf16(BwdArgs a) {
  constexpr int NW = RA_BWD_DKV_NW;
  constexpr int WG_ROWS = NW * WR;      // stationary rows per workgroup
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE + 2 * RS_BYTES];  // Q0 Q1 O0 O1 RS0 RS1

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int c = a.c;

  const int nkt = (c + WG_ROWS - 1) / WG_ROWS;
  int stream, kt;
  map_block(a.xcd_major, a.BH * a.n_kv, nkt, false, stream, kt);
  const int bh = stream % a.BH;
  const int kvi = stream / a.BH;
  const int kblk = a.kv_base + kvi;
  const int x_wg0 = kt * WG_ROWS;
  const int kw0 = x_wg0 + wave_u * WR;
  const int kw_last = min(c, kw0 + WR) - 1;
  const bool wave_live = kw0 < c;
  const int x = kw0 + l32;

  // LDS offsets of step 0 / column block 0; the others are these XOR constants (tr_xor)
  const int rw0 = a_rowwise_off<SWZ_T>(lane, 0);
  const int tr0 = a_tr_off<SWZ_T>(lane, 0, 0);
  unsigned dma[DmaShape<NW, TS>::PER_WAVE];
  dma_init<NW, TS>(dma, SWZ_T, wave_u, lane, a.row_step);

  // B operands: this lane's key row of K and V
  const int64_t rstride = (int64_t)a.row_step * D;   // elements between rows of a block
  const int64_t kvo = bh * a.kv_bh_stride + (int64_t)kvi * a.kv_blk_stride + x * rstride + hh * 8;
  bf16x8 kf[8], vf[8];
#pragma unroll
  for (int dk = 0; dk < 8; ++dk) {
    kf[dk] = load_row8((const __bf16*)a.k + kvo + dk * 16, x < c);
    vf[dk] = load_row8((const __bf16*)a.v + kvo + dk * 16, x < c);
  }
  const float cs = a.scale * LOG2E;
  const float nis = -1.0f / a.scale;

  f32x16 dka[4], dva[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) { dka[db] = f32x16{}; dva[db] = f32x16{}; }

  const int ntq = (c + TS - 1) / TS;
  for (int di = 0; di < a.n_dev; ++di) {
    const int p = a.p_begin + di;
    const int mode = round_mode(a.layout, a.causal, p, kblk);
    const int delta = mode == MODE_STRICT ? 1 : 0;
    if (mode == MODE_SKIP) continue;
    // first query tile holding a row y >= x_wg0 + delta (a visible pair for some key here)
    const int t0 = first_query_tile(mode, x_wg0, TS);
    if (t0 >= ntq) continue;

    const char* qblk = (const char*)((const __bf16*)a.q + bh * a.q_bh_stride + di * a.q_dev_stride);
    const char* oblk = (const char*)((const __bf16*)a.dout + bh * a.do_bh_stride + di * a.do_dev_stride);
    const float* lblk = a.lse + bh * a.row_bh_stride + di * a.row_dev_stride;
    const float* dblk = a.delta + bh * a.row_bh_stride + di * a.row_dev_stride;

    auto issue = [&](int t, int S) __attribute__((always_inline)) {
      const int y0 = t * TS;
      dma_issue<NW, TS>(dma, qblk, smem + S * TILE, y0, c, a.row_step, wave_u);
      dma_issue<NW, TS>(dma, oblk, smem + (2 + S) * TILE, y0, c, a.row_step, wave_u);
      if (wave_u == 0 && lane < 32) {
        // lane i < 32 copies L and D of row y0 + i to bytes 4 i of the stage's L and D areas;
        // the descriptors end after the block's last row, so rows past it read as 0
        char* rs = smem + 4 * TILE + S * RS_BYTES;
        const unsigned last = (unsigned)(min(c - y0, TS) - 1);
        const int bytes = (int)((last * (unsigned)a.row_step + 1) * 4);
        const int64_t base = (int64_t)y0 * a.row_step;
        const unsigned off = (unsigned)lane * (unsigned)a.row_step * 4;
        const __amdgpu_buffer_rsrc_t lr = __builtin_amdgcn_make_buffer_rsrc((void*)(lblk + base), 0, bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t dr = __builtin_amdgcn_make_buffer_rsrc((void*)(dblk + base), 0, bytes, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(lr, (lds_void*)rs, 4, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(dr, (lds_void*)(rs + TS * 4), 4, off, 0, 0, 0);
      }
    };

    // 0: no visible pair for this wave; 1: all visible; 2: element mask
    auto tile_class = [&](int t) -> int {
      const int y0 = t * TS;
      const int y_last = min(c, y0 + TS) - 1;
      if (!wave_live || (mode != MODE_FULL && kw0 > y_last - delta)) return 0;
      return (mode == MODE_FULL || kw_last <= y0 - delta) ? 1 : 2;
    };

    auto compute = [&](const char* qs_, const char* os_, const char* rs_, int t, bool masked) __attribute__((always_inline)) {
      // S = Q K^T, then P and dV^T += dO^T P before dP is formed, so that S, P and dP are never
      // all live at once; A fragments come from LDS four at a time.
      // LDS offsets as (lane base) ^ (constant): two registers instead of sixteen.  The empty asm
      // makes the bases opaque so that the XORs are formed here, not hoisted out of the loop.
      int rwb = (int)(qs_ - smem) + rw0, trb = (int)(qs_ - smem) + tr0;
      asm volatile("" : "+v"(rwb), "+v"(trb));
      const int dq_o = (int)(os_ - qs_);
      // The tile's DMA was waited for at the barrier; the next tile's, issued after it, fills
      // the other stage, so these reads need not wait for it (RA_BWD_DKV_NOWAIT).
      constexpr bool NW_ = RA_BWD_DKV_NOWAIT != 0;
      auto rd16 = [&](int off) -> bf16x8 {
        return NW_ ? lds_read_nowait<bf16x8>(smem, off) : *reinterpret_cast<const bf16x8*>(smem + off);
      };
      auto rdtr = [&](int lo, int hi) -> bf16x8 {
        return NW_ ? read_a_tr_nowait(smem, lo, hi) : read_a_tr(smem, lo, hi);
      };
      auto rd4f = [&](const char* p) -> float4 {
        return NW_ ? lds_read_nowait<float4>(p, 0) : *reinterpret_cast<const float4*>(p);
      };
      auto q_tra = [&](int ks, int db) { return rdtr((trb + ks * 16 * ROWB) ^ tr_xor(db, 0), (trb + ks * 16 * ROWB) ^ tr_xor(db, 1)); };
      auto o_tra = [&](int ks, int db) { return rdtr((trb + dq_o + ks * 16 * ROWB) ^ tr_xor(db, 0), (trb + dq_o + ks * 16 * ROWB) ^ tr_xor(db, 1)); };
      // The accumulator starts at -L / scale for its row (acc_row(rg, hh): four runs of 4
      // consecutive rows), so that the products leave S - L / scale, and the exp2 argument is one
      // multiply by scale log2(e).
      f32x16 s;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 l4 = rd4f(rs_ + (8 * g + 4 * hh) * 4);
        s[4 * g] = l4.x * nis;
        s[4 * g + 1] = l4.y * nis;
        s[4 * g + 2] = l4.z * nis;
        s[4 * g + 3] = l4.w * nis;
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        bf16x8 qa[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) qa[j] = rd16(rwb ^ ((4 * h2 + j) << 5));
#pragma unroll
        for (int j = 0; j < 4; ++j) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[j], kf[4 * h2 + j], s, 0, 0, 0);
      }
      if (masked) {
        const int y0 = t * TS;
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) {
          const int yy = y0 + acc_row(rg, hh);
          const bool vis = mode == MODE_FULL || x <= yy - delta;
          s[rg] = vis ? s[rg] : -INFINITY;
        }
      }
      // P = exp2((S - L / scale) scale log2(e)).  A row that sees no key (L = -inf) has +inf
      // here, but it has no visible pair, so every tile it meets takes the element mask above
      // (or is skipped) and its pairs are -inf: P = 0.
#pragma unroll
      for (int rg = 0; rg < 16; ++rg) s[rg] = __builtin_amdgcn_exp2f(s[rg] * cs);
      {
        const bf16x8 p0 = pack8([&](int r) { return s[r]; }, 0);
        const bf16x8 p1 = pack8([&](int r) { return s[r]; }, 1);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 o0 = o_tra(0, db);
          const bf16x8 o1 = o_tra(1, db);
          dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o0, p0, dva[db], 0, 0, 0);
          dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o1, p1, dva[db], 0, 0, 0);
        }
      }
      f32x16 dp = f32x16{};
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        bf16x8 oa[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) oa[j] = rd16((rwb + dq_o) ^ ((4 * h2 + j) << 5));
#pragma unroll
        for (int j = 0; j < 4; ++j) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[j], vf[4 * h2 + j], dp, 0, 0, 0);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 d4 = rd4f(rs_ + TS * 4 + (8 * g + 4 * hh) * 4);
        const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) dp[4 * g + j] = s[4 * g + j] * (dp[4 * g + j] - dv[j]);
      }
      const bf16x8 s0 = pack8([&](int r) { return dp[r]; }, 0);
      const bf16x8 s1 = pack8([&](int r) { return dp[r]; }, 1);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 q0 = q_tra(0, db);
        const bf16x8 q1 = q_tra(1, db);
        dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q0, s0, dka[db], 0, 0, 0);
        dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q1, s1, dka[db], 0, 0, 0);
      }
    };

    issue(t0, 0);
    auto iter = [&](int t, auto stage_c) __attribute__((always_inline)) {
      constexpr int S = decltype(stage_c)::value;
      wait_dma_and_barrier();
      if (t + 1 < ntq) issue(t + 1, 1 - S);
      const int cls = tile_class(t);
      if (cls) compute(smem + S * TILE, smem + (2 + S) * TILE, smem + 4 * TILE + S * RS_BYTES, t, cls == 2);
    };
    int t = t0;
    for (; t + 1 < ntq; t += 2) {
      iter(t, std::integral_constant<int, 0>{});
      iter(t + 1, std::integral_constant<int, 1>{});
    }
    if (t < ntq) iter(t, std::integral_constant<int, 0>{});
    __syncthreads();
  }

  if (x < c) {
    const int64_t ro = bh * a.dkv_bh_stride + (int64_t)kvi * a.dkv_blk_stride + x * rstride;
    store_rows(a.dk + ro, dka, a.scale, hh, a.accumulate != 0);
    store_rows(a.dv + ro, dva, 1.0f, hh, a.accumulate != 0);
  }
}

}  // namespace

bool bwd_bf16_supported(int64_t d) { return d == D; }

namespace {

template <int NR, int NS, bool PAIR = false>
hipError_t launch_dq(const BwdArgs& a, hipStream_t s) {
  constexpr int rows = NR * WR, nt = NR * NS * 64;
  const int64_t nstream = (int64_t)a.BH * a.n_dev;
  const int64_t nqt = (a.c + rows - 1) / rows;
  const int64_t blocks = (PAIR ? pair_count((int)nqt) : nqt) * nstream;
  if (blocks * nt >= (1ll << 32)) return hipErrorInvalidConfiguration;
  BwdArgs b = a;
  b.xcd_major = nstream % 8 == 0 ? 1 : 0;
  hipLaunchKernelGGL((k_bwd_dq_bf16<NR, NS, PAIR>), dim3((unsigned)blocks), dim3(nt), 0, s, b);
  return hipGetLastError();
}

// True when every round of the launch is causal-triangular for every launched device: causal,
// and no contiguous round brings a block from an earlier device (k < p), which every query row
// sees whole.
bool all_rounds_triangular(const BwdArgs& a) {
  if (!a.causal) return false;
  if (a.layout != RA_CONTIGUOUS) return true;
  for (int dv = 0; dv < a.n_dev; ++dv)
    for (int i = 0; i < a.r_count; ++i) {
      const int p = a.p_begin + dv;
      if (round_mode(a.layout, a.causal, p, ring_block(p, a.r_begin + i, a.P)) == MODE_FULL) return false;
    }
  return true;
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, int d, bool dq, bool dkv, hipStream_t s) {
  if (d != D) return hipErrorInvalidValue;
  if (dkv) {
    constexpr int rows = RA_BWD_DKV_NW * WR, nt = RA_BWD_DKV_NW * 64;
    const int64_t nstream = (int64_t)a.BH * a.n_kv;
    const int64_t blocks = (a.c + rows - 1) / rows * nstream;
    if (blocks * nt >= (1ll << 32)) return hipErrorInvalidConfiguration;
    BwdArgs b = a;
    b.xcd_major = nstream % 8 == 0 ? 1 : 0;
    hipLaunchKernelGGL(k_bwd_dkv_bf16, dim3((unsigned)blocks), dim3(nt), 0, s, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dq) {
    // dQ workgroup shape by grid size: 8-wave workgroups when there are at least two per CU;
    // below that, with G = 32-row groups in the launch and C compute units, 2 row groups x 4 key
    // splits up to G = 4 C, else 4 x 2 (each split with its own two K/V stages in LDS).
    const int64_t cus = cu_count();
    constexpr int WIDE_ROWS = RA_BWD_DQ_NW * WR;
    const int64_t wide = (int64_t)((a.c + WIDE_ROWS - 1) / WIDE_ROWS) * a.BH * a.n_dev;
    if (wide >= 2 * cus)
      return RA_BWD_DQ_PAIR && all_rounds_triangular(a) ? launch_dq<RA_BWD_DQ_NW, 1, true>(a, s)
                                                        : launch_dq<RA_BWD_DQ_NW, 1>(a, s);
    const int64_t groups = (int64_t)((a.c + WR - 1) / WR) * a.BH * a.n_dev;
    if (groups <= 4 * cus) return launch_dq<2, 4>(a, s);
    return launch_dq<4, 2>(a, s);
  }
  return hipSuccess;
}

}  // namespace ra
