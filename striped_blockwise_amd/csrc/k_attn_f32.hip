// Float32 blockwise attention: the exact-arithmetic path for float32 inputs (small head dims,
// correctness-sized problems).  One wavefront owns 64 query rows, one row per lane, and streams
// 64-key K/V tiles through LDS.  Scores and the online softmax are plain fp32 VALU work.
//
// Per query row and ring round r (K/V block k = (p - r) mod P, Ring Attention review step 2),
// the round's GetMask class decides which keys count (Striped Attention review, "GetMask 函数"),
// and the running max m, normaliser l and unnormalised output acc follow the online-softmax
// recurrence (Ring Attention review, step 3).  Scores are kept in log2 units (the query is
// pre-multiplied by scale * log2(e)) so every exponential is one exp2.
#include "ra_internal.h"

namespace ra {
namespace {

constexpr int TQ = 64;   // query rows per workgroup (= lanes)
constexpr int TK = 64;   // keys per LDS tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

template <int D>
__global__ __launch_bounds__(64) void k_attn_f32(AttnArgs a) {
  __shared__ float4 sk[TK * D / 4];
  __shared__ float4 sv[TK * D / 4];

  const int lane = threadIdx.x;
  const int c = a.c;
  const int nqt = (c + TQ - 1) / TQ;
  const int bh = blockIdx.x % a.BH;
  const int rest = blockIdx.x / a.BH;
  const int dev = rest % a.n_dev;
  const int qt = nqt - 1 - rest / a.n_dev;
  const int p = a.p_begin + dev;
  const int q0 = qt * TQ;
  const int y = q0 + lane;                                 // local query row of this lane
  const int q_last = min(c, q0 + TQ) - 1;                  // last in-range row of the tile

  const float* qp = (const float*)a.q + bh * a.q_bh_stride + dev * a.q_dev_stride;
  const int64_t rstride = (int64_t)a.row_step * D;        // elements between rows of a block
  float qv[D];
  const float qs = a.scale * LOG2E;
  if (y < c) {
#pragma unroll
    for (int j = 0; j < D; ++j) qv[j] = qp[y * rstride + j] * qs;
  } else {
#pragma unroll
    for (int j = 0; j < D; ++j) qv[j] = 0.f;
  }
  float acc[D];
#pragma unroll
  for (int j = 0; j < D; ++j) acc[j] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int ntk_all = (c + TK - 1) / TK;
  for (int rr = 0; rr < a.r_count; ++rr) {
    const int r = a.r_begin + rr;
    const int k = ring_block(p, r, a.P);
    const int mode = round_mode(a.layout, a.causal, p, k);
    const int delta = mode == MODE_STRICT ? 1 : 0;
    const int ntk = visited_tiles(mode, q_last, ntk_all, TK);

    const float* kp = (const float*)a.k + bh * a.kv_bh_stride + (int64_t)(k - a.kv_base) * a.kv_blk_stride;
    const float* vp = (const float*)a.v + bh * a.kv_bh_stride + (int64_t)(k - a.kv_base) * a.kv_blk_stride;
    uint64_t n_full = 0, n_diag = 0, pairs = 0;
    for (int t = 0; t < ntk; ++t) {
      const int x0 = t * TK;
      const int x_last = min(c, x0 + TK) - 1;
      __syncthreads();                                     // previous tile fully consumed
      for (int i = lane; i < TK * D / 4; i += 64) {
        const int row = x0 + i / (D / 4);
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
        sk[i] = row < c ? reinterpret_cast<const float4*>(kp + row * rstride)[i % (D / 4)] : z;
        sv[i] = row < c ? reinterpret_cast<const float4*>(vp + row * rstride)[i % (D / 4)] : z;
      }
      __syncthreads();
      // tile class on its in-range part (same for every lane of the workgroup)
      const bool full = mode == MODE_FULL || x_last <= q0 - delta;
      const bool skip = mode != MODE_FULL && x0 > q_last - delta;
      if (skip) continue;
      if (full) ++n_full; else ++n_diag;
      const float* K = reinterpret_cast<const float*>(sk);
      const float* V = reinterpret_cast<const float*>(sv);
      for (int j = 0; j < TK; ++j) {
        const int x = x0 + j;
        const bool vis = y < c && x < c && (mode == MODE_FULL || x <= y - delta);
        if (!vis) continue;
        ++pairs;
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) s = fmaf(qv[e], K[j * D + e], s);
        if (s > m) {                                        // new running max: rescale
          const float alpha = __builtin_amdgcn_exp2f(m - s);  // m = -inf -> 0
          l *= alpha;
#pragma unroll
          for (int e = 0; e < D; ++e) acc[e] *= alpha;
          m = s;
        }
        const float pj = __builtin_amdgcn_exp2f(s - m);
        l += pj;
#pragma unroll
        for (int e = 0; e < D; ++e) acc[e] = fmaf(pj, V[j * D + e], acc[e]);
      }
    }
    if (a.stats) {
      // pairs: per lane; reduce over the wavefront
      unsigned long long tot = pairs;
      for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off);
      if (lane == 0) {
        ra_round_stats_t* st = a.stats_single ? a.stats : a.stats + ((int64_t)p * a.P + r);
        const uint64_t tiles = (uint64_t)ntk_all;          // this query tile's row of the grid
        atomicAdd((unsigned long long*)&st->unmasked_pairs, tot);
        atomicAdd((unsigned long long*)&st->tiles_full, (unsigned long long)n_full);
        atomicAdd((unsigned long long*)&st->tiles_diag, (unsigned long long)n_diag);
        atomicAdd((unsigned long long*)&st->tiles_skipped,
                  (unsigned long long)(tiles - n_full - n_diag));
      }
    }
  }

  if (y < c) {
    const bool live = !(l <= 0.f);        // NaN (from NaN inputs) propagates to O and LSE
    const float inv = live ? 1.f / l : 0.f;
    const int64_t oel = bh * a.o_bh_stride + dev * a.o_dev_stride + y * rstride;
    if (a.o_f32) {
      float* op = (float*)a.o + oel;
#pragma unroll
      for (int e = 0; e < D; ++e) op[e] = acc[e] * inv;
    } else {
      __bf16* op = (__bf16*)a.o + oel;
#pragma unroll
      for (int e = 0; e < D; ++e) op[e] = (__bf16)(acc[e] * inv);
    }
    if (a.lse) a.lse[bh * a.lse_bh_stride + dev * a.lse_dev_stride + (int64_t)y * a.row_step] = live ? (m + __log2f(l)) * LN2 : -INFINITY;
  }
}

}  // namespace

bool attn_f32_supported(int64_t d) { return d == 32 || d == 64 || d == 128; }
void attn_f32_tile(int* tq, int* tk) { *tq = TQ; *tk = TK; }

hipError_t launch_attn_f32(const AttnArgs& a, int d, hipStream_t s) {
  const int64_t blocks = (int64_t)((a.c + TQ - 1) / TQ) * a.BH * a.n_dev;
  if (blocks * 64 >= (1ll << 32)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks);
  switch (d) {
    case 32: hipLaunchKernelGGL(k_attn_f32<32>, grid, dim3(64), 0, s, a); break;
    case 64: hipLaunchKernelGGL(k_attn_f32<64>, grid, dim3(64), 0, s, a); break;
    case 128: hipLaunchKernelGGL(k_attn_f32<128>, grid, dim3(64), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ra
