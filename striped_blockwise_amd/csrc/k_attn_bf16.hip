// bf16 blockwise attention on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), head dim 128.
//
// What one workgroup computes: NW wavefronts x QW query rows of device p's Q block, against
// the K/V blocks of the ring rounds it is given (Ring Attention review, step 2: round r brings
// the block of device (p - r) mod P), folding each round in with the online softmax (step 3).
// Masks follow the GetMask procedures of the Striped Attention review ("GetMask 函数"), applied
// per tile: a tile with no visible pair is skipped ("分块与分瓦片"), a tile with every pair
// visible runs unmasked, and only tiles that straddle the diagonal pay for an element mask.
//
// Data flow per 64-key tile:
//   HBM --(16 B per lane, coalesced)--> registers --> LDS (K row-major, V transposed), double
//   buffered so the next tile's global loads are in flight while this tile computes.
//   S^T = K Q^T on MFMA: A = K rows from LDS, B = the wave's Q columns held in registers.
//   In this orientation each lane owns one query column, so row max / row sum are in-lane
//   reductions plus one v_permlane32_swap with the other half of the wavefront.
//   P = exp2(S * scale * log2e - m) in fp32, rounded to bf16 (round-to-nearest-even).
//   O^T += V^T P^T on MFMA: A = V^T from LDS, B = P straight from the score registers (the MFMA
//   contraction index is permuted consistently on both operands, so no register shuffles).
// The output accumulator O^T keeps one query per lane too, so the online-softmax rescale is a
// per-lane multiply.
#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;          // head dim
constexpr int TK = 64;          // keys per tile
constexpr int NW = 4;           // wavefronts per workgroup
constexpr int NT = NW * 64;     // threads per workgroup
constexpr int KS_BYTES = TK * D * 2;       // K tile in LDS
constexpr int VS_BYTES = TK * D * 2;       // V^T tile in LDS
constexpr int STAGE_BYTES = KS_BYTES + VS_BYTES;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

static_assert(NT == 256, "loader mapping assumes 256 threads");

// ---- LDS layouts ------------------------------------------------------------------------------
// K tile: row = key (0..63), 256 B per row = 16 chunks of 16 B; chunk index XOR (row & 15) so
// that the 32 rows one MFMA operand read touches spread over all banks.
__device__ inline int k_off(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }

// V^T tile: row = head-dim index d (0..127), 64 keys x 2 B = 128 B per row = 8 chunks of 16 B.
// Keys are stored in MFMA-operand order: inside each group of 16 keys the order is
// [0-3, 8-11, 4-7, 12-15], so lane half h reads its 8 keys {4h..4h+3, 8+4h..8+4h+3} as one
// 16-byte chunk.  Chunk index XOR a hash of d keeps both the operand reads (32 consecutive d)
// and the transposing writes (d spaced by 8) spread over the banks.
__device__ inline int vt_swz(int d) { return (d & 7) ^ ((d >> 3) & 7); }
__device__ inline int vt_off(int d, int chunk8, int within_bytes) {
  return d * 128 + ((chunk8 ^ vt_swz(d)) << 4) + within_bytes;
}

struct KVRegs {
  u32x4 k[4];
  u32x4 v[4];
};

// Global -> registers for tile starting at key x0.  Thread t loads K rows x0 + t/16 + 16 i
// (16-byte chunk t % 16) and V rows x0 + 4 (t/16) + i (same chunk): 256 threads x 4 x 16 B per
// tensor.  Rows at or past c read as zeros.
__device__ inline void load_tile(KVRegs& R, const __bf16* kp, const __bf16* vp, int x0, int c,
                                 int tid) {
  const int ch = tid & 15;
  const int g = tid >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rk = x0 + g + 16 * i;
    const int rv = x0 + 4 * g + i;
    R.k[i] = rk < c ? *reinterpret_cast<const u32x4*>(kp + (int64_t)rk * D + ch * 8) : u32x4{0, 0, 0, 0};
    R.v[i] = rv < c ? *reinterpret_cast<const u32x4*>(vp + (int64_t)rv * D + ch * 8) : u32x4{0, 0, 0, 0};
  }
}

// Registers -> LDS stage.  K rows go straight in; V is transposed: each thread holds the same
// 8 head-dim values of 4 consecutive keys and writes, per head-dim index, those 4 keys (8 B).
__device__ inline void store_tile(char* stage, const KVRegs& R, int tid) {
  char* ks = stage;
  char* vs = stage + KS_BYTES;
  const int ch = tid & 15;
  const int g = tid >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = g + 16 * i;
    *reinterpret_cast<u32x4*>(ks + k_off(row, ch)) = R.k[i];
  }
  // keys 4g..4g+3 -> operand order position: group g/4 of 16, quad q = g % 4
  const int quad = g & 3;
  const int chunk8 = 2 * (g >> 2) + (quad & 1);
  const int within = (quad >> 1) * 8;     // bytes: 4 keys x 2 B
#pragma unroll
  for (int j = 0; j < 4; ++j) {           // dword j of the chunk = head-dim pair (2j, 2j+1)
    const uint32_t a0 = R.v[0][j], a1 = R.v[1][j], a2 = R.v[2][j], a3 = R.v[3][j];
    const u32x2 lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
    const u32x2 hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
    const int d0 = ch * 8 + 2 * j;
    *reinterpret_cast<u32x2*>(vs + vt_off(d0, chunk8, within)) = lo;
    *reinterpret_cast<u32x2*>(vs + vt_off(d0 + 1, chunk8, within)) = hi;
  }
}

__device__ inline float pair_max(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ inline float pair_sum(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Key index (within the 32-key MFMA block) held by accumulator register r in lane half h.
__device__ inline int acc_row(int r, int h) { return (r >> 2) * 8 + h * 4 + (r & 3); }

template <int QB, bool STATS>
__global__ __launch_bounds__(NT, (QB == 1 ? 2 : 1)) void k_attn_bf16(AttnArgs a) {
  constexpr int QW = 32 * QB;            // query rows per wavefront
  constexpr int TQ = NW * QW;            // query rows per workgroup
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int c = a.c;

  const int nqt = (c + TQ - 1) / TQ;
  const int bh = blockIdx.x % a.BH;      // heads fastest: block i runs on XCD i % 8, so the
  const int rest = blockIdx.x / a.BH;    // q-tiles of one head share that XCD's L2
  const int dev = rest % a.n_dev;
  const int qt = nqt - 1 - rest / a.n_dev;   // most causal work first
  const int p = a.p_begin + dev;
  const int q_wg0 = qt * TQ;
  const int q_wg_last = min(c, q_wg0 + TQ) - 1;
  const int qw0 = q_wg0 + wave * QW;
  const int qw_last = min(c, qw0 + QW) - 1;  // < qw0 when the wave has no rows
  const bool wave_live = qw0 < c;

  // ---- Q columns for the B operand: lane holds row qw0 + 32 qb + l32, head-dim chunk
  //      16 dk + 8 hh .. +7 for every dk.
  const __bf16* qp = (const __bf16*)a.q + bh * a.q_bh_stride + dev * a.q_dev_stride;
  bf16x8 qf[QB][8];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw0 + qb * 32 + l32;
#pragma unroll
    for (int dk = 0; dk < 8; ++dk) {
      qf[qb][dk] = row < c ? *reinterpret_cast<const bf16x8*>(qp + (int64_t)row * D + dk * 16 + hh * 8)
                           : bf16x8{};
    }
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

  const int ntk_all = (c + TK - 1) / TK;
  for (int rr = 0; rr < a.r_count; ++rr) {
    const int r = a.r_begin + rr;
    const int k = ring_block(p, r, a.P);
    const int mode = round_mode(a.layout, a.causal, p, k);
    const int delta = mode == MODE_STRICT ? 1 : 0;
    // tiles this workgroup must visit: up to the last one with a visible pair for its rows
    int ntk = ntk_all;
    if (mode == MODE_SKIP) ntk = 0;
    else if (mode != MODE_FULL) ntk = (q_wg_last - delta < 0) ? 0 : min(ntk_all, (q_wg_last - delta) / TK + 1);

    const int64_t kvo = bh * a.kv_bh_stride + (int64_t)(k - a.kv_base) * a.kv_blk_stride;
    const __bf16* kp = (const __bf16*)a.k + kvo;
    const __bf16* vp = (const __bf16*)a.v + kvo;

    uint64_t st_full = 0, st_diag = 0, st_pairs_uniform = 0;
    uint32_t st_pairs_lane = 0;

    if (ntk > 0) {
      KVRegs R;
      load_tile(R, kp, vp, 0, c, tid);
      store_tile(smem, R, tid);
      __syncthreads();
      for (int t = 0; t < ntk; ++t) {
        const bool more = t + 1 < ntk;
        if (more) load_tile(R, kp, vp, (t + 1) * TK, c, tid);
        const char* stage = smem + (t & 1) * STAGE_BYTES;
        const int x0 = t * TK;
        const int x_last = min(c, x0 + TK) - 1;
        // this wavefront's tile class (on its in-range part)
        const bool skip = !wave_live || (mode != MODE_FULL && x0 > qw_last - delta);
        const bool full = mode == MODE_FULL || x_last <= qw0 - delta;
        if (!skip) {
          const bool need_mask = !full || (x0 + TK > c);
          if (STATS) {
            if (full) { ++st_full; st_pairs_uniform += (uint64_t)(qw_last - qw0 + 1) * (x_last - x0 + 1); }
            else ++st_diag;
          }
          // ---- S^T = K Q^T
          f32x16 s[QB][2];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) { s[qb][0] = f32x16{}; s[qb][1] = f32x16{}; }
#pragma unroll
          for (int dk = 0; dk < 8; ++dk) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              const bf16x8 ka = *reinterpret_cast<const bf16x8*>(stage + k_off(32 * b + l32, 2 * dk + hh));
#pragma unroll
              for (int qb = 0; qb < QB; ++qb)
                s[qb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[qb][dk], s[qb][b], 0, 0, 0);
            }
          }
          // ---- mask (diagonal tiles, ragged edge)
          if (need_mask) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              const int y = qw0 + qb * 32 + l32;
#pragma unroll
              for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int rg = 0; rg < 16; ++rg) {
                  const int x = x0 + 32 * b + acc_row(rg, hh);
                  const bool vis = x < c && (mode == MODE_FULL || x <= y - delta);
                  if (STATS && !full) st_pairs_lane += (vis && y < c) ? 1u : 0u;
                  if (!vis) s[qb][b][rg] = -INFINITY;
                }
            }
          }
          // ---- online softmax; P packed to bf16 in MFMA B-operand order
          bf16x8 pf[QB][4];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            float mx = s[qb][0][0];
#pragma unroll
            for (int rg = 1; rg < 16; ++rg) mx = fmaxf(mx, s[qb][0][rg]);
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) mx = fmaxf(mx, s[qb][1][rg]);
            mx = pair_max(mx);
            const float m_new = fmaxf(m[qb], mx * cs);
            const float ref = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m[qb] - ref);
            m[qb] = m_new;
            float rs = 0.f;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
#pragma unroll
              for (int half = 0; half < 2; ++half) {
                bf16x8 pk;
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                  const float p0 = __builtin_amdgcn_exp2f(fmaf(s[qb][b][half * 8 + e], cs, -ref));
                  const float p1 = __builtin_amdgcn_exp2f(fmaf(s[qb][b][half * 8 + e + 1], cs, -ref));
                  rs += p0 + p1;
                  const bf16x2 pp = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
                  pk[e] = pp[0];
                  pk[e + 1] = pp[1];
                }
                pf[qb][2 * b + half] = pk;
              }
            }
            l[qb] = l[qb] * alpha + rs;
#pragma unroll
            for (int db = 0; db < 4; ++db) o[qb][db] *= alpha;
          }
          // ---- O^T += V^T P^T
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int db = 0; db < 4; ++db) {
              const int dd = 32 * db + l32;
              const bf16x8 va = *reinterpret_cast<const bf16x8*>(stage + KS_BYTES + vt_off(dd, 2 * ks + hh, 0));
#pragma unroll
              for (int qb = 0; qb < QB; ++qb)
                o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[qb][ks], o[qb][db], 0, 0, 0);
            }
          }
        }
        if (more) store_tile(smem + ((t + 1) & 1) * STAGE_BYTES, R, tid);
        __syncthreads();
      }
    }

    if (STATS && wave_live) {
      unsigned long long pairs = st_pairs_lane;
      for (int off = 32; off > 0; off >>= 1) pairs += __shfl_xor(pairs, off);
      if (lane == 0) {
        ra_round_stats_t* st = a.stats_single ? a.stats : a.stats + ((int64_t)p * a.P + r);
        atomicAdd((unsigned long long*)&st->unmasked_pairs, (unsigned long long)(pairs + st_pairs_uniform));
        atomicAdd((unsigned long long*)&st->tiles_full, (unsigned long long)st_full);
        atomicAdd((unsigned long long*)&st->tiles_diag, (unsigned long long)st_diag);
        atomicAdd((unsigned long long*)&st->tiles_skipped,
                  (unsigned long long)(ntk_all - st_full - st_diag));
      }
    }
  }

  // ---- finalize: O = acc / l, LSE = ln(2) * (m + log2 l); rows with no key: 0 and -inf
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = pair_sum(l[qb]);
    const bool live = lt > 0.f;
    const float inv = live ? 1.f / lt : 0.f;
    const int y = qw0 + qb * 32 + l32;
    if (y < c) {
      const int64_t orow = (int64_t)dev * c + y;
      if (a.o_f32) {
        float* op = (float*)a.o + bh * a.o_bh_stride + orow * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 w = make_float4(o[qb][db][4 * g] * inv, o[qb][db][4 * g + 1] * inv,
                                         o[qb][db][4 * g + 2] * inv, o[qb][db][4 * g + 3] * inv);
            *reinterpret_cast<float4*>(op + 32 * db + 8 * g + 4 * hh) = w;
          }
      } else {
        __bf16* op = (__bf16*)a.o + bh * a.o_bh_stride + orow * D;
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
        a.lse[bh * a.lse_bh_stride + orow] = live ? (m[qb] + __log2f(lt)) * LN2 : -INFINITY;
    }
  }
}

constexpr int QB_DEFAULT = 1;

}  // namespace

bool attn_bf16_supported(int64_t d) { return d == D; }
void attn_bf16_tile(int* tq, int* tk) { *tq = 32 * QB_DEFAULT; *tk = TK; }

hipError_t launch_attn_bf16(const AttnArgs& a, int d, hipStream_t s) {
  if (d != D) return hipErrorInvalidValue;
  constexpr int TQ = NW * 32 * QB_DEFAULT;
  const int64_t blocks = (int64_t)((a.c + TQ - 1) / TQ) * a.BH * a.n_dev;
  if (blocks * NT >= (1ll << 32)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks);
  if (a.stats)
    hipLaunchKernelGGL((k_attn_bf16<QB_DEFAULT, true>), grid, dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((k_attn_bf16<QB_DEFAULT, false>), grid, dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace ra
