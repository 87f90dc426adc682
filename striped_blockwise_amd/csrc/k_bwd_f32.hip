// Float32 backward of blockwise attention: the exact-arithmetic path for float32 inputs (small
// head dims, correctness-sized problems).  Plain fp32 VALU work, one row per lane.
//
// Gradients of O = softmax(S + C) V, S = Q K^T * scale (Striped Attention review, "核心公式";
// Ring Attention review, step 3), pair by pair with the forward's log-sum-exp L:
// P = exp(S + C - L), dS = P * (dP - D) with dP = dO V^T and D = rowsum(O * dO).  The GetMask
// class of each (query device, K/V block) pair decides which pairs count (Striped Attention
// review, "GetMask 函数").
//   k_bwd_dq_f32   one query row per lane; K/V tiles of the given rounds through LDS;
//                  dQ = scale * sum_x dS[y, x] K[x].
//   k_bwd_dkv_f32  one key row per lane; Q / dO / L / D tiles of every query device through
//                  LDS; dV = sum_y P[y, x] dO[y], dK = scale * sum_y dS[y, x] Q[y].
#include "ra_internal.h"

namespace ra {
namespace {

constexpr int TR = 64;   // stationary rows per workgroup (= lanes)
constexpr int TS = 64;   // streamed rows per LDS tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_BIG = -1e30f;   // clamp for L = -inf: such a row has no visible pair

template <int D>
__global__ __launch_bounds__(64) void k_bwd_dq_f32(BwdArgs a) {
  __shared__ float sk[TS * D];
  __shared__ float sv[TS * D];

  const int lane = threadIdx.x;
  const int c = a.c;
  const int bh = blockIdx.x % a.BH;
  const int rest = blockIdx.x / a.BH;
  const int dev = rest % a.n_dev;
  const int qt = rest / a.n_dev;
  const int p = a.p_begin + dev;
  const int q0 = qt * TR;
  const int y = q0 + lane;
  const int q_last = min(c, q0 + TR) - 1;

  const float cs = a.scale * LOG2E;
  const int64_t rstride = (int64_t)a.row_step * D;        // elements between rows of a block
  float qv[D], dov[D], dq[D];
  float nl = 0.f, dl = 0.f;
  if (y < c) {
    const float* qp = (const float*)a.q + bh * a.q_bh_stride + dev * a.q_dev_stride + y * rstride;
    const float* dop = (const float*)a.dout + bh * a.do_bh_stride + dev * a.do_dev_stride + y * rstride;
#pragma unroll
    for (int j = 0; j < D; ++j) { qv[j] = qp[j] * cs; dov[j] = dop[j]; }
    const int64_t ro = bh * a.row_bh_stride + dev * a.row_dev_stride + (int64_t)y * a.row_step;
    nl = -fmaxf(a.lse[ro], NEG_BIG) * LOG2E;
    dl = a.delta[ro];
  } else {
#pragma unroll
    for (int j = 0; j < D; ++j) { qv[j] = 0.f; dov[j] = 0.f; }
  }
#pragma unroll
  for (int j = 0; j < D; ++j) dq[j] = 0.f;

  const int ntk_all = (c + TS - 1) / TS;
  for (int rr = 0; rr < a.r_count; ++rr) {
    const int r = a.r_begin + rr;
    const int k = ring_block(p, r, a.P);
    const int mode = round_mode(a.layout, a.causal, p, k);
    const int delta = mode == MODE_STRICT ? 1 : 0;
    int ntk = ntk_all;
    if (mode == MODE_SKIP) ntk = 0;
    else if (mode != MODE_FULL) ntk = q_last - delta < 0 ? 0 : min(ntk_all, (q_last - delta) / TS + 1);
    const int64_t kvo = bh * a.kv_bh_stride + (int64_t)(k - a.kv_base) * a.kv_blk_stride;
    const float* kp = (const float*)a.k + kvo;
    const float* vp = (const float*)a.v + kvo;
    for (int t = 0; t < ntk; ++t) {
      const int x0 = t * TS;
      __syncthreads();
      for (int i = lane; i < TS * D; i += 64) {
        const int row = x0 + i / D;
        sk[i] = row < c ? kp[row * rstride + i % D] : 0.f;
        sv[i] = row < c ? vp[row * rstride + i % D] : 0.f;
      }
      __syncthreads();
      for (int j = 0; j < TS; ++j) {
        const int x = x0 + j;
        const bool vis = y < c && x < c && (mode == MODE_FULL || x <= y - delta);
        if (!vis) continue;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) {
          s = fmaf(qv[e], sk[j * D + e], s);
          dp = fmaf(dov[e], sv[j * D + e], dp);
        }
        const float ds = __builtin_amdgcn_exp2f(s + nl) * (dp - dl);
#pragma unroll
        for (int e = 0; e < D; ++e) dq[e] = fmaf(ds, sk[j * D + e], dq[e]);
      }
    }
  }
  if (y < c) {
    float* out = a.dq + bh * a.dq_bh_stride + dev * a.dq_dev_stride + y * rstride;
#pragma unroll
    for (int e = 0; e < D; ++e) out[e] = dq[e] * a.scale + (a.accumulate ? out[e] : 0.f);
  }
}

template <int D>
__global__ __launch_bounds__(64) void k_bwd_dkv_f32(BwdArgs a) {
  __shared__ float sq[TS * D];
  __shared__ float so[TS * D];
  __shared__ float sl[TS];
  __shared__ float sd[TS];

  const int lane = threadIdx.x;
  const int c = a.c;
  const int bh = blockIdx.x % a.BH;
  const int rest = blockIdx.x / a.BH;
  const int kvi = rest % a.n_kv;
  const int kt = rest / a.n_kv;
  const int kblk = a.kv_base + kvi;
  const int x0 = kt * TR;
  const int x = x0 + lane;

  const float cs = a.scale * LOG2E;
  float kv[D], vv[D], dk[D], dv[D];
  const int64_t rstride = (int64_t)a.row_step * D;        // elements between rows of a block
  const int64_t kvo = bh * a.kv_bh_stride + (int64_t)kvi * a.kv_blk_stride + x * rstride;
#pragma unroll
  for (int j = 0; j < D; ++j) {
    kv[j] = x < c ? ((const float*)a.k)[kvo + j] * cs : 0.f;
    vv[j] = x < c ? ((const float*)a.v)[kvo + j] : 0.f;
    dk[j] = 0.f;
    dv[j] = 0.f;
  }

  const int ntq = (c + TS - 1) / TS;
  for (int di = 0; di < a.n_dev; ++di) {
    const int p = a.p_begin + di;
    const int mode = round_mode(a.layout, a.causal, p, kblk);
    const int delta = mode == MODE_STRICT ? 1 : 0;
    if (mode == MODE_SKIP) continue;
    const int t0 = mode == MODE_FULL ? 0 : (x0 + delta) / TS;
    const float* qp = (const float*)a.q + bh * a.q_bh_stride + di * a.q_dev_stride;
    const float* dop = (const float*)a.dout + bh * a.do_bh_stride + di * a.do_dev_stride;
    const float* lp = a.lse + bh * a.row_bh_stride + di * a.row_dev_stride;
    const float* dp_ = a.delta + bh * a.row_bh_stride + di * a.row_dev_stride;
    for (int t = t0; t < ntq; ++t) {
      const int y0 = t * TS;
      __syncthreads();
      for (int i = lane; i < TS * D; i += 64) {
        const int row = y0 + i / D;
        sq[i] = row < c ? qp[row * rstride + i % D] : 0.f;
        so[i] = row < c ? dop[row * rstride + i % D] : 0.f;
      }
      {
        const int row = y0 + lane;
        sl[lane] = row < c ? -fmaxf(lp[(int64_t)row * a.row_step], NEG_BIG) * LOG2E : 0.f;
        sd[lane] = row < c ? dp_[(int64_t)row * a.row_step] : 0.f;
      }
      __syncthreads();
      for (int j = 0; j < TS; ++j) {
        const int yy = y0 + j;
        const bool vis = x < c && yy < c && (mode == MODE_FULL || x <= yy - delta);
        if (!vis) continue;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) {
          s = fmaf(sq[j * D + e], kv[e], s);
          dp = fmaf(so[j * D + e], vv[e], dp);
        }
        const float pr = __builtin_amdgcn_exp2f(s + sl[j]);
        const float ds = pr * (dp - sd[j]);
#pragma unroll
        for (int e = 0; e < D; ++e) {
          dv[e] = fmaf(pr, so[j * D + e], dv[e]);
          dk[e] = fmaf(ds, sq[j * D + e], dk[e]);
        }
      }
    }
  }
  if (x < c) {
    const int64_t ro = bh * a.dkv_bh_stride + (int64_t)kvi * a.dkv_blk_stride + x * rstride;
#pragma unroll
    for (int e = 0; e < D; ++e) {
      a.dk[ro + e] = dk[e] * a.scale + (a.accumulate ? a.dk[ro + e] : 0.f);
      a.dv[ro + e] = dv[e] + (a.accumulate ? a.dv[ro + e] : 0.f);
    }
  }
}

template <int D>
hipError_t launch_d(const BwdArgs& a, bool dq, bool dkv, hipStream_t s) {
  const int64_t ntile = (a.c + TR - 1) / TR;
  if (dkv) {
    const int64_t blocks = ntile * a.BH * a.n_kv;
    if (blocks * 64 >= (1ll << 32)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_bwd_dkv_f32<D>, dim3((unsigned)blocks), dim3(64), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dq) {
    const int64_t blocks = ntile * a.BH * a.n_dev;
    if (blocks * 64 >= (1ll << 32)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_bwd_dq_f32<D>, dim3((unsigned)blocks), dim3(64), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

bool bwd_f32_supported(int64_t d) { return d == 32 || d == 64 || d == 128; }

hipError_t launch_bwd_f32(const BwdArgs& a, int d, bool dq, bool dkv, hipStream_t s) {
  switch (d) {
    case 32: return launch_d<32>(a, dq, dkv, s);
    case 64: return launch_d<64>(a, dq, dkv, s);
    case 128: return launch_d<128>(a, dq, dkv, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ra
