// Row-movement and row-combination kernels: the striped permutation and the log-sum-exp merge.
// Both are HBM-bandwidth bound; each lane moves 16 bytes per access where the row allows it.
#include "ra_internal.h"

namespace ra {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------------
// Striped permutation (Striped Attention review, "分区策略对比" / "位置编码处理"): token t goes
// to device t mod P, slot t / P, i.e. layout row pi(t) = (t mod P) * c + t / P.  Grid-stride
// over destination chunks so that writes are sequential; the rows being read are the
// scattered side.  VEC is the bytes one lane moves (16 or 4).
template <int VEC>
__global__ __launch_bounds__(256) void k_permute(const char* __restrict__ src,
                                                 char* __restrict__ dst, uint64_t total,
                                                 uint32_t chunks_per_row, uint32_t n,
                                                 uint32_t P, uint32_t c, int inverse,
                                                 uint64_t row_bytes) {
  typedef typename std::conditional<VEC == 16, u32x4, uint32_t>::type T;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t e = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const uint64_t row_lin = e / chunks_per_row;          // bh * n + destination row
    const uint32_t ch = (uint32_t)(e - row_lin * chunks_per_row);
    const uint64_t bh = row_lin / n;
    const uint32_t drow = (uint32_t)(row_lin - bh * n);
    uint32_t srow;
    if (inverse) {
      srow = (drow % P) * c + drow / P;                   // dst[t] = src[pi(t)]
    } else {
      // dst[pi(t)] = src[t]: destination row (dev, slot) holds token slot * P + dev
      const uint32_t dev = drow / c;
      srow = (drow - dev * c) * P + dev;
    }
    const T* s = reinterpret_cast<const T*>(src + (bh * n + srow) * row_bytes) + ch;
    T* d = reinterpret_cast<T*>(dst + row_lin * row_bytes) + ch;
    *d = *s;
  }
}

// ---------------------------------------------------------------------------------------------
// Log-sum-exp merge ("Computing Attention Weights in Sequence Parallelism": the denominator is
// a sum of per-node sums): L = ln(e^La + e^Lb), O = e^(La-L) Oa + e^(Lb-L) Ob, in place on the
// accumulator.  Every row is handled by LPR lanes of one wavefront (LPR a power of two <= 64),
// so all reads of lse_acc[row] complete before the one lane that rewrites it stores.
template <int LPR>
__global__ __launch_bounds__(256) void k_merge(float* __restrict__ o_acc, float* __restrict__ lse_acc,
                                               const float* __restrict__ o_part,
                                               const float* __restrict__ lse_part,
                                               int64_t rows, int64_t d) {
  constexpr int RPW = 64 / LPR;                           // rows per wavefront pass
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR;
  const int li = lane % LPR;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const bool vec4 = (d & 3) == 0;
  for (int64_t row0 = wave * RPW; row0 < rows; row0 += nwaves * RPW) {
    const int64_t row = row0 + sub;
    if (row >= rows) continue;
    const float la = lse_acc[row];
    const float lb = lse_part[row];
    const float mx = fmaxf(la, lb);
    float wa = 0.f, wb = 0.f, L = -INFINITY;
    if (mx != -INFINITY) {
      const float ea = expf(la - mx);
      const float eb = expf(lb - mx);
      const float sum = ea + eb;
      L = mx + logf(sum);
      wa = ea / sum;
      wb = eb / sum;
    }
    float* oa = o_acc + row * d;
    const float* ob = o_part + row * d;
    if (vec4) {
      for (int64_t j = li; j < (d >> 2); j += LPR) {
        float4 a = reinterpret_cast<float4*>(oa)[j];
        const float4 b = reinterpret_cast<const float4*>(ob)[j];
        a.x = wa * a.x + wb * b.x;
        a.y = wa * a.y + wb * b.y;
        a.z = wa * a.z + wb * b.z;
        a.w = wa * a.w + wb * b.w;
        reinterpret_cast<float4*>(oa)[j] = a;
      }
    } else {
      for (int64_t j = li; j < d; j += LPR) oa[j] = wa * oa[j] + wb * ob[j];
    }
    if (li == 0) lse_acc[row] = L;
  }
}

// ---------------------------------------------------------------------------------------------
// Backward row term D_i = sum_e O_ie dO_ie (fp32 sums).  16 lanes of one wavefront per row, each
// taking groups of 4 consecutive elements (or single elements when d % 4 != 0).
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const __bf16* p) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}

template <typename TO, typename TD>
__global__ __launch_bounds__(256) void k_delta(const TO* __restrict__ o, const TD* __restrict__ dout,
                                               int64_t rows, int64_t d, float* __restrict__ delta) {
  constexpr int LPR = 16;
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR;
  const int li = lane % LPR;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const bool vec4 = (d & 3) == 0;
  for (int64_t row0 = wave * (64 / LPR); row0 < rows; row0 += nwaves * (64 / LPR)) {
    const int64_t row = row0 + sub;
    float acc = 0.f;
    if (row < rows) {
      const TO* orow = o + row * d;
      const TD* drow = dout + row * d;
      if (vec4) {
        for (int64_t j = 4 * li; j < d; j += 4 * LPR) {
          const float4 a = load4(orow + j);
          const float4 b = load4(drow + j);
          acc = fmaf(a.x, b.x, acc);
          acc = fmaf(a.y, b.y, acc);
          acc = fmaf(a.z, b.z, acc);
          acc = fmaf(a.w, b.w, acc);
        }
      } else {
        for (int64_t j = li; j < d; j += LPR) acc = fmaf((float)orow[j], (float)drow[j], acc);
      }
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (li == 0 && row < rows) delta[row] = acc;
  }
}

int grid_for(uint64_t work_items, int per_block) {
  uint64_t g = (work_items + per_block - 1) / per_block;
  const uint64_t cap = 256ull * 64;                       // plenty of waves for every CU
  if (g > cap) g = cap;
  return g < 1 ? 1 : (int)g;
}

}  // namespace

hipError_t launch_permute(const void* src, void* dst, int64_t BH, int64_t n, int64_t row_bytes,
                          int P, int inverse, hipStream_t s) {
  const uint32_t c = (uint32_t)(n / P);
  const bool v16 = (row_bytes % 16 == 0) && ((uintptr_t)src % 16 == 0) && ((uintptr_t)dst % 16 == 0);
  const int vec = v16 ? 16 : 4;
  const uint32_t cpr = (uint32_t)(row_bytes / vec);
  const uint64_t total = (uint64_t)BH * (uint64_t)n * cpr;
  const int grid = grid_for(total, 256 * 4);
  if (v16)
    hipLaunchKernelGGL(k_permute<16>, dim3(grid), dim3(256), 0, s, (const char*)src, (char*)dst,
                       total, cpr, (uint32_t)n, (uint32_t)P, c, inverse, (uint64_t)row_bytes);
  else
    hipLaunchKernelGGL(k_permute<4>, dim3(grid), dim3(256), 0, s, (const char*)src, (char*)dst,
                       total, cpr, (uint32_t)n, (uint32_t)P, c, inverse, (uint64_t)row_bytes);
  return hipGetLastError();
}

hipError_t launch_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                        int64_t rows, int64_t d, hipStream_t s) {
  const int64_t lanes_needed = (d % 4 == 0) ? d / 4 : d;
  int lpr = 1;
  while (lpr < lanes_needed && lpr < 64) lpr <<= 1;
  const uint64_t waves = (uint64_t)((rows + (64 / lpr) - 1) / (64 / lpr));
  const int grid = grid_for(waves * 64, 256);
#define RA_MERGE_CASE(L)                                                                       \
  case L:                                                                                      \
    hipLaunchKernelGGL(k_merge<L>, dim3(grid), dim3(256), 0, s, o_acc, lse_acc, o_part,        \
                       lse_part, rows, d);                                                     \
    break;
  switch (lpr) {
    RA_MERGE_CASE(1) RA_MERGE_CASE(2) RA_MERGE_CASE(4) RA_MERGE_CASE(8) RA_MERGE_CASE(16)
    RA_MERGE_CASE(32) RA_MERGE_CASE(64)
    default: return hipErrorInvalidValue;
  }
#undef RA_MERGE_CASE
  return hipGetLastError();
}

hipError_t launch_delta(const void* o, int o_f32, const void* dout, int do_f32, int64_t rows,
                        int64_t d, float* delta, hipStream_t s) {
  const int grid = grid_for((uint64_t)((rows + 3) / 4) * 64, 256);
#define RA_DELTA(TO, TD)                                                                        \
  hipLaunchKernelGGL((k_delta<TO, TD>), dim3(grid), dim3(256), 0, s, (const TO*)o, (const TD*)dout, \
                     rows, d, delta)
  if (o_f32 && do_f32) RA_DELTA(float, float);
  else if (o_f32) RA_DELTA(float, __bf16);
  else if (do_f32) RA_DELTA(__bf16, float);
  else RA_DELTA(__bf16, __bf16);
#undef RA_DELTA
  return hipGetLastError();
}

}  // namespace ra
