// Row-movement and row-combination kernels: the striped permutation (plain, and fused with the
// rotary embedding), the log-sum-exp merge and the backward's row term D.  All are
// HBM-bandwidth bound; each lane moves 16 bytes per access where the row allows it.
#include "ra_internal.h"

namespace ra {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

#ifndef RA_ROWS_NT
#define RA_ROWS_NT 1            // 1: streamed loads and stores marked non-temporal (merge, delta, RoPE)
#endif
#ifndef RA_MERGE_ROWS
#define RA_MERGE_ROWS 4         // merge rows in flight per lane group for d = 64 and 128 (1: generic kernel)
#endif
// Every byte these kernels move is touched once, so marking the accesses non-temporal keeps
// them from displacing useful lines in the caches.
template <typename V>
__device__ __forceinline__ V ld_stream(const V* p) {
  if (RA_ROWS_NT) return __builtin_nontemporal_load(p);
  return *p;
}
template <typename V>
__device__ __forceinline__ void st_stream(V v, V* p) {
  if (RA_ROWS_NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// ---------------------------------------------------------------------------------------------
// Striped permutation (Striped Attention review, "分区策略对比" / "位置编码处理"): token t goes
// to device t mod P, slot t / P, i.e. layout row pi(t) = (t mod P) * c + t / P.  Grid-stride
// over destination chunks so that writes are sequential; the rows being read are the
// scattered side.  VEC is the bytes one lane moves (16 or 4).  This general form serves rows
// that k_permute_rows below does not take (LSE values, position IDs, odd row sizes).
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

#ifndef RA_PERMUTE_IMPL
#define RA_PERMUTE_IMPL 2       // 0: element grid-stride kernel; 1: row kernel; 2: row kernel, non-temporal
#endif

// The same permutation, row by row, for rows of 16-byte chunks whose count divides 256: `lpr`
// lanes move one row, a block pass covers 256 / lpr rows, and each thread keeps RPT rows in
// flight.  One 32-bit division per row replaces the per-chunk 64-bit index arithmetic of
// k_permute.  blockIdx.y is the (b, h) matrix (looping when BH exceeds the grid's y range).
template <bool NTEMP>
__global__ __launch_bounds__(256) void k_permute_rows(const char* __restrict__ src, char* __restrict__ dst,
                                                      uint64_t BH, uint32_t n, uint32_t lpr, uint32_t P,
                                                      uint32_t c, int inverse, uint64_t row_bytes) {
  constexpr int RPT = 4;
  const uint32_t rpp = 256 / lpr;                         // rows per block pass
  const uint32_t r_in = threadIdx.x / lpr;
  const uint32_t ch = threadIdx.x - r_in * lpr;
  const uint32_t rows_per_block = rpp * RPT;
  for (uint64_t bh = blockIdx.y; bh < BH; bh += gridDim.y) {
    const char* sbase = src + bh * n * row_bytes;
    char* dbase = dst + bh * n * row_bytes;
    for (uint32_t r0 = blockIdx.x * rows_per_block; r0 < n; r0 += gridDim.x * rows_per_block) {
      u32x4 v[RPT];
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const uint32_t drow = r0 + k * rpp + r_in;
        if (drow < n) {
          uint32_t srow;
          if (inverse) {
            srow = (drow % P) * c + drow / P;             // dst[t] = src[pi(t)]
          } else {
            const uint32_t dev = drow / c;                // dst[pi(t)] = src[t]
            srow = (drow - dev * c) * P + dev;
          }
          const u32x4* sp = reinterpret_cast<const u32x4*>(sbase + (uint64_t)srow * row_bytes) + ch;
          v[k] = NTEMP ? __builtin_nontemporal_load(sp) : *sp;
        }
      }
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const uint32_t drow = r0 + k * rpp + r_in;
        if (drow < n) {
          u32x4* dp = reinterpret_cast<u32x4*>(dbase + (uint64_t)drow * row_bytes) + ch;
          if (NTEMP) __builtin_nontemporal_store(v[k], dp);
          else *dp = v[k];
        }
      }
    }
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
    if (la != la || lb != lb) wa = wb = L = la + lb;          // a NaN LSE on either side: NaN out
    float* oa = o_acc + row * d;
    const float* ob = o_part + row * d;
    if (vec4) {
      for (int64_t j = li; j < (d >> 2); j += LPR) {
        f32x4v a = ld_stream(reinterpret_cast<const f32x4v*>(oa) + j);
        const f32x4v b = ld_stream(reinterpret_cast<const f32x4v*>(ob) + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = wa * a[e] + wb * b[e];
        st_stream(a, reinterpret_cast<f32x4v*>(oa) + j);
      }
    } else {
      for (int64_t j = li; j < d; j += LPR) oa[j] = wa * oa[j] + wb * ob[j];
    }
    if (li == 0) lse_acc[row] = L;
  }
}

// The same merge for rows of exactly LPR float4s (d = 4 LPR, LPR a power of two <= 64): each
// lane owns one float4 of a row, and the loads of U row groups (both LSEs, both O slices) are
// all issued before any of them is used, so that U times more reads are in flight per lane.
template <int LPR, int U>
__global__ __launch_bounds__(256) void k_merge_v4(float* __restrict__ o_acc, float* __restrict__ lse_acc,
                                                  const float* __restrict__ o_part,
                                                  const float* __restrict__ lse_part, int64_t rows) {
  constexpr int RPW = 64 / LPR;                           // rows per wavefront and group
  constexpr int D = 4 * LPR;
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR;
  const int li = lane % LPR;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t base = wave * (RPW * U); base < rows; base += nwaves * (RPW * U)) {
    float la[U], lb[U];
    f32x4v a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = base + u * RPW + sub;
      la[u] = lb[u] = -INFINITY;
      a[u] = b[u] = f32x4v{};
      if (row < rows) {
        la[u] = lse_acc[row];
        lb[u] = lse_part[row];
        a[u] = ld_stream(reinterpret_cast<const f32x4v*>(o_acc + row * D) + li);
        b[u] = ld_stream(reinterpret_cast<const f32x4v*>(o_part + row * D) + li);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = base + u * RPW + sub;
      if (row >= rows) continue;
      const float mx = fmaxf(la[u], lb[u]);
      float wa = 0.f, wb = 0.f, L = -INFINITY;
      if (mx != -INFINITY) {
        const float ea = expf(la[u] - mx);
        const float eb = expf(lb[u] - mx);
        const float sum = ea + eb;
        L = mx + logf(sum);
        wa = ea / sum;
        wb = eb / sum;
      }
      if (la[u] != la[u] || lb[u] != lb[u]) wa = wb = L = la[u] + lb[u];   // NaN LSE: NaN out
      f32x4v r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = wa * a[u][e] + wb * b[u][e];
      st_stream(r, reinterpret_cast<f32x4v*>(o_acc + row * D) + li);
      if (li == 0) lse_acc[row] = L;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Backward row term D_i = sum_e O_ie dO_ie (fp32 sums).  16 lanes of one wavefront per row, each
// taking groups of 4 consecutive elements (or single elements when d % 4 != 0).
__device__ __forceinline__ float4 load4(const float* p) {
  const f32x4v v = ld_stream(reinterpret_cast<const f32x4v*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float4 load4(const __bf16* p) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 v = ld_stream(reinterpret_cast<const bf16x4*>(p));
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

// ---------------------------------------------------------------------------------------------
// Rotary position embedding fused with the striped permutation (Striped Attention review,
// "位置编码处理": RoPE must see the position IDs permuted like the tokens).  Pair i of a token at
// position m is rotated by m * base^(-2i/d) (RoFormer's rotary embedding; pairs (2i, 2i+1), or
// (i, i + d/2) with `half`).  One wavefront per token: each lane forms the cosine and sine of
// its pairs once, in fp64 (positions reach 10^6 and more, where an fp32 angle has lost its
// fraction), and applies them to the token's row in every (b, h) matrix.  The rotation is also
// done in fp64 and rounded once to fp32, then (for bf16) once more to bf16.
//   inverse == 0: dst[bh][pi(t)] = R(m_t) src[bh][t]
//   inverse != 0: dst[bh][t] = R(m_t)^T src[bh][pi(t)]   (the adjoint: gradients back through it)
__device__ __forceinline__ double load_elem(const float* p) { return (double)*p; }
__device__ __forceinline__ double load_elem(const __bf16* p) { return (double)(float)*p; }
__device__ __forceinline__ void store_elem(float* p, double v) { *p = (float)v; }
__device__ __forceinline__ void store_elem(__bf16* p, double v) { *p = (__bf16)(float)v; }

template <typename T>
__global__ __launch_bounds__(256) void k_rope_permute(const T* __restrict__ src, T* __restrict__ dst,
                                                      const int64_t* __restrict__ pos, int64_t BH,
                                                      uint32_t n, uint32_t d, uint32_t P, uint32_t c,
                                                      int striped, int inverse, int half, double base) {
  const int lane = threadIdx.x & 63;
  const uint64_t wave = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const uint64_t nwaves = ((uint64_t)gridDim.x * blockDim.x) >> 6;
  const uint32_t npairs = d / 2;
  for (uint64_t tt = wave; tt < n; tt += nwaves) {
    const uint32_t t = (uint32_t)tt;
    const uint32_t lrow = striped ? (t % P) * c + t / P : t;
    const uint32_t srow = inverse ? lrow : t;
    const uint32_t drow = inverse ? t : lrow;
    const double m = pos ? (double)pos[t] : (double)t;
    for (uint32_t i = lane; i < npairs; i += 64) {
      const double theta = pow(base, -2.0 * (double)i / (double)d);
      double sn, cs;
      sincos(m * theta, &sn, &cs);
      if (inverse) sn = -sn;
      const uint32_t ia = half ? i : 2 * i;
      const uint32_t ib = half ? i + npairs : 2 * i + 1;
      for (int64_t bh = 0; bh < BH; ++bh) {
        const T* s = src + ((uint64_t)bh * n + srow) * d;
        T* o = dst + ((uint64_t)bh * n + drow) * d;
        const double xa = load_elem(s + ia), xb = load_elem(s + ib);
        store_elem(o + ia, fma(xa, cs, -xb * sn));
        store_elem(o + ib, fma(xa, sn, xb * cs));
      }
    }
  }
}

// Vector form of k_rope_permute for head dims with 64 % (d / 8) == 0 (d = 8 .. 512, powers of
// two): a lane owns a unit of 4 pairs -- 8 consecutive elements (interleaved pairing) or 4 + 4
// elements d/2 apart (half pairing) -- moved with 16-byte (or 8-byte) accesses, and a wave
// covers 64 / (d / 8) rows of the token per step.  A lane forms its 4 cosines and sines once per
// token, as above in fp64.
template <int N, typename T> struct Vec;
template <> struct Vec<8, __bf16> { typedef __bf16 type __attribute__((ext_vector_type(8))); };
template <> struct Vec<4, __bf16> { typedef __bf16 type __attribute__((ext_vector_type(4))); };
template <> struct Vec<8, float> { typedef float type __attribute__((ext_vector_type(8))); };
template <> struct Vec<4, float> { typedef float type __attribute__((ext_vector_type(4))); };

template <int N, typename T>
__device__ __forceinline__ void load_n(const T* p, double (&v)[N]) {
  const typename Vec<N, T>::type x = ld_stream(reinterpret_cast<const typename Vec<N, T>::type*>(p));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = (double)(float)x[i];
}
template <int N, typename T>
__device__ __forceinline__ void store_n(T* p, const double (&v)[N]) {
  typename Vec<N, T>::type x;
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = (T)(float)v[i];
  st_stream(x, reinterpret_cast<typename Vec<N, T>::type*>(p));
}

template <typename T, bool HALF>
__global__ __launch_bounds__(256) void k_rope_permute_vec(const T* __restrict__ src, T* __restrict__ dst,
                                                          const int64_t* __restrict__ pos, int64_t BH,
                                                          uint32_t n, uint32_t d, uint32_t P, uint32_t c,
                                                          int striped, int inverse, double base) {
  const int lane = threadIdx.x & 63;
  const uint64_t wave = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const uint64_t nwaves = ((uint64_t)gridDim.x * blockDim.x) >> 6;
  const uint32_t units = d / 8;                    // units of 4 pairs per row
  const uint32_t rows_per_step = 64 / units;
  const uint32_t u = lane % units;
  const uint32_t rsub = lane / units;
  double theta[4];                                  // this lane's pairs 4u .. 4u+3
#pragma unroll
  for (int j = 0; j < 4; ++j) theta[j] = pow(base, -2.0 * (double)(4 * u + j) / (double)d);
  for (uint64_t tt = wave; tt < n; tt += nwaves) {
    const uint32_t t = (uint32_t)tt;
    const uint32_t lrow = striped ? (t % P) * c + t / P : t;
    const uint32_t srow = inverse ? lrow : t;
    const uint32_t drow = inverse ? t : lrow;
    const double m = pos ? (double)pos[t] : (double)t;
    double cs[4], sn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sincos(m * theta[j], &sn[j], &cs[j]);
      if (inverse) sn[j] = -sn[j];
    }
    // two (b, h) rows per step, both loaded before either is rotated
    for (int64_t bh0 = rsub; bh0 < BH; bh0 += 2 * (int64_t)rows_per_step) {
      const bool two = bh0 + rows_per_step < BH;
      const int64_t bh1 = two ? bh0 + rows_per_step : bh0;
      const T* s0 = src + ((uint64_t)bh0 * n + srow) * d;
      const T* s1 = src + ((uint64_t)bh1 * n + srow) * d;
      T* d0 = dst + ((uint64_t)bh0 * n + drow) * d;
      T* d1 = dst + ((uint64_t)bh1 * n + drow) * d;
      if (HALF) {
        double a0[4], b0[4], a1[4], b1[4], oa[4], ob[4];
        load_n<4>(s0 + 4 * u, a0);
        load_n<4>(s0 + d / 2 + 4 * u, b0);
        if (two) {
          load_n<4>(s1 + 4 * u, a1);
          load_n<4>(s1 + d / 2 + 4 * u, b1);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          oa[j] = fma(a0[j], cs[j], -b0[j] * sn[j]);
          ob[j] = fma(a0[j], sn[j], b0[j] * cs[j]);
        }
        store_n<4>(d0 + 4 * u, oa);
        store_n<4>(d0 + d / 2 + 4 * u, ob);
        if (two) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            oa[j] = fma(a1[j], cs[j], -b1[j] * sn[j]);
            ob[j] = fma(a1[j], sn[j], b1[j] * cs[j]);
          }
          store_n<4>(d1 + 4 * u, oa);
          store_n<4>(d1 + d / 2 + 4 * u, ob);
        }
      } else {
        double e0[8], e1[8], o[8];
        load_n<8>(s0 + 8 * u, e0);
        if (two) load_n<8>(s1 + 8 * u, e1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o[2 * j] = fma(e0[2 * j], cs[j], -e0[2 * j + 1] * sn[j]);
          o[2 * j + 1] = fma(e0[2 * j], sn[j], e0[2 * j + 1] * cs[j]);
        }
        store_n<8>(d0 + 8 * u, o);
        if (two) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            o[2 * j] = fma(e1[2 * j], cs[j], -e1[2 * j + 1] * sn[j]);
            o[2 * j + 1] = fma(e1[2 * j], sn[j], e1[2 * j + 1] * cs[j]);
          }
          store_n<8>(d1 + 8 * u, o);
        }
      }
    }
  }
}

int grid_for(uint64_t work_items, int per_block) {
  uint64_t g = (work_items + per_block - 1) / per_block;
  const uint64_t cap = 256ull * 64;                       // plenty of waves for every CU
  if (g > cap) g = cap;
  return g < 1 ? 1 : (int)g;
}

// Zero fill of n 64-bit words (the work counters that ra_forward overwrites).  A kernel rather
// than hipMemsetAsync, so that a caller may capture the call in a HIP graph.
__global__ __launch_bounds__(256) void k_zero_u64(uint64_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_zero_u64(uint64_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_zero_u64, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_permute(const void* src, void* dst, int64_t BH, int64_t n, int64_t row_bytes,
                          int P, int inverse, hipStream_t s) {
  const uint32_t c = (uint32_t)(n / P);
  const bool v16 = (row_bytes % 16 == 0) && ((uintptr_t)src % 16 == 0) && ((uintptr_t)dst % 16 == 0);
  const int vec = v16 ? 16 : 4;
  const uint32_t cpr = (uint32_t)(row_bytes / vec);
  if (RA_PERMUTE_IMPL && v16 && cpr <= 256 && 256 % cpr == 0) {
    const uint32_t rows_per_block = (256 / cpr) * 4;
    const uint64_t gx = ((uint64_t)n + rows_per_block - 1) / rows_per_block;
    const dim3 grid((unsigned)(gx < 1 ? 1 : gx), (unsigned)(BH < 65535 ? BH : 65535));
    if (RA_PERMUTE_IMPL == 2)
      hipLaunchKernelGGL(k_permute_rows<true>, grid, dim3(256), 0, s, (const char*)src, (char*)dst,
                         (uint64_t)BH, (uint32_t)n, cpr, (uint32_t)P, c, inverse, (uint64_t)row_bytes);
    else
      hipLaunchKernelGGL(k_permute_rows<false>, grid, dim3(256), 0, s, (const char*)src, (char*)dst,
                         (uint64_t)BH, (uint32_t)n, cpr, (uint32_t)P, c, inverse, (uint64_t)row_bytes);
    return hipGetLastError();
  }
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
  constexpr int U = RA_MERGE_ROWS;
  if (U > 1 && (d == 128 || d == 64)) {
    const int lpr = (int)(d / 4);
    const uint64_t waves = (uint64_t)((rows + (64 / lpr) * U - 1) / ((64 / lpr) * U));
    const int grid = grid_for(waves * 64, 256);
    if (lpr == 32)
      hipLaunchKernelGGL((k_merge_v4<32, U>), dim3(grid), dim3(256), 0, s, o_acc, lse_acc, o_part, lse_part, rows);
    else
      hipLaunchKernelGGL((k_merge_v4<16, U>), dim3(grid), dim3(256), 0, s, o_acc, lse_acc, o_part, lse_part, rows);
    return hipGetLastError();
  }
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

hipError_t launch_rope_permute(const void* src, void* dst, const int64_t* pos, int64_t BH, int64_t n, int64_t d,
                               int f32, int P, int striped, int inverse, int half, double base,
                               hipStream_t s) {
  const int grid = grid_for((uint64_t)n * 64, 256);
  const uint32_t c = (uint32_t)(n / P);
  // vector path: rows of d % 8 == 0 elements from 32-byte aligned bases keep every lane's 8-element
  // (or 4-element) access aligned to its own size
  const bool vec = d % 8 == 0 && d / 8 <= 64 && 64 % (d / 8) == 0 &&
                   (uintptr_t)src % 32 == 0 && (uintptr_t)dst % 32 == 0;
#define RA_ROPE(K, T, ...)                                                                       \
  hipLaunchKernelGGL(K, dim3(grid), dim3(256), 0, s, (const T*)src, (T*)dst, pos, BH, (uint32_t)n, \
                     (uint32_t)d, (uint32_t)P, c, striped, inverse, __VA_ARGS__)
  if (vec) {
    if (f32) {
      if (half) RA_ROPE((k_rope_permute_vec<float, true>), float, base);
      else RA_ROPE((k_rope_permute_vec<float, false>), float, base);
    } else {
      if (half) RA_ROPE((k_rope_permute_vec<__bf16, true>), __bf16, base);
      else RA_ROPE((k_rope_permute_vec<__bf16, false>), __bf16, base);
    }
  } else if (f32) {
    RA_ROPE(k_rope_permute<float>, float, half, base);
  } else {
    RA_ROPE(k_rope_permute<__bf16>, __bf16, half, base);
  }
#undef RA_ROPE
  return hipGetLastError();
}

}  // namespace ra
