// Internal declarations shared by the HIP translation units of libra.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra.h"
#include "tile_deal.h"

namespace ra {

// Launch description for the attention kernels (one for ra_round, one for ra_forward).
struct AttnArgs {
  const void* q;          // block of device p_begin (element type per kernel)
  const void* k;          // K/V block kv_base
  const void* v;
  int64_t q_bh_stride;    // elements between consecutive (b, h) matrices of q
  int64_t kv_bh_stride;   // same for k and v
  int64_t q_dev_stride;   // elements between consecutive device blocks of q
  int64_t kv_blk_stride;  // elements between consecutive K/V blocks
  int row_step;           // rows between consecutive rows of a block in q, k, v, o and lse: 1,
                          // or P for a striped block read from a token-order tensor
  void* o;                // output rows of device p_begin, then p_begin+1, ...
  float* lse;             // nullable
  int64_t o_bh_stride;    // elements between (b, h) matrices of o
  int64_t o_dev_stride;   // elements between the first rows of consecutive devices in o
  int64_t lse_bh_stride;  // elements between (b, h) vectors of lse
  int64_t lse_dev_stride; // same for lse
  int c;                  // rows per block
  int P;                  // devices
  int BH;                 // B * H
  int p_begin;            // absolute index of the first query device
  int n_dev;              // number of query devices
  int kv_base;            // block index the k / v pointers point at
  int r_begin;            // first ring round
  int r_count;            // number of rounds
  int layout;
  int causal;
  float scale;            // score multiplier (natural units)
  int o_f32;              // 1: o is float32, 0: bf16
  ra_round_stats_t* stats;  // nullable
  int stats_single;       // 1: one entry (ra_round), 0: [P][P] indexed [p][r]
  int xcd_major;          // set by the bf16 launcher: block order (see k_attn_bf16.hip)
};

// Launch description for the backward kernels.  Two kernels share it: the dQ kernel (query
// rows stationary, K/V blocks of the given rounds streamed past them, like the forward) and the
// dK/dV kernel (key rows of K/V blocks kv_base .. kv_base+n_kv-1 stationary, the query blocks of
// devices p_begin .. p_begin+n_dev-1 streamed past them).
struct BwdArgs {
  const void* q;          // rows of query device p_begin; device blocks q_dev_stride apart
  const void* dout;       // dO rows of device p_begin; device blocks do_dev_stride apart
  const float* lse;       // forward log-sum-exp (natural log) of the same rows
  const float* delta;     // D = rowsum(O * dO) of the same rows
  const void* k;          // K/V block kv_base; blocks kv_blk_stride apart
  const void* v;
  int64_t q_bh_stride;    // elements between (b, h) matrices of q
  int64_t do_bh_stride;   // ... of dout
  int64_t row_bh_stride;  // ... of lse and delta
  int64_t kv_bh_stride;   // ... of k and v
  int64_t q_dev_stride;   // elements between device blocks of q
  int64_t do_dev_stride;  // ... of dout
  int64_t row_dev_stride; // ... of lse and delta
  int64_t kv_blk_stride;  // elements between K/V blocks
  int row_step;           // rows between consecutive rows of a block in every row-indexed
                          // tensor (q, dout, lse, delta, k, v, dq, dk, dv): 1, or P for a
                          // striped block of a token-order tensor
  float* dq;              // rows of device p_begin, then p_begin+1, ...
  int64_t dq_bh_stride;
  int64_t dq_dev_stride;  // elements between the first rows of consecutive devices in dq
  float* dk;              // rows of block kv_base, then kv_base+1, ...
  float* dv;
  int64_t dkv_bh_stride;
  int64_t dkv_blk_stride; // elements between the first rows of consecutive blocks in dk, dv
  int c;                  // rows per block
  int P;                  // devices
  int BH;                 // B * H
  int p_begin;            // absolute index of the first query device
  int n_dev;              // number of query devices
  int kv_base;            // absolute index of the first K/V block
  int n_kv;               // dK/dV kernel: number of K/V blocks
  int r_begin;            // dQ kernel: first ring round
  int r_count;            // dQ kernel: number of rounds
  int layout;
  int causal;
  float scale;            // score multiplier (natural units)
  int accumulate;         // 1: add into dq / dk / dv, 0: overwrite them
  int xcd_major;          // set by the bf16 launchers
};

hipError_t launch_permute(const void* src, void* dst, int64_t BH, int64_t n, int64_t row_bytes,
                          int P, int inverse, hipStream_t s);
hipError_t launch_zero_u64(uint64_t* p, int64_t n, hipStream_t s);
hipError_t launch_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                        int64_t rows, int64_t d, hipStream_t s);
hipError_t launch_rope_permute(const void* src, void* dst, const int64_t* pos, int64_t BH, int64_t n, int64_t d,
                               int f32, int P, int striped, int inverse, int half, double base,
                               hipStream_t s);
hipError_t launch_delta(const void* o, int o_f32, const void* dout, int do_f32, int64_t rows,
                        int64_t d, float* delta, hipStream_t s);
hipError_t launch_bwd_f32(const BwdArgs& a, int d, bool dq, bool dkv, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs& a, int d, bool dq, bool dkv, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, int d, hipStream_t s);
hipError_t launch_attn_bf16(const AttnArgs& a, int d, hipStream_t s);
// Compute units of the current device (queried once per device), for the launchers' choice of
// workgroup shape.
int cu_count();

bool attn_f32_supported(int64_t d);
bool attn_bf16_supported(int64_t d);
bool bwd_f32_supported(int64_t d);
bool bwd_bf16_supported(int64_t d);
void attn_f32_tile(int* tq, int* tk);
void attn_bf16_tile(int* tq, int* tk);

}  // namespace ra
