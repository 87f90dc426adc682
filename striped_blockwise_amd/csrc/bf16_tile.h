// Building blocks shared by the bf16 attention kernels (head dim 128, gfx950 matrix cores).
//
//  * v_mfma_f32_32x32x16_bf16 operand layouts: A (32 rows x 16 contraction) -- lane l holds
//    row l % 32, contraction elements 8 (l / 32) .. +7; B (16 contraction x 32 columns) -- lane
//    l holds column l % 32, the same contraction elements; C (32 x 32 fp32) -- lane l holds
//    column l % 32, rows acc_row(r, l / 32) for r = 0..15.
//  * A C tile can feed the next MFMA as its B operand directly (column stays in the lane): its
//    rows become the contraction index in the order acc_row gives them, and the A operand of
//    that MFMA is then read with the same order (the transposed reads below do that).
//  * Tiles of 128-element bf16 rows (256 B) live in LDS with each row's sixteen 16-byte chunks
//    permuted by an XOR mask of the row; HBM -> LDS moves are direct DMA (buffer_load ... lds).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {
namespace bf16t {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int D = 128;          // head dim
constexpr int ROWB = D * 2;     // bytes per row of a tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Row (within a 32-row MFMA block) held by accumulator register r in lane half h.
__device__ __forceinline__ int acc_row(int r, int h) { return (r >> 2) * 8 + h * 4 + (r & 3); }

// Swizzle masks (XOR on the 16-byte chunk index of a row).
//  k_swz: for tiles read only row-wise as A operands (32 consecutive rows, one chunk): any 16
//         consecutive rows fall on 16 different chunks.
//  v_swz: for tiles read only with ds_read_b64_tr_b16, where one 32-lane half reads 4
//         consecutive rows x 4 consecutive chunks (8 B per lane): bits {0b1010 for row bit 0,
//         0b0100 for row bit 1} put those 16 (row, chunk) pairs on 16 different chunks and any
//         16 lanes on 8 different chunk pairs.
//  t_swz: for tiles read both ways: v_swz, whose four values on an aligned group of 4 rows keep
//         the transposed reads conflict-free, XORed with a per-group term {0, 1, 8, 9} (constant
//         within the group) that makes any 16 aligned rows take 16 different masks and any 8
//         aligned rows 8 different values of mask & 7, as the row-wise reads need.
__device__ __forceinline__ int k_swz(int row) { return row & 15; }
__device__ __forceinline__ int v_swz(int row) { return ((row & 1) ? 10 : 0) ^ ((row & 2) ? 4 : 0); }
__device__ __forceinline__ int t_swz(int row) {
  return v_swz(row) ^ ((row & 4) ? 1 : 0) ^ ((row & 8) ? 8 : 0);
}
enum Swz { SWZ_K = 0, SWZ_V = 1, SWZ_T = 2 };
template <int S>
__device__ __forceinline__ int swz(int row) {
  return S == SWZ_K ? k_swz(row) : (S == SWZ_V ? v_swz(row) : t_swz(row));
}
template <int S>
__device__ __forceinline__ int tile_off(int row, int byte_in_row) {
  return row * ROWB + ((((byte_in_row >> 4) ^ swz<S>(row))) << 4) + (byte_in_row & 15);
}

__device__ __forceinline__ float pair_max(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// LDS offset (relative to a tile) of lane `lane`'s row-wise A-operand read of contraction step
// dk (16 elements) for 32-row block 0: row l % 32, elements 16 dk + 8 (l / 32) .. +7.
template <int S>
__device__ __forceinline__ int a_rowwise_off(int lane, int dk) {
  return tile_off<S>(lane & 31, (2 * dk + (lane >> 5)) * 16);
}

// LDS offsets of the transposed A-operand reads (ds_read_b64_tr_b16) for column block db (32
// columns of the tile, i.e. 32 consecutive head-dim elements) and half `sec` of a 16-row
// contraction step.  In each 16-lane group, result lane 4a+b element e comes from element b of
// source lane 4e+a; source lane (G, e, a) therefore points at row 4 h + e (+8 for sec = 1),
// h = G / 2, elements 32 db + 16 (G % 2) + 4 a .. +3, so that result lane L holds column
// 32 db + L % 32 and rows {4h..4h+3} / {8+4h..8+4h+3} -- the rows acc_row gives lane half h.
template <int S>
__device__ __forceinline__ int a_tr_off(int lane, int db, int sec) {
  const int G = lane >> 4, e = (lane >> 2) & 3, aa = lane & 3;
  const int h = G >> 1, g2 = G & 1;
  const int row = 4 * h + e + 8 * sec;
  const int d = 32 * db + 16 * g2 + 4 * aa;
  return tile_off<S>(row, 2 * d);
}

// XOR form of the same offsets, for kernels short of registers.  With any of the chunk masks,
// the row-wise offset of step dk is a_rowwise_off(lane, 0) ^ (dk << 5) (the step index moves
// chunk bits 1-3 only), and the transposed offset of (db, sec) is a_tr_off(lane, 0, 0) ^
// tr_xor(db, sec) under t_swz (db moves chunk bits 2-3; sec adds 8 rows, which flips bit 3 of
// the t_swz mask).  Tile bases that are multiples of 8 KB (and the 4 KB step between the two
// 16-row halves of a 32-row tile) leave bits 3-11 free, so they can be added before the XOR.
__device__ __forceinline__ constexpr int tr_xor(int db, int sec) { return (db << 6) ^ (sec ? (2048 | 128) : 0); }

// Transposed A operand (rows of the tile become the contraction index): the two 8-byte
// ds_read_b64_tr_b16 reads at `tile` + a_tr_off(lane, db, 0) / a_tr_off(lane, db, 1) give the
// lane's column 32 db + lane % 32 over the 16 rows of one contraction step.
__device__ __forceinline__ bf16x8 read_a_tr(const char* tile, int off_lo, int off_hi) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off_lo));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off_hi));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// DMA of tiles of ROWS rows (256 B per row) into LDS, split into 1 KB segments (4 rows) over NW
// wavefronts: wave w does segments w, w + NW, ...  In global memory consecutive rows of a block
// are row_step rows apart (1 for a block stored on its own; P for a striped block read straight
// from a token-order tensor, whose row y is token y P + k).  Each wave keeps the per-lane
// offsets of its segments in `unsigned voff[DmaShape<NW, ROWS>::PER_WAVE]`: lane j of segment
// seg fills LDS row 4 seg + j / 16 at physical chunk j % 16, which holds logical chunk
// (j % 16) ^ mask(row) of that row (the XOR permutation is its own inverse).  The offsets pass as
// plain pointers: with an array reference, or a struct holding the array, hipcc's host pass
// reported a substitution failure for these device templates (or, for member functions, quietly
// dropped the launch stub of every kernel instantiation after the first).
template <int NW, int ROWS>
struct DmaShape {
  static constexpr int SEGS = ROWS * ROWB / 1024;
  static constexpr int PER_WAVE = (SEGS + NW - 1) / NW;
};

template <int NW, int ROWS>
__device__ __forceinline__ void dma_init(unsigned* voff, Swz kind, int wave_u, int lane, int row_step) {
#pragma unroll
  for (int i = 0; i < DmaShape<NW, ROWS>::PER_WAVE; ++i) {
    const int row = (wave_u + i * NW) * 4 + (lane >> 4);
    const int mask = kind == SWZ_K ? swz<SWZ_K>(row) : (kind == SWZ_V ? swz<SWZ_V>(row) : swz<SWZ_T>(row));
    voff[i] = (unsigned)row * (unsigned)row_step * ROWB + (unsigned)(((lane & 15) ^ mask) << 4);
  }
}

// Rows x0 .. x0 + ROWS - 1 (x0 < c) of a block of c rows at `block` into the LDS tile `tile`.
// The buffer descriptor starts at row x0 and ends after the last row that exists, so the
// per-lane offsets are loop constants and rows past the end of the block are out of range: the
// buffer unit returns zeros for them, which land in LDS.  (ROWS - 1) * row_step * 256 + 256 must
// fit in 32 bits.
template <int NW, int ROWS>
__device__ __forceinline__ void dma_issue(const unsigned* voff, const char* block, char* tile, int x0, int c,
                                          int row_step, int wave_u) {
  constexpr int SEGS = DmaShape<NW, ROWS>::SEGS;
  const unsigned last = (unsigned)(min(c - x0, ROWS) - 1);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(block + (int64_t)x0 * row_step * ROWB), 0, (int)((last * (unsigned)row_step + 1) * ROWB),
      0x00020000);
#pragma unroll
  for (int i = 0; i < DmaShape<NW, ROWS>::PER_WAVE; ++i) {
    const int seg = wave_u + i * NW;
    if (SEGS % NW == 0 || seg < SEGS)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(tile + seg * 1024), 16, voff[i], 0, 0, 0);
  }
}

// The same transposed read with the tile pointer marked restrict.  After inlining, the two reads
// then carry alias-scope metadata, and the compiler's wait-count pass no longer makes them wait
// for every LDS DMA still in flight (it does so for LDS reads that carry no alias information).
// The caller must itself wait for the DMA that filled `tile` (vm_wait) before the call.
__device__ __forceinline__ bf16x8 read_a_tr_nowait(const char* __restrict__ tile, int off_lo, int off_hi) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off_lo));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off_hi));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A plain LDS read through a restrict-qualified pointer, for the same reason as
// read_a_tr_nowait: the compiler then does not make it wait for every LDS DMA in flight.  The
// caller must have waited for the DMA that filled the data.
template <typename T>
__device__ __forceinline__ T lds_read_nowait(const char* __restrict__ base, int off) {
  return *reinterpret_cast<const T*>(base + off);
}

// s_waitcnt with vmcnt(N) only (expcnt and lgkmcnt left at their maxima): at most N of this
// thread's vector-memory loads, LDS DMA included, still outstanding.  They complete in order.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0) only: this thread's LDS reads have all returned.
__device__ __forceinline__ void lgkm_wait0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ void wait_dma_and_barrier() {
  vm_wait<0>();                         // this thread's LDS DMA has landed
  __syncthreads();
}

}  // namespace bf16t
}  // namespace ra
