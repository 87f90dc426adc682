/*
 * ra.h -- C ABI of libra.so: per-device blockwise exact attention for Ring Attention and
 * Striped Attention, on AMD Instinct MI355X (gfx950).
 *
 * The method (pages cited by title and section):
 *   - "ICLR 2024論文解説: Ring Attention — 複数GPU間でのブロックワイズ分散アテンションによる
 *     超長コンテキスト処理" (the Ring Attention review): a sequence of n tokens is split over
 *     P devices, c = n / P tokens each (step 1); every device keeps its query block Q_p and in
 *     round r works on the K/V block that started on device (p - r) mod P (step 2); partial
 *     results are combined with the online softmax (step 3), so that after P rounds each
 *     device holds exact softmax attention for its queries.
 *   - "Striped Attention: Faster Ring Attention for Causal Transformers" (paper review): the
 *     causal mask (section "核心公式"), the striped layout in which token t lives on device
 *     t mod P ("分区策略对比"), the per-round mask GetMask ("GetMask 函数"), skipping tiles
 *     whose pairs are all masked ("分块与分瓦片"), and permuting position IDs the same way
 *     ("位置编码处理").
 *   - "Computing Attention Weights in Sequence Parallelism": the softmax denominator of a query
 *     is the sum of per-node sums, which is what ra_merge combines.
 *
 * On one GPU the P devices are virtual: their rounds run in order on the caller's stream and
 * a K/V "transfer" is a pointer into the full tensor.
 *
 * Conventions shared by every entry point
 *   - Tensors are row-major.  Q, K, V, O are [B, H, n, d] (or [B, H, c, d] for one block),
 *     d contiguous, the token axis in layout order (contiguous or striped; token order for
 *     RA_STRIPED_TOKENS).  LSE is [B, H, n] (or [B, H, c]) float32, natural-log log-sum-exp of
 *     the scaled, masked scores of the row.
 *   - Device p's block is the token rows [p*c, (p+1)*c) of the layout-ordered tensor (rows
 *     p, p+P, ... of the token-order tensor for RA_STRIPED_TOKENS).
 *   - Every pointer argument is DEVICE memory owned by the caller unless stated otherwise; the
 *     library keeps no allocation between calls and never frees caller memory.
 *   - Calls only enqueue work on `stream` (a hipStream_t; NULL = the default stream) and never
 *     synchronize.  Inputs are read-only; outputs must not alias inputs (except ra_merge's
 *     accumulators, which are updated in place).
 *   - Validation runs on the host before anything is enqueued: a non-zero status means nothing
 *     was launched.  ra_last_error() then holds a message (per calling thread).  A failed
 *     launch returns RA_E_HIP.  No C++ exception or abort crosses the ABI.
 *   - An empty problem (B, H or n equal to 0) is valid and enqueues nothing.
 *   - No kernel loops on data values, so any input (NaN and infinities included) ends.  A NaN
 *     input reaches the outputs of the rows that use it; a NaN in V can also reach the O rows
 *     of the 32 x 32 tiles that mask it (0 x NaN in a matrix product), and no other row.
 */
#ifndef RA_H_
#define RA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RA_ABI_VERSION 5

typedef int32_t ra_status_t;
enum {
  RA_OK = 0,
  RA_E_INVAL = -1,        /* bad argument: null/misaligned pointer, index out of range, n % P != 0 */
  RA_E_UNSUPPORTED = -2,  /* valid but not implemented: head dim, dtype or layout combination */
  RA_E_HIP = -3           /* the HIP runtime reported an error when launching */
};

/* Element type of Q, K, V (and of O for ra_forward). */
enum { RA_BF16 = 0, RA_F32 = 1 };

/* Token layout of the Q/K/V rows. */
enum {
  RA_CONTIGUOUS = 0,      /* device p owns tokens [p*c, (p+1)*c)                                  */
  RA_STRIPED = 1,         /* device p owns tokens p, p+P, p+2P, ... (rows already permuted,
                             ra_permute)                                                          */
  RA_STRIPED_TOKENS = 2   /* the partition and masks of RA_STRIPED, with the tensors left in token
                             order: row y of device p's block is token row y*P + p, and the
                             kernels apply the permutation in their addressing.  ra_forward,
                             ra_backward and ra_permute_rope (identity permutation) only;
                             P <= 65536.                                                          */
};

/* One attention problem.  Plain host struct, passed by pointer. */
typedef struct {
  int64_t B, H;      /* batch, heads                                                        */
  int64_t n;         /* total tokens of the (emulated) sequence; n % P == 0                 */
  int64_t d;         /* head dim of Q, K and V                                              */
  int32_t P;         /* number of (virtual) sequence-parallel devices, >= 1                 */
  int32_t dtype;     /* RA_BF16 or RA_F32                                                   */
  int32_t layout;    /* RA_CONTIGUOUS or RA_STRIPED                                         */
  int32_t causal;    /* 0: every key visible; 1: key visible iff its position <= query's   */
  float scale;       /* score scale; <= 0 selects 1/sqrt(d)                                 */
} ra_problem_t;

/* Integer work counters for one (device, round), summed over B*H.  A tile is the kernel's
 * tq x tk unit of work (ra_tile_shape); edge tiles of a ragged block are classified on their
 * in-range part.  full: every pair visible; diag: some visible (element mask applied);
 * skipped: none visible (no work done). */
typedef struct {
  uint64_t unmasked_pairs;
  uint64_t tiles_full;
  uint64_t tiles_diag;
  uint64_t tiles_skipped;
} ra_round_stats_t;

/* Version of this ABI (RA_ABI_VERSION of the library that was built). */
int32_t ra_abi_version(void);

/* Message for the last non-zero status returned on the calling thread ("" if none).  The
 * string is owned by the library and valid until the next call on the same thread. */
const char* ra_last_error(void);

/* Host-only validation of `prob` and of a round's device indices (p: query device, kv: origin
 * device of the K/V block), exactly as ra_round performs it.  Touches no GPU.  Pass p = kv = 0
 * to validate the problem alone. */
ra_status_t ra_check(const ra_problem_t* prob, int32_t p, int32_t kv);

/* Tile shape (query rows x key columns) that the attention kernels for (dtype, d) classify
 * and skip at; the counters in ra_round_stats_t refer to it.  Host-only. */
ra_status_t ra_tile_shape(int32_t dtype, int64_t d, int32_t* tq, int32_t* tk);

/* Striped permutation of rows (Striped Attention review, "分区策略对比" and "位置编码处理"):
 * token t goes to layout row pi(t) = (t mod P) * (n / P) + t / P.
 *   inverse == 0: dst[bh][pi(t)] = src[bh][t]   (token order -> striped layout)
 *   inverse != 0: dst[bh][t] = src[bh][pi(t)]   (striped layout -> token order)
 * src and dst hold BH matrices of n rows of row_bytes bytes each, back to back.  row_bytes must
 * be a positive multiple of 4 and both pointers 4-byte aligned (16-byte rows and alignment
 * take the fast path).  src and dst must not overlap.  Works on any element type: Q/K/V/O
 * rows, LSE values (row_bytes 4), int64 position IDs (row_bytes 8). */
ra_status_t ra_permute(const void* src, void* dst, int64_t BH, int64_t n, int64_t row_bytes,
                       int32_t P, int32_t inverse, void* stream);

/* ra_permute for one vector of int64 position IDs of length n. */
ra_status_t ra_permute_ids(const int64_t* src, int64_t* dst, int64_t n, int32_t P,
                           int32_t inverse, void* stream);

/* Pairings of the head dim for ra_permute_rope. */
enum {
  RA_ROPE_INTERLEAVED = 0,  /* pair i = elements (2i, 2i+1)   */
  RA_ROPE_HALF = 1          /* pair i = elements (i, i + d/2) */
};

/* Rotary position embedding fused with the striped permutation (Striped Attention review,
 * "位置编码处理": RoPE-style encodings must see the position IDs permuted like the tokens).  The
 * pages do not define RoPE; this is RoFormer's rotary embedding: pair i of a token at position
 * m is rotated by the angle m * base^(-2i/d), so that a rotated query-key score depends on the
 * two positions only through their difference.
 *   inverse == 0: dst[bh][pi(t)] = R(m_t) src[bh][t]    (token order -> rotated, layout order)
 *   inverse != 0: dst[bh][t] = R(m_t)^T src[bh][pi(t)]  (the adjoint: carries dQ / dK back)
 * pi is the striped permutation of ra_permute for layout RA_STRIPED and the identity for
 * RA_CONTIGUOUS.  src, dst: BH matrices of n rows x d elements (dtype RA_BF16 or RA_F32, d even),
 * back to back; they must not overlap.  pos: NULL (m_t = t) or device int64 [n] positions in
 * token order.  Angles, cosines, sines and the rotation are computed in fp64 and rounded once
 * to fp32 (and then once to bf16 for bf16 data).  Striped needs n % P == 0. */
ra_status_t ra_permute_rope(const void* src, void* dst, const int64_t* pos, int64_t BH, int64_t n,
                            int64_t d, int32_t dtype, int32_t P, int32_t layout, double base,
                            int32_t style, int32_t inverse, void* stream);

/* One ring round (Ring Attention review, step 2): the query block of device p against the
 * K/V block that originated on device kv, under that pair's GetMask (causal) or no mask.
 *   q:  device p's block, B*H matrices of c = n/P rows x d, q_stride_bh elements apart
 *   k, v: block kv, B*H matrices of c rows x d, kv_stride_bh elements apart
 *         (so pointers into full [B,H,n,d] tensors work with strides n*d)
 *   o_part:   [B, H, c, d] float32, contiguous: softmax over this block's visible keys only
 *   lse_part: [B, H, c] float32: log-sum-exp of those scores
 * A query row with no visible key in this block (striped later-device row 0, or a contiguous
 * block from a later device) gets o_part = 0 and lse_part = -inf, the identity of ra_merge.
 * stats: NULL, or one device-memory ra_round_stats_t that the call adds its counts to.
 * Outputs (o_part, lse_part, stats) must not overlap q, k, v or each other (RA_E_INVAL). */
ra_status_t ra_round(const ra_problem_t* prob, const void* q, const void* k, const void* v,
                     int64_t q_stride_bh, int64_t kv_stride_bh, int32_t p, int32_t kv,
                     float* o_part, float* lse_part, ra_round_stats_t* stats, void* stream);

/* Log-sum-exp merge of a round partial into an accumulator ("Computing Attention Weights in
 * Sequence Parallelism": per-node denominators add):
 *   L = ln(e^{lse_acc} + e^{lse_part}),  o_acc = e^{lse_acc - L} o_acc + e^{lse_part - L} o_part,
 *   lse_acc = L, for `rows` rows of d float32 values (o arrays contiguous [rows, d]).
 * Rows where both sides are -inf stay (0, -inf); a NaN LSE on either side gives NaN O and LSE.
 * Start an accumulation from o_acc = 0,
 * lse_acc = -inf (or copy the first partial).  o_part/lse_part must not alias the acc. */
ra_status_t ra_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                     int64_t rows, int64_t d, void* stream);

/* All P rounds of the devices p_begin <= p < p_end, fused: each device's running max,
 * normaliser and output stay on chip across its rounds, which run in ring order
 * r = 0..P-1 (K/V block (p - r) mod P, Ring Attention review step 3).
 *   q, k, v: full [B, H, n, d] tensors in layout order (contiguous)
 *   o:   [B, H, (p_end - p_begin) * c, d] in o_dtype (RA_BF16 or RA_F32), rows of device
 *        p_begin first; lse: NULL or [B, H, (p_end - p_begin) * c] float32
 *   RA_STRIPED_TOKENS: q, k, v, o and lse are all in token order, o [B, H, n, d] and lse
 *        [B, H, n]; only the rows of the selected devices (tokens t with p_begin <= t mod P
 *        < p_end) are written, so the range 0..P gives causal attention over the sequence with
 *        no permutation pass before or after
 *   stats: NULL or device memory [P][P] ra_round_stats_t indexed [p][r]; the call clears rows
 *          p_begin..p_end-1 on the stream and writes their counts there; other rows are not
 *          touched.
 * Outputs (o, lse, stats) must not overlap q, k, v or each other (RA_E_INVAL). */
ra_status_t ra_forward(const ra_problem_t* prob, const void* q, const void* k, const void* v,
                       int32_t p_begin, int32_t p_end, void* o, int32_t o_dtype, float* lse,
                       ra_round_stats_t* stats, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Backward pass.  The pages describe the forward only; the gradients are those of its
 * definition O = softmax(Q K^T * scale + C) V (Striped Attention review, "核心公式"; Ring
 * Attention review, step 3).  With the forward's LSE L of each query row and
 * D = rowsum(O * dO), every (query block p, K/V block k) pair contributes independently:
 *   P = exp(S + C - L), dP = dO V^T, dS = P * (dP - D),
 *   dQ_p += scale * dS K_k,  dK_k += scale * dS^T Q_p,  dV_k += P^T dO_p,
 * with the pair's GetMask deciding C (Striped Attention review, "GetMask 函数").  In a ring,
 * dQ stays on device p while dK, dV travel with their K/V block (Ring Attention review, step
 * 2), collecting one contribution per device.  Gradients are float32; Q, K, V and dO share the
 * problem's dtype.  No atomics: results are deterministic run to run.
 * ------------------------------------------------------------------------------------------- */

/* Backward row term D_i = sum_e O[i, e] * dO[i, e] for `rows` rows of d values.
 *   o: [rows, d] in o_dtype (RA_BF16 or RA_F32), the forward output; dout: [rows, d] in
 *   dout_dtype; delta: [rows] float32 (written).  Arrays contiguous; o and dout 16-byte (f32)
 *   or 8-byte (bf16) aligned when d % 4 == 0, else element aligned. */
ra_status_t ra_bwd_delta(const void* o, int32_t o_dtype, const void* dout, int32_t dout_dtype,
                         int64_t rows, int64_t d, float* delta, void* stream);

/* Backward of one ring round: the query block of device p against the K/V block kv.
 *   q:       device p's rows, B*H matrices of c x d, q_stride_bh elements apart
 *   dout:    the same rows' dO, B*H matrices of c x d, do_stride_bh elements apart
 *   k, v:    block kv, B*H matrices of c x d, kv_stride_bh elements apart
 *   lse, delta: device p's rows, B*H vectors of c float32, row_stride_bh elements apart;
 *            lse is the FINAL log-sum-exp of the rows over all keys (ra_forward's, or the
 *            ra_merge result), not a round partial; delta from ra_bwd_delta
 *   dq_acc:  [B, H, c, d] float32, contiguous: this pair's dQ contribution is ADDED
 *   dk_acc, dv_acc: [B, H, c, d] float32, contiguous: dK, dV contributions ADDED
 * A pair with no visible key (contiguous block from a later device) adds nothing. */
ra_status_t ra_backward_round(const ra_problem_t* prob, const void* q, const void* k,
                              const void* v, const void* dout, const float* lse,
                              const float* delta, int64_t q_stride_bh, int64_t do_stride_bh,
                              int64_t kv_stride_bh, int64_t row_stride_bh, int32_t p, int32_t kv,
                              float* dq_acc, float* dk_acc, float* dv_acc, void* stream);

/* All rounds of the devices p_begin <= p < p_end, fused (the backward of ra_forward).
 *   q, k, v: full [B, H, n, d] tensors in layout order (contiguous)
 *   dout:    [B, H, m, d], m = (p_end - p_begin) * c, rows of device p_begin first
 *   lse, delta: [B, H, m] float32 (ra_forward's lse; ra_bwd_delta)
 *   dq:      [B, H, m, d] float32, written
 *   dk, dv:  [B, H, n, d] float32, written: the gradient that the queries of devices
 *            p_begin..p_end-1 send to every key (the full gradient when the range is 0..P)
 *   RA_STRIPED_TOKENS: every tensor in token order, with m = n: dout and dq [B, H, n, d],
 *            lse and delta [B, H, n]; dq is written only on the rows of the selected devices
 *            (tokens t with p_begin <= t mod P < p_end), dk and dv on every row.
 * Each output element belongs to one workgroup, which writes it in a fixed order (a dQ row may
 * be stored after one round and added to after later rounds by that same workgroup); no
 * atomics, so the results are the same from run to run. */
ra_status_t ra_backward(const ra_problem_t* prob, const void* q, const void* k, const void* v,
                        const void* dout, const float* lse, const float* delta, int32_t p_begin,
                        int32_t p_end, float* dq, float* dk, float* dv, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RA_H_ */
