// Host side of libra.so: argument validation, error reporting and kernel dispatch for the C ABI
// declared in include/ra.h.  Nothing here allocates device memory or synchronizes.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "ra_internal.h"

namespace ra {

// Queried once per device; concurrent first calls from several host threads store the same
// value.
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace ra

namespace {

thread_local char g_err[512] = "";

ra_status_t fail(ra_status_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

ra_status_t ok() {
  g_err[0] = '\0';
  return RA_OK;
}

ra_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(RA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t elem_bytes(int32_t dtype) { return dtype == RA_F32 ? 4 : 2; }

// Largest P for RA_STRIPED_TOKENS: a K/V tile's rows are P rows apart, and a tile's span must
// stay far inside the 32-bit range of a buffer descriptor.
constexpr int32_t kMaxTokenP = 65536;

bool empty_problem(const ra_problem_t* pr) { return pr->B == 0 || pr->H == 0 || pr->n == 0; }

// Problem-level checks shared by every attention entry point.
ra_status_t check_problem(const ra_problem_t* pr) {
  if (!pr) return fail(RA_E_INVAL, "problem pointer is NULL");
  if (pr->B < 0 || pr->H < 0 || pr->n < 0) return fail(RA_E_INVAL, "B, H and n must be >= 0");
  if (pr->d <= 0) return fail(RA_E_INVAL, "head dim d must be > 0 (got %lld)", (long long)pr->d);
  if (pr->P < 1) return fail(RA_E_INVAL, "P must be >= 1 (got %d)", pr->P);
  if (pr->n % pr->P != 0)
    return fail(RA_E_INVAL, "n (%lld) must be a multiple of P (%d)", (long long)pr->n, pr->P);
  if (pr->dtype != RA_BF16 && pr->dtype != RA_F32) return fail(RA_E_INVAL, "unknown dtype %d", pr->dtype);
  if (pr->layout != RA_CONTIGUOUS && pr->layout != RA_STRIPED && pr->layout != RA_STRIPED_TOKENS)
    return fail(RA_E_INVAL, "unknown layout %d", pr->layout);
  if (pr->layout == RA_STRIPED_TOKENS && pr->P > kMaxTokenP)
    return fail(RA_E_INVAL, "RA_STRIPED_TOKENS needs P <= %d (got %d)", kMaxTokenP, pr->P);
  if (pr->causal != 0 && pr->causal != 1) return fail(RA_E_INVAL, "causal must be 0 or 1");
  if (!std::isfinite(pr->scale)) return fail(RA_E_INVAL, "scale must be finite");
  const int64_t c = pr->n / pr->P;
  if (c > (int64_t)INT32_MAX / pr->d || pr->B > INT32_MAX || pr->H > INT32_MAX ||
      pr->B * pr->H > INT32_MAX / 64)
    return fail(RA_E_INVAL, "problem too large: rows per block x d must fit in int32");
  if (pr->B > 0 && pr->H > 0 && pr->n > INT64_MAX / pr->B / pr->H / pr->d)
    return fail(RA_E_INVAL, "problem too large: B*H*n*d overflows int64");
  const bool sup = pr->dtype == RA_BF16 ? ra::attn_bf16_supported(pr->d) : ra::attn_f32_supported(pr->d);
  if (!sup)
    return fail(RA_E_UNSUPPORTED, "head dim %lld is not supported for %s inputs (bf16: 128; f32: 32, 64, 128)",
                (long long)pr->d, pr->dtype == RA_BF16 ? "bf16" : "f32");
  return ok();
}

// The per-round entry points take one block per pointer, with its rows back to back.
ra_status_t check_block_layout(const ra_problem_t* pr) {
  if (pr->layout == RA_STRIPED_TOKENS)
    return fail(RA_E_UNSUPPORTED, "per-round entry points take blocks in layout order: use RA_STRIPED "
                                  "(rows permuted by ra_permute)");
  return ok();
}

float eff_scale(const ra_problem_t* pr) {
  return pr->scale > 0.f ? pr->scale : (float)(1.0 / std::sqrt((double)pr->d));
}

ra_status_t launch_attn(const ra_problem_t* pr, const ra::AttnArgs& a, hipStream_t s) {
  hipError_t e = pr->dtype == RA_BF16 ? ra::launch_attn_bf16(a, (int)pr->d, s)
                                      : ra::launch_attn_f32(a, (int)pr->d, s);
  return hip_status(e, "attention kernel launch");
}


bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const char* x = (const char*)a;
  const char* y = (const char*)b;
  return x < y + bbytes && y < x + abytes;
}

// A memory range [ptr, ptr + bytes) of one argument, for the aliasing checks.
struct Span {
  const void* p;
  int64_t bytes;
  const char* name;
};

// Every output span must be disjoint from every input span and from the other outputs (inputs
// may alias each other: Q, K and V may be one tensor).
template <size_t NO, size_t NI>
ra_status_t check_no_alias(const Span (&outs)[NO], const Span (&ins)[NI]) {
  for (size_t i = 0; i < NO; ++i) {
    if (!outs[i].p || outs[i].bytes <= 0) continue;
    for (size_t j = 0; j < NI; ++j)
      if (ins[j].p && ins[j].bytes > 0 && overlaps(outs[i].p, outs[i].bytes, ins[j].p, ins[j].bytes))
        return fail(RA_E_INVAL, "output %s overlaps input %s", outs[i].name, ins[j].name);
    for (size_t j = i + 1; j < NO; ++j)
      if (outs[j].p && outs[j].bytes > 0 && overlaps(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes))
        return fail(RA_E_INVAL, "outputs %s and %s overlap", outs[i].name, outs[j].name);
  }
  return ok();
}

ra_status_t check_bwd_support(const ra_problem_t* pr) {
  const bool sup = pr->dtype == RA_BF16 ? ra::bwd_bf16_supported(pr->d) : ra::bwd_f32_supported(pr->d);
  if (!sup)
    return fail(RA_E_UNSUPPORTED, "backward: head dim %lld is not supported for %s inputs",
                (long long)pr->d, pr->dtype == RA_BF16 ? "bf16" : "f32");
  return ok();
}

// dq, dk, dv must be three disjoint float32 arrays of `dq_bytes` / `dkv_bytes` bytes.
ra_status_t check_grad_outputs(const float* dq, int64_t dq_bytes, const float* dk, const float* dv,
                               int64_t dkv_bytes) {
  if (!aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return fail(RA_E_INVAL, "dq, dk and dv must be 16-byte aligned");
  if (overlaps(dq, dq_bytes, dk, dkv_bytes) || overlaps(dq, dq_bytes, dv, dkv_bytes) ||
      overlaps(dk, dkv_bytes, dv, dkv_bytes))
    return fail(RA_E_INVAL, "dq, dk and dv must not overlap");
  return ok();
}

ra_status_t launch_bwd(const ra_problem_t* pr, const ra::BwdArgs& a, hipStream_t s) {
  hipError_t e = pr->dtype == RA_BF16 ? ra::launch_bwd_bf16(a, (int)pr->d, true, true, s)
                                      : ra::launch_bwd_f32(a, (int)pr->d, true, true, s);
  return hip_status(e, "backward kernel launch");
}

}  // namespace

extern "C" {

int32_t ra_abi_version(void) { return RA_ABI_VERSION; }

const char* ra_last_error(void) { return g_err; }

ra_status_t ra_check(const ra_problem_t* prob, int32_t p, int32_t kv) {
  ra_status_t st = check_problem(prob);
  if (st != RA_OK) return st;
  if (p < 0 || p >= prob->P) return fail(RA_E_INVAL, "query device p=%d out of range [0, %d)", p, prob->P);
  if (kv < 0 || kv >= prob->P) return fail(RA_E_INVAL, "K/V device kv=%d out of range [0, %d)", kv, prob->P);
  return ok();
}

ra_status_t ra_tile_shape(int32_t dtype, int64_t d, int32_t* tq, int32_t* tk) {
  if (!tq || !tk) return fail(RA_E_INVAL, "tq / tk out-pointers must not be NULL");
  if (dtype == RA_BF16) {
    if (!ra::attn_bf16_supported(d)) return fail(RA_E_UNSUPPORTED, "bf16 head dim %lld not supported", (long long)d);
    ra::attn_bf16_tile(tq, tk);
  } else if (dtype == RA_F32) {
    if (!ra::attn_f32_supported(d)) return fail(RA_E_UNSUPPORTED, "f32 head dim %lld not supported", (long long)d);
    ra::attn_f32_tile(tq, tk);
  } else {
    return fail(RA_E_INVAL, "unknown dtype %d", dtype);
  }
  return ok();
}

ra_status_t ra_permute(const void* src, void* dst, int64_t BH, int64_t n, int64_t row_bytes,
                       int32_t P, int32_t inverse, void* stream) {
  if (BH < 0 || n < 0) return fail(RA_E_INVAL, "BH and n must be >= 0");
  if (P < 1) return fail(RA_E_INVAL, "P must be >= 1 (got %d)", P);
  if (n % P != 0) return fail(RA_E_INVAL, "n (%lld) must be a multiple of P (%d)", (long long)n, P);
  if (row_bytes <= 0 || row_bytes % 4 != 0) return fail(RA_E_INVAL, "row_bytes must be a positive multiple of 4");
  if (n > (int64_t)UINT32_MAX / 2) return fail(RA_E_INVAL, "n too large");
  if (BH == 0 || n == 0) return ok();
  if (!src || !dst) return fail(RA_E_INVAL, "src / dst must not be NULL");
  if (!aligned(src, 4) || !aligned(dst, 4)) return fail(RA_E_INVAL, "src / dst must be 4-byte aligned");
  if (BH > INT64_MAX / n / row_bytes) return fail(RA_E_INVAL, "BH*n*row_bytes overflows");
  const int64_t bytes = BH * n * row_bytes;
  const char* s0 = (const char*)src;
  const char* d0 = (const char*)dst;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(RA_E_INVAL, "src and dst overlap");
  return hip_status(ra::launch_permute(src, dst, BH, n, row_bytes, P, inverse ? 1 : 0, (hipStream_t)stream),
                    "permute kernel launch");
}

ra_status_t ra_permute_ids(const int64_t* src, int64_t* dst, int64_t n, int32_t P, int32_t inverse,
                           void* stream) {
  return ra_permute(src, dst, 1, n, 8, P, inverse, stream);
}

ra_status_t ra_permute_rope(const void* src, void* dst, const int64_t* pos, int64_t BH, int64_t n,
                            int64_t d, int32_t dtype, int32_t P, int32_t layout, double base,
                            int32_t style, int32_t inverse, void* stream) {
  if (BH < 0 || n < 0) return fail(RA_E_INVAL, "BH and n must be >= 0");
  if (d <= 0 || d % 2) return fail(RA_E_INVAL, "head dim d must be positive and even (got %lld)", (long long)d);
  if (dtype != RA_BF16 && dtype != RA_F32) return fail(RA_E_INVAL, "unknown dtype %d", dtype);
  if (layout != RA_CONTIGUOUS && layout != RA_STRIPED && layout != RA_STRIPED_TOKENS)
    return fail(RA_E_INVAL, "unknown layout %d", layout);
  if (style != RA_ROPE_INTERLEAVED && style != RA_ROPE_HALF) return fail(RA_E_INVAL, "unknown RoPE style %d", style);
  if (!(base > 0.0) || !std::isfinite(base)) return fail(RA_E_INVAL, "base must be positive and finite");
  if (P < 1) return fail(RA_E_INVAL, "P must be >= 1 (got %d)", P);
  if (layout == RA_STRIPED && n % P != 0) return fail(RA_E_INVAL, "n (%lld) must be a multiple of P (%d)", (long long)n, P);
  if (n > (int64_t)UINT32_MAX / 2 || d > (int64_t)UINT32_MAX / 2) return fail(RA_E_INVAL, "n or d too large");
  if (BH == 0 || n == 0) return ok();
  if (!src || !dst) return fail(RA_E_INVAL, "src / dst must not be NULL");
  const int64_t eb = elem_bytes(dtype);
  if (!aligned(src, eb) || !aligned(dst, eb) || (pos && !aligned(pos, 8)))
    return fail(RA_E_INVAL, "src / dst must be element aligned, pos 8-byte aligned");
  if (BH > INT64_MAX / n / d / eb) return fail(RA_E_INVAL, "BH*n*d overflows");
  const int64_t bytes = BH * n * d * eb;
  if (overlaps(src, bytes, dst, bytes)) return fail(RA_E_INVAL, "src and dst overlap");
  const int Pe = layout == RA_STRIPED ? P : 1;
  return hip_status(ra::launch_rope_permute(src, dst, pos, BH, n, d, dtype == RA_F32, Pe, layout == RA_STRIPED,
                                            inverse ? 1 : 0, style == RA_ROPE_HALF, base, (hipStream_t)stream),
                    "rope kernel launch");
}

ra_status_t ra_round(const ra_problem_t* prob, const void* q, const void* k, const void* v,
                     int64_t q_stride_bh, int64_t kv_stride_bh, int32_t p, int32_t kv,
                     float* o_part, float* lse_part, ra_round_stats_t* stats, void* stream) {
  ra_status_t st = ra_check(prob, p, kv);
  if (st != RA_OK) return st;
  st = check_block_layout(prob);
  if (st != RA_OK) return st;
  if (empty_problem(prob)) return ok();
  const int64_t c = prob->n / prob->P;
  const int64_t d = prob->d;
  if (!q || !k || !v || !o_part || !lse_part) return fail(RA_E_INVAL, "q, k, v, o_part and lse_part must not be NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o_part, 16) || !aligned(lse_part, 4))
    return fail(RA_E_INVAL, "q, k, v and o_part must be 16-byte aligned, lse_part 4-byte aligned");
  const int64_t vec = 16 / elem_bytes(prob->dtype);
  if (q_stride_bh < 0 || kv_stride_bh < 0 || q_stride_bh % vec || kv_stride_bh % vec)
    return fail(RA_E_INVAL, "strides must be >= 0 and multiples of %lld elements", (long long)vec);
  if (prob->B * prob->H > 1 && (q_stride_bh < c * d || kv_stride_bh < c * d))
    return fail(RA_E_INVAL, "strides must be at least c*d = %lld elements", (long long)(c * d));
  if (stats && !aligned(stats, 8)) return fail(RA_E_INVAL, "stats must be 8-byte aligned");
  {
    const int64_t BH = prob->B * prob->H;
    const int64_t eb = elem_bytes(prob->dtype);
    const int64_t qb = ((BH - 1) * q_stride_bh + c * d) * eb, kvb = ((BH - 1) * kv_stride_bh + c * d) * eb;
    const Span outs[] = {{o_part, BH * c * d * 4, "o_part"}, {lse_part, BH * c * 4, "lse_part"},
                         {stats, (int64_t)sizeof(ra_round_stats_t), "stats"}};
    const Span ins[] = {{q, qb, "q"}, {k, kvb, "k"}, {v, kvb, "v"}};
    st = check_no_alias(outs, ins);
    if (st != RA_OK) return st;
  }
  ra::AttnArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.q_bh_stride = q_stride_bh; a.kv_bh_stride = kv_stride_bh;
  a.q_dev_stride = 0; a.kv_blk_stride = 0;
  a.row_step = 1;
  a.o = o_part; a.lse = lse_part;
  a.o_bh_stride = c * d; a.lse_bh_stride = c;
  a.o_dev_stride = c * d; a.lse_dev_stride = c;
  a.c = (int)c; a.P = prob->P; a.BH = (int)(prob->B * prob->H);
  a.p_begin = p; a.n_dev = 1; a.kv_base = kv;
  a.r_begin = ra::ring_block(p, kv, prob->P);   // (p - kv) mod P: the round that brings block kv
  a.r_count = 1;
  a.layout = prob->layout; a.causal = prob->causal;
  a.scale = eff_scale(prob);
  a.o_f32 = 1;
  a.stats = stats; a.stats_single = 1;
  return launch_attn(prob, a, (hipStream_t)stream);
}

ra_status_t ra_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                     int64_t rows, int64_t d, void* stream) {
  if (rows < 0 || d <= 0) return fail(RA_E_INVAL, "rows must be >= 0 and d > 0");
  if (rows == 0) return ok();
  if (!o_acc || !lse_acc || !o_part || !lse_part) return fail(RA_E_INVAL, "pointers must not be NULL");
  if (!aligned(o_acc, 4) || !aligned(lse_acc, 4) || !aligned(o_part, 4) || !aligned(lse_part, 4))
    return fail(RA_E_INVAL, "pointers must be 4-byte aligned");
  if (d % 4 == 0 && (!aligned(o_acc, 16) || !aligned(o_part, 16)))
    return fail(RA_E_INVAL, "o_acc / o_part must be 16-byte aligned when d %% 4 == 0");
  if (rows > INT64_MAX / d / 4) return fail(RA_E_INVAL, "rows*d overflows");
  const char* a0 = (const char*)o_acc;
  const char* b0 = (const char*)o_part;
  const int64_t ob = rows * d * 4;
  if (a0 < b0 + ob && b0 < a0 + ob) return fail(RA_E_INVAL, "o_part overlaps o_acc");
  if ((const char*)lse_acc < (const char*)lse_part + rows * 4 && (const char*)lse_part < (const char*)lse_acc + rows * 4)
    return fail(RA_E_INVAL, "lse_part overlaps lse_acc");
  return hip_status(ra::launch_merge(o_acc, lse_acc, o_part, lse_part, rows, d, (hipStream_t)stream),
                    "merge kernel launch");
}

ra_status_t ra_forward(const ra_problem_t* prob, const void* q, const void* k, const void* v,
                       int32_t p_begin, int32_t p_end, void* o, int32_t o_dtype, float* lse,
                       ra_round_stats_t* stats, void* stream) {
  ra_status_t st = check_problem(prob);
  if (st != RA_OK) return st;
  if (p_begin < 0 || p_end > prob->P || p_begin >= p_end)
    return fail(RA_E_INVAL, "device range [%d, %d) must be non-empty inside [0, %d)", p_begin, p_end, prob->P);
  if (o_dtype != RA_BF16 && o_dtype != RA_F32) return fail(RA_E_INVAL, "unknown o_dtype %d", o_dtype);
  if (empty_problem(prob)) return ok();
  if (!q || !k || !v || !o) return fail(RA_E_INVAL, "q, k, v and o must not be NULL");
  const int64_t c = prob->n / prob->P;
  const int64_t d = prob->d;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
    return fail(RA_E_INVAL, "q, k and v must be 16-byte aligned");
  if (!aligned(o, o_dtype == RA_F32 ? 16 : 8) || (lse && !aligned(lse, 4)))
    return fail(RA_E_INVAL, "o must be 16-byte (f32) or 8-byte (bf16) aligned, lse 4-byte aligned");
  if (stats && !aligned(stats, 8)) return fail(RA_E_INVAL, "stats must be 8-byte aligned");
  const int64_t ndev = p_end - p_begin;
  {
    const int64_t BH = prob->B * prob->H;
    const int64_t in_b = BH * prob->n * d * elem_bytes(prob->dtype);
    const int64_t orows = prob->layout == RA_STRIPED_TOKENS ? prob->n : ndev * c;
    const Span outs[] = {{o, BH * orows * d * (o_dtype == RA_F32 ? 4 : 2), "o"}, {lse, BH * orows * 4, "lse"},
                         {stats, (int64_t)prob->P * prob->P * (int64_t)sizeof(ra_round_stats_t), "stats"}};
    const Span ins[] = {{q, in_b, "q"}, {k, in_b, "k"}, {v, in_b, "v"}};
    st = check_no_alias(outs, ins);
    if (st != RA_OK) return st;
  }
  ra::AttnArgs a{};
  a.k = k; a.v = v;
  a.q_bh_stride = prob->n * d; a.kv_bh_stride = prob->n * d;
  a.lse = lse;
  if (prob->layout == RA_STRIPED_TOKENS) {
    // Row y of device p's block is token y * P + p of the token-order tensors.
    a.q = (const char*)q + (int64_t)p_begin * d * elem_bytes(prob->dtype);
    a.q_dev_stride = d; a.kv_blk_stride = d; a.row_step = prob->P;
    a.o = (char*)o + (int64_t)p_begin * d * (o_dtype == RA_F32 ? 4 : 2);
    if (lse) a.lse = lse + p_begin;
    a.o_bh_stride = prob->n * d; a.lse_bh_stride = prob->n;
    a.o_dev_stride = d; a.lse_dev_stride = 1;
  } else {
    a.q = (const char*)q + (int64_t)p_begin * c * d * elem_bytes(prob->dtype);
    a.q_dev_stride = c * d; a.kv_blk_stride = c * d; a.row_step = 1;
    a.o = o;
    a.o_bh_stride = ndev * c * d; a.lse_bh_stride = ndev * c;
    a.o_dev_stride = c * d; a.lse_dev_stride = c;
  }
  a.c = (int)c; a.P = prob->P; a.BH = (int)(prob->B * prob->H);
  a.p_begin = p_begin; a.n_dev = (int)ndev; a.kv_base = 0;
  a.r_begin = 0; a.r_count = prob->P;
  a.layout = prob->layout == RA_CONTIGUOUS ? RA_CONTIGUOUS : RA_STRIPED; a.causal = prob->causal;
  a.scale = eff_scale(prob);
  a.o_f32 = o_dtype == RA_F32 ? 1 : 0;
  a.stats = stats; a.stats_single = 0;
  if (stats) {
    // the counts of rows p_begin..p_end-1 are this call's own: clear them on the stream first
    st = hip_status(ra::launch_zero_u64(reinterpret_cast<uint64_t*>(stats + (int64_t)p_begin * prob->P),
                                        ndev * prob->P * 4, (hipStream_t)stream),
                    "counter clear launch");
    if (st != RA_OK) return st;
  }
  return launch_attn(prob, a, (hipStream_t)stream);
}

ra_status_t ra_bwd_delta(const void* o, int32_t o_dtype, const void* dout, int32_t dout_dtype,
                         int64_t rows, int64_t d, float* delta, void* stream) {
  if (rows < 0 || d <= 0) return fail(RA_E_INVAL, "rows must be >= 0 and d > 0");
  if ((o_dtype != RA_BF16 && o_dtype != RA_F32) || (dout_dtype != RA_BF16 && dout_dtype != RA_F32))
    return fail(RA_E_INVAL, "o_dtype / dout_dtype must be RA_BF16 or RA_F32");
  if (rows == 0) return ok();
  if (!o || !dout || !delta) return fail(RA_E_INVAL, "o, dout and delta must not be NULL");
  const size_t ao = d % 4 == 0 ? (size_t)(4 * elem_bytes(o_dtype)) : (size_t)elem_bytes(o_dtype);
  const size_t ad = d % 4 == 0 ? (size_t)(4 * elem_bytes(dout_dtype)) : (size_t)elem_bytes(dout_dtype);
  if (!aligned(o, ao) || !aligned(dout, ad) || !aligned(delta, 4))
    return fail(RA_E_INVAL, "o / dout must be aligned to 4 elements when d %% 4 == 0 (else 1), delta to 4 bytes");
  if (rows > INT64_MAX / d / 4) return fail(RA_E_INVAL, "rows*d overflows");
  if (overlaps(delta, rows * 4, o, rows * d * elem_bytes(o_dtype)) ||
      overlaps(delta, rows * 4, dout, rows * d * elem_bytes(dout_dtype)))
    return fail(RA_E_INVAL, "delta must not overlap o or dout");
  return hip_status(ra::launch_delta(o, o_dtype == RA_F32, dout, dout_dtype == RA_F32, rows, d, delta,
                                     (hipStream_t)stream),
                    "delta kernel launch");
}

ra_status_t ra_backward_round(const ra_problem_t* prob, const void* q, const void* k,
                              const void* v, const void* dout, const float* lse,
                              const float* delta, int64_t q_stride_bh, int64_t do_stride_bh,
                              int64_t kv_stride_bh, int64_t row_stride_bh, int32_t p, int32_t kv,
                              float* dq_acc, float* dk_acc, float* dv_acc, void* stream) {
  ra_status_t st = ra_check(prob, p, kv);
  if (st != RA_OK) return st;
  st = check_block_layout(prob);
  if (st != RA_OK) return st;
  st = check_bwd_support(prob);
  if (st != RA_OK) return st;
  if (empty_problem(prob)) return ok();
  const int64_t c = prob->n / prob->P;
  const int64_t d = prob->d;
  if (!q || !k || !v || !dout || !lse || !delta || !dq_acc || !dk_acc || !dv_acc)
    return fail(RA_E_INVAL, "q, k, v, dout, lse, delta, dq_acc, dk_acc and dv_acc must not be NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) || !aligned(lse, 4) ||
      !aligned(delta, 4))
    return fail(RA_E_INVAL, "q, k, v and dout must be 16-byte aligned, lse and delta 4-byte aligned");
  const int64_t vec = 16 / elem_bytes(prob->dtype);
  if (q_stride_bh < 0 || do_stride_bh < 0 || kv_stride_bh < 0 || row_stride_bh < 0 || q_stride_bh % vec ||
      do_stride_bh % vec || kv_stride_bh % vec)
    return fail(RA_E_INVAL, "strides must be >= 0, q/dout/kv strides multiples of %lld elements", (long long)vec);
  const int64_t BH = prob->B * prob->H;
  if (BH > 1 && (q_stride_bh < c * d || do_stride_bh < c * d || kv_stride_bh < c * d || row_stride_bh < c))
    return fail(RA_E_INVAL, "strides must be at least c*d = %lld (q, dout, kv) and c = %lld (rows) elements",
                (long long)(c * d), (long long)c);
  const int64_t gbytes = BH * c * d * 4;
  st = check_grad_outputs(dq_acc, gbytes, dk_acc, dv_acc, gbytes);
  if (st != RA_OK) return st;
  {
    const int64_t eb = elem_bytes(prob->dtype);
    const int64_t qb = ((BH - 1) * q_stride_bh + c * d) * eb, dob = ((BH - 1) * do_stride_bh + c * d) * eb;
    const int64_t kvb = ((BH - 1) * kv_stride_bh + c * d) * eb, rb = ((BH - 1) * row_stride_bh + c) * 4;
    const Span outs[] = {{dq_acc, gbytes, "dq_acc"}, {dk_acc, gbytes, "dk_acc"}, {dv_acc, gbytes, "dv_acc"}};
    const Span ins[] = {{q, qb, "q"}, {k, kvb, "k"}, {v, kvb, "v"}, {dout, dob, "dout"}, {lse, rb, "lse"},
                        {delta, rb, "delta"}};
    st = check_no_alias(outs, ins);
    if (st != RA_OK) return st;
  }
  if (ra::round_mode(prob->layout, prob->causal, p, kv) == ra::MODE_SKIP) return ok();
  ra::BwdArgs a{};
  a.q = q; a.dout = dout; a.lse = lse; a.delta = delta; a.k = k; a.v = v;
  a.q_bh_stride = q_stride_bh; a.do_bh_stride = do_stride_bh;
  a.row_bh_stride = row_stride_bh; a.kv_bh_stride = kv_stride_bh;
  a.row_step = 1;
  a.dq = dq_acc; a.dq_bh_stride = c * d; a.dq_dev_stride = c * d;
  a.dk = dk_acc; a.dv = dv_acc; a.dkv_bh_stride = c * d; a.dkv_blk_stride = c * d;
  a.c = (int)c; a.P = prob->P; a.BH = (int)BH;
  a.p_begin = p; a.n_dev = 1;
  a.kv_base = kv; a.n_kv = 1;
  a.r_begin = ra::ring_block(p, kv, prob->P); a.r_count = 1;
  a.layout = prob->layout; a.causal = prob->causal;
  a.scale = eff_scale(prob);
  a.accumulate = 1;
  return launch_bwd(prob, a, (hipStream_t)stream);
}

ra_status_t ra_backward(const ra_problem_t* prob, const void* q, const void* k, const void* v,
                        const void* dout, const float* lse, const float* delta, int32_t p_begin,
                        int32_t p_end, float* dq, float* dk, float* dv, void* stream) {
  ra_status_t st = check_problem(prob);
  if (st != RA_OK) return st;
  st = check_bwd_support(prob);
  if (st != RA_OK) return st;
  if (p_begin < 0 || p_end > prob->P || p_begin >= p_end)
    return fail(RA_E_INVAL, "device range [%d, %d) must be non-empty inside [0, %d)", p_begin, p_end, prob->P);
  if (empty_problem(prob)) return ok();
  if (!q || !k || !v || !dout || !lse || !delta || !dq || !dk || !dv)
    return fail(RA_E_INVAL, "q, k, v, dout, lse, delta, dq, dk and dv must not be NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) || !aligned(lse, 4) ||
      !aligned(delta, 4))
    return fail(RA_E_INVAL, "q, k, v and dout must be 16-byte aligned, lse and delta 4-byte aligned");
  const int64_t c = prob->n / prob->P;
  const int64_t d = prob->d;
  const int64_t BH = prob->B * prob->H;
  const int64_t ndev = p_end - p_begin;
  const bool tokens = prob->layout == RA_STRIPED_TOKENS;
  const int64_t m = tokens ? prob->n : ndev * c;     // rows of dout, lse, delta and dq
  st = check_grad_outputs(dq, BH * m * d * 4, dk, dv, BH * prob->n * d * 4);
  if (st != RA_OK) return st;
  const int64_t eb = elem_bytes(prob->dtype);
  {
    const int64_t in_b = BH * prob->n * d * eb;
    const Span outs[] = {{dq, BH * m * d * 4, "dq"}, {dk, BH * prob->n * d * 4, "dk"},
                         {dv, BH * prob->n * d * 4, "dv"}};
    const Span ins[] = {{q, in_b, "q"}, {k, in_b, "k"}, {v, in_b, "v"}, {dout, BH * m * d * eb, "dout"},
                        {lse, BH * m * 4, "lse"}, {delta, BH * m * 4, "delta"}};
    st = check_no_alias(outs, ins);
    if (st != RA_OK) return st;
  }
  ra::BwdArgs a{};
  a.k = k; a.v = v;
  a.q_bh_stride = prob->n * d; a.do_bh_stride = m * d; a.row_bh_stride = m; a.kv_bh_stride = prob->n * d;
  a.dq_bh_stride = m * d;
  a.dk = dk; a.dv = dv; a.dkv_bh_stride = prob->n * d;
  if (tokens) {
    // Row y of device p's block is token y * P + p of the token-order tensors.
    const int64_t r0 = p_begin;
    a.q = (const char*)q + r0 * d * eb; a.dout = (const char*)dout + r0 * d * eb;
    a.lse = lse + r0; a.delta = delta + r0; a.dq = dq + r0 * d;
    a.q_dev_stride = d; a.do_dev_stride = d; a.row_dev_stride = 1; a.dq_dev_stride = d;
    a.kv_blk_stride = d; a.dkv_blk_stride = d;
    a.row_step = prob->P;
  } else {
    a.q = (const char*)q + (int64_t)p_begin * c * d * eb;
    a.dout = dout; a.lse = lse; a.delta = delta; a.dq = dq;
    a.q_dev_stride = c * d; a.do_dev_stride = c * d; a.row_dev_stride = c; a.dq_dev_stride = c * d;
    a.kv_blk_stride = c * d; a.dkv_blk_stride = c * d;
    a.row_step = 1;
  }
  a.c = (int)c; a.P = prob->P; a.BH = (int)BH;
  a.p_begin = p_begin; a.n_dev = (int)ndev;
  a.kv_base = 0; a.n_kv = prob->P;
  a.r_begin = 0; a.r_count = prob->P;
  a.layout = tokens ? RA_STRIPED : prob->layout; a.causal = prob->causal;
  a.scale = eff_scale(prob);
  a.accumulate = 0;
  return launch_bwd(prob, a, (hipStream_t)stream);
}

}  // extern "C"
