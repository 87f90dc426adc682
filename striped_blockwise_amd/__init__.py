"""Python binding of libra.so: blockwise Ring / Striped attention on MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP kernels behind the
C ABI (include/ra.h); PyTorch provides device memory and the current stream.  There is no
fallback: if libra.so is missing or the tensors are not on a GPU the calls raise.

Layout names: "contiguous" (device p owns tokens [p*c, (p+1)*c); Ring Attention review, step 1)
and "striped" (device p owns tokens p, p+P, ...; Striped Attention review, "分区策略对比"), with
the rows permuted into layout order by ``permute``; "striped_tokens" is the striped partition
with the tensors left in token order (``forward``, ``backward`` and ``permute_rope`` only): the
kernels read and write row y of device p's block at token y*P + p.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "CONTIGUOUS", "STRIPED", "STRIPED_TOKENS", "BF16", "F32", "lib", "abi_version", "check", "tile_shape",
    "permute", "permute_ids", "round", "merge", "forward", "new_stats", "bwd_delta",
    "backward_round", "backward", "permute_rope", "ROPE_INTERLEAVED", "ROPE_HALF", "RaError",
]

CONTIGUOUS, STRIPED, STRIPED_TOKENS = 0, 1, 2
BF16, F32 = 0, 1
ROPE_INTERLEAVED, ROPE_HALF = 0, 1
RA_OK, RA_E_INVAL, RA_E_UNSUPPORTED, RA_E_HIP = 0, -1, -2, -3

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libra.so")
_lib = None


class RaError(RuntimeError):
    """Raised for a non-zero status of the C ABI."""


class _Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("n", ctypes.c_int64),
                ("d", ctypes.c_int64), ("P", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("causal", ctypes.c_int32), ("scale", ctypes.c_float)]


_P = ctypes.POINTER(_Problem)
_vp = ctypes.c_void_p
_i32, _i64 = ctypes.c_int32, ctypes.c_int64

_SIGS = {
    "ra_abi_version": (_i32, []),
    "ra_last_error": (ctypes.c_char_p, []),
    "ra_check": (_i32, [_P, _i32, _i32]),
    "ra_tile_shape": (_i32, [_i32, _i64, ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "ra_permute": (_i32, [_vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp]),
    "ra_permute_ids": (_i32, [_vp, _vp, _i64, _i32, _i32, _vp]),
    "ra_round": (_i32, [_P, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp]),
    "ra_merge": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _vp]),
    "ra_forward": (_i32, [_P, _vp, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _vp, _vp]),
    "ra_permute_rope": (_i32, [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, ctypes.c_double, _i32,
                               _i32, _vp]),
    "ra_bwd_delta": (_i32, [_vp, _i32, _vp, _i32, _i64, _i64, _vp, _vp]),
    "ra_backward_round": (_i32, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i32, _i32,
                                 _vp, _vp, _vp, _vp]),
    "ra_backward": (_i32, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp]),
}


def lib():
    """Load libra.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RaError(f"{_LIB_PATH} not found: build it with `python -m striped_blockwise_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _raise(status: int, what: str):
    if status == RA_OK:
        return
    msg = lib().ra_last_error().decode(errors="replace")
    if status == RA_E_INVAL:
        raise ValueError(f"{what}: {msg}")
    if status == RA_E_UNSUPPORTED:
        raise NotImplementedError(f"{what}: {msg}")
    raise RaError(f"{what} (status {status}): {msg}")


def _layout(x) -> int:
    if isinstance(x, str):
        return {"contiguous": CONTIGUOUS, "ring": CONTIGUOUS, "striped": STRIPED,
                "striped_tokens": STRIPED_TOKENS}[x]
    return int(x)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return BF16
    if dt == torch.float32:
        return F32
    raise ValueError(f"unsupported dtype {dt} (bfloat16 or float32)")


def _problem(B, H, n, d, P, dtype, layout, causal, scale) -> _Problem:
    return _Problem(int(B), int(H), int(n), int(d), int(P), int(dtype), _layout(layout),
                    1 if causal else 0, float(scale))


def _gpu(*ts: torch.Tensor):
    dev = ts[0].device
    for t in ts:
        if t.device.type != "cuda":
            raise ValueError("tensors must be on a GPU (device 'cuda')")
        if t.device != dev:
            raise ValueError("tensors must be on the same GPU")
    return dev


def _check_out(t, shape, dtype, dev, name: str) -> None:
    """A caller-provided output must be exactly what the kernels write: the library checks sizes
    from the problem, not from the tensor, so a smaller buffer would be overrun."""
    if (not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape) or t.dtype != dtype
            or not t.is_contiguous() or t.device != dev):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {dev}")


def _check_stats(stats, numel: int, dev) -> None:
    if stats is not None and (stats.dtype != torch.int64 or stats.numel() < numel or not stats.is_contiguous()
                              or stats.device != dev):
        raise ValueError(f"stats must be a contiguous int64 tensor of >= {numel} elements on {dev}")


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def abi_version() -> int:
    return int(lib().ra_abi_version())


def check(B, H, n, d, P, dtype=BF16, layout=CONTIGUOUS, causal=True, scale=0.0, p=0, kv=0) -> None:
    """Host-only validation (no GPU needed); raises on a bad problem."""
    pr = _problem(B, H, n, d, P, dtype, layout, causal, scale)
    _raise(lib().ra_check(ctypes.byref(pr), int(p), int(kv)), "ra_check")


def tile_shape(dtype=BF16, d=128):
    tq, tk = _i32(), _i32()
    _raise(lib().ra_tile_shape(int(dtype), int(d), ctypes.byref(tq), ctypes.byref(tk)), "ra_tile_shape")
    return tq.value, tk.value


def permute(x: torch.Tensor, P: int, dim: int = -2, inverse: bool = False, out=None) -> torch.Tensor:
    """Striped permutation of the token axis ``dim`` of a contiguous GPU tensor.

    inverse=False: token order -> striped layout; inverse=True: striped layout -> token order.
    """
    _gpu(x)
    if not x.is_contiguous():
        raise ValueError("permute needs a contiguous tensor")
    dim = dim % x.dim()
    n = x.shape[dim]
    BH = 1
    for s in x.shape[:dim]:
        BH *= s
    row = x.element_size()
    for s in x.shape[dim + 1:]:
        row *= s
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must match x (shape, dtype) and be contiguous")
    _gpu(x, out)
    with torch.cuda.device(x.device):
        _raise(lib().ra_permute(_ptr(x), _ptr(out), BH, n, row, int(P), 1 if inverse else 0,
                                _vp(_stream(x.device))), "ra_permute")
    return out


def permute_ids(ids: torch.Tensor, P: int, inverse: bool = False, out=None) -> torch.Tensor:
    """Striped permutation of an int64 position-ID vector."""
    _gpu(ids)
    if ids.dtype != torch.int64 or ids.dim() != 1 or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous 1-D int64 tensor")
    if out is None:
        out = torch.empty_like(ids)
    _check_out(out, ids.shape, torch.int64, ids.device, "out")
    with torch.cuda.device(ids.device):
        _raise(lib().ra_permute_ids(_ptr(ids), _ptr(out), ids.numel(), int(P), 1 if inverse else 0,
                                    _vp(_stream(ids.device))), "ra_permute_ids")
    return out


def _block_strides(t: torch.Tensor, name: str):
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, c, d]")
    B, H, c, d = t.shape
    if t.stride(3) != 1 or (c > 1 and t.stride(2) != d):
        raise ValueError(f"{name}: rows must be contiguous (strides [.., .., d, 1])")
    if B * H > 1 and H > 1 and B > 1 and t.stride(0) != H * t.stride(1):
        raise ValueError(f"{name}: (b, h) matrices must be evenly strided")
    return t.stride(1) if H > 1 else (t.stride(0) if B > 1 else c * d)


def new_stats(P: int, device="cuda") -> torch.Tensor:
    """Zeroed device buffer of [P, P] ra_round_stats_t (4 uint64 each, as int64)."""
    return torch.zeros((P, P, 4), dtype=torch.int64, device=device)


def round(q_blk, k_blk, v_blk, P: int, p: int, kv: int, layout="contiguous", causal=True,
          scale: float = 0.0, stats=None, out=None):
    """One ring round: device p's query block against K/V block kv.

    q_blk, k_blk, v_blk: [B, H, c, d] views (bf16 or f32), rows contiguous (views into full
    [B, H, n, d] tensors are fine).  Returns (o_part [B,H,c,d] f32, lse_part [B,H,c] f32).
    stats: None or an int64 tensor with >= 4 elements (one ra_round_stats_t) to add counts to.
    """
    dev = _gpu(q_blk, k_blk, v_blk)
    B, H, c, d = q_blk.shape
    if k_blk.shape != q_blk.shape or v_blk.shape != q_blk.shape:
        raise ValueError("q, k, v blocks must have the same shape")
    if not (q_blk.dtype == k_blk.dtype == v_blk.dtype):
        raise ValueError("q, k, v must share a dtype")
    sq = _block_strides(q_blk, "q")
    sk = _block_strides(k_blk, "k")
    sv = _block_strides(v_blk, "v")
    if sk != sv:
        raise ValueError("k and v must have the same (b, h) stride")
    if out is None:
        o = torch.empty((B, H, c, d), dtype=torch.float32, device=dev)
        lse = torch.empty((B, H, c), dtype=torch.float32, device=dev)
    else:
        o, lse = out
        _check_out(o, (B, H, c, d), torch.float32, dev, "out[0]")
        _check_out(lse, (B, H, c), torch.float32, dev, "out[1]")
    _check_stats(stats, 4, dev)
    pr = _problem(B, H, c * P, d, P, _dtype_code(q_blk.dtype), layout, causal, scale)
    with torch.cuda.device(dev):
        _raise(lib().ra_round(ctypes.byref(pr), _ptr(q_blk), _ptr(k_blk), _ptr(v_blk), sq, sk,
                              int(p), int(kv), _ptr(o), _ptr(lse), _ptr(stats), _vp(_stream(dev))),
               "ra_round")
    return o, lse


def merge(o_acc, lse_acc, o_part, lse_part) -> None:
    """In-place log-sum-exp merge of a round partial into (o_acc, lse_acc); float32, contiguous."""
    _gpu(o_acc, lse_acc, o_part, lse_part)
    for t in (o_acc, lse_acc, o_part, lse_part):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("merge operands must be contiguous float32")
    d = o_acc.shape[-1]
    rows = lse_acc.numel()
    if o_acc.numel() != rows * d or o_part.shape != o_acc.shape or lse_part.shape != lse_acc.shape:
        raise ValueError("shape mismatch between accumulator and partial")
    with torch.cuda.device(o_acc.device):
        _raise(lib().ra_merge(_ptr(o_acc), _ptr(lse_acc), _ptr(o_part), _ptr(lse_part), rows, d,
                              _vp(_stream(o_acc.device))), "ra_merge")


def forward(q, k, v, P: int, layout="contiguous", causal=True, p_begin: int = 0, p_end=None,
            o_dtype=None, want_lse: bool = True, scale: float = 0.0, stats=None, out=None):
    """All P rounds for devices [p_begin, p_end), fused in one launch.

    q, k, v: contiguous [B, H, n, d] in layout order.  Returns (o, lse): o is
    [B, H, (p_end-p_begin)*c, d] in o_dtype (default: q's dtype), lse the matching float32
    log-sum-exp (None if want_lse is False).  stats: None or new_stats(P); the call clears the rows
    p_begin..p_end-1 of it on the stream and writes their counts there.
    layout "striped_tokens": q, k, v, o and lse in token order, o [B, H, n, d] and lse [B, H, n];
    rows of devices outside the range are left as they were (zeros when out is None).
    out: None or (o, lse) of those shapes, contiguous (lse may be None).
    """
    dev = _gpu(q, k, v)
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must be [B, H, n, d] of one shape")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    B, H, n, d = q.shape
    p_end = P if p_end is None else p_end
    c = n // P if P > 0 else 0
    tokens = _layout(layout) == STRIPED_TOKENS
    rows = n if tokens else max(0, p_end - p_begin) * c
    o_dtype = q.dtype if o_dtype is None else o_dtype
    if out is None:
        alloc = torch.zeros if tokens and (p_begin, p_end) != (0, P) else torch.empty
        o = alloc((B, H, rows, d), dtype=o_dtype, device=dev)
        lse = alloc((B, H, rows), dtype=torch.float32, device=dev) if want_lse else None
    else:
        o, lse = out
        _check_out(o, (B, H, rows, d), o_dtype, dev, "out[0]")
        if lse is not None:
            _check_out(lse, (B, H, rows), torch.float32, dev, "out[1]")
    _check_stats(stats, P * P * 4, dev)
    pr = _problem(B, H, n, d, P, _dtype_code(q.dtype), layout, causal, scale)
    with torch.cuda.device(dev):
        _raise(lib().ra_forward(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), int(p_begin), int(p_end),
                                _ptr(o), _dtype_code(o_dtype), _ptr(lse), _ptr(stats), _vp(_stream(dev))),
               "ra_forward")
    return o, lse


def _row_stride(t: torch.Tensor, name: str):
    if t.dim() != 3 or t.dtype != torch.float32:
        raise ValueError(f"{name} must be a float32 [B, H, c] tensor")
    B, H, c = t.shape
    if c > 1 and t.stride(2) != 1:
        raise ValueError(f"{name}: rows must be contiguous")
    if B > 1 and H > 1 and t.stride(0) != H * t.stride(1):
        raise ValueError(f"{name}: (b, h) vectors must be evenly strided")
    return t.stride(1) if H > 1 else (t.stride(0) if B > 1 else c)


def bwd_delta(o: torch.Tensor, dout: torch.Tensor, out=None) -> torch.Tensor:
    """Backward row term D = sum over the last dim of O * dO, as float32 of shape o.shape[:-1].

    o, dout: contiguous GPU tensors of one shape, bfloat16 or float32 each.
    """
    _gpu(o, dout)
    if o.shape != dout.shape or not (o.is_contiguous() and dout.is_contiguous()):
        raise ValueError("o and dout must be contiguous and of one shape")
    d = o.shape[-1]
    rows = o.numel() // d if d else 0
    if out is None:
        out = torch.empty(o.shape[:-1], dtype=torch.float32, device=o.device)
    else:
        _check_out(out, o.shape[:-1], torch.float32, o.device, "out")
    with torch.cuda.device(o.device):
        _raise(lib().ra_bwd_delta(_ptr(o), _dtype_code(o.dtype), _ptr(dout), _dtype_code(dout.dtype), rows, d,
                                  _ptr(out), _vp(_stream(o.device))), "ra_bwd_delta")
    return out


def backward_round(q_blk, k_blk, v_blk, dout_blk, lse_blk, delta_blk, P: int, p: int, kv: int,
                   layout="contiguous", causal=True, scale: float = 0.0, grads=None):
    """Backward of one ring round: device p's query block against K/V block kv.

    q_blk, dout_blk, k_blk, v_blk: [B, H, c, d] views (rows contiguous; k and v with one (b, h)
    stride); lse_blk, delta_blk: float32 [B, H, c] views (lse: the rows' final log-sum-exp).
    grads: None or (dq_acc, dk_acc, dv_acc), contiguous float32 [B, H, c, d] accumulators that
    the pair's contributions are added to (new zeroed ones when None).  Returns the three.
    """
    dev = _gpu(q_blk, k_blk, v_blk, dout_blk, lse_blk, delta_blk)
    B, H, c, d = q_blk.shape
    for t in (k_blk, v_blk, dout_blk):
        if t.shape != q_blk.shape or t.dtype != q_blk.dtype:
            raise ValueError("q, k, v and dout blocks must share a shape and dtype")
    sq = _block_strides(q_blk, "q")
    sdo = _block_strides(dout_blk, "dout")
    sk = _block_strides(k_blk, "k")
    if _block_strides(v_blk, "v") != sk:
        raise ValueError("k and v must have the same (b, h) stride")
    sr = _row_stride(lse_blk, "lse")
    if _row_stride(delta_blk, "delta") != sr or lse_blk.shape != (B, H, c) or delta_blk.shape != (B, H, c):
        raise ValueError("lse and delta must be [B, H, c] with the same (b, h) stride")
    if grads is None:
        grads = tuple(torch.zeros((B, H, c, d), dtype=torch.float32, device=dev) for _ in range(3))
    if len(grads) != 3:
        raise ValueError("grads must be (dq_acc, dk_acc, dv_acc)")
    for g, name in zip(grads, ("dq_acc", "dk_acc", "dv_acc")):
        _check_out(g, (B, H, c, d), torch.float32, dev, name)
    pr = _problem(B, H, c * P, d, P, _dtype_code(q_blk.dtype), layout, causal, scale)
    with torch.cuda.device(dev):
        _raise(lib().ra_backward_round(ctypes.byref(pr), _ptr(q_blk), _ptr(k_blk), _ptr(v_blk), _ptr(dout_blk),
                                       _ptr(lse_blk), _ptr(delta_blk), sq, sdo, sk, sr, int(p), int(kv),
                                       _ptr(grads[0]), _ptr(grads[1]), _ptr(grads[2]), _vp(_stream(dev))),
               "ra_backward_round")
    return grads


def backward(q, k, v, dout, lse, P: int, layout="contiguous", causal=True, p_begin: int = 0,
             p_end=None, delta=None, o=None, scale: float = 0.0, out=None):
    """Gradients of forward(q, k, v, ...) for devices [p_begin, p_end), all rounds fused.

    q, k, v: contiguous [B, H, n, d] in layout order; dout: [B, H, m, d], m = (p_end-p_begin)*c,
    same dtype as q; lse: float32 [B, H, m] from forward; delta: float32 [B, H, m] from
    bwd_delta, or None with o (forward's output) given to compute it.  Returns float32
    (dq [B, H, m, d], dk [B, H, n, d], dv [B, H, n, d]); dk and dv hold what the queries of
    the device range send to every key.
    layout "striped_tokens": all tensors in token order and m = n (dout, dq [B, H, n, d]; lse,
    delta [B, H, n]); dq rows of devices outside the range are left as they were (zeros when
    out is None).
    """
    dev = _gpu(q, k, v, dout, lse)
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must be [B, H, n, d] of one shape")
    if not all(t.is_contiguous() for t in (q, k, v, dout, lse)):
        raise ValueError("q, k, v, dout and lse must be contiguous")
    if not (q.dtype == k.dtype == v.dtype == dout.dtype):
        raise ValueError("q, k, v and dout must share a dtype")
    B, H, n, d = q.shape
    p_end = P if p_end is None else p_end
    c = n // P if P > 0 else 0
    tokens = _layout(layout) == STRIPED_TOKENS
    m = n if tokens else max(0, p_end - p_begin) * c
    if dout.shape != (B, H, m, d) or lse.shape != (B, H, m) or lse.dtype != torch.float32:
        raise ValueError(f"dout must be [B, H, {m}, d] and lse float32 [B, H, {m}]")
    if delta is None:
        if o is None:
            raise ValueError("pass delta, or o to compute it")
        delta = bwd_delta(o, dout)
    if delta.shape != (B, H, m) or delta.dtype != torch.float32 or not delta.is_contiguous():
        raise ValueError(f"delta must be contiguous float32 [B, H, {m}]")
    if out is None:
        dq = (torch.zeros if tokens and (p_begin, p_end) != (0, P) else torch.empty)(
            (B, H, m, d), dtype=torch.float32, device=dev)
        dk = torch.empty((B, H, n, d), dtype=torch.float32, device=dev)
        dv = torch.empty((B, H, n, d), dtype=torch.float32, device=dev)
    else:
        dq, dk, dv = out
        _check_out(dq, (B, H, m, d), torch.float32, dev, "out[0] (dq)")
        _check_out(dk, (B, H, n, d), torch.float32, dev, "out[1] (dk)")
        _check_out(dv, (B, H, n, d), torch.float32, dev, "out[2] (dv)")
    _gpu(q, dq, dk, dv, delta)
    pr = _problem(B, H, n, d, P, _dtype_code(q.dtype), layout, causal, scale)
    with torch.cuda.device(dev):
        _raise(lib().ra_backward(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta),
                                 int(p_begin), int(p_end), _ptr(dq), _ptr(dk), _ptr(dv), _vp(_stream(dev))),
               "ra_backward")
    return dq, dk, dv


def permute_rope(x: torch.Tensor, P: int, layout="striped", pos=None, base: float = 10000.0,
                 style="interleaved", inverse: bool = False, out=None) -> torch.Tensor:
    """Rotary position embedding fused with the striped permutation of the token axis.

    x: contiguous GPU tensor [..., n, d] (bfloat16 or float32, d even), token order.  Returns
    the rows rotated by their token's position (pos: int64 [n] on the GPU, default 0..n-1) in
    the layout order; inverse=True applies the adjoint (layout -> token order, rotated back),
    which carries gradients dQ / dK back through it.  style: "interleaved" (pairs 2i, 2i+1) or
    "half" (pairs i, i + d/2).
    """
    _gpu(x)
    if not x.is_contiguous() or x.dim() < 2:
        raise ValueError("x must be a contiguous [..., n, d] tensor")
    n, d = x.shape[-2], x.shape[-1]
    BH = x.numel() // (n * d) if n * d else 0
    if pos is not None:
        _gpu(x, pos)
        if pos.dtype != torch.int64 or pos.shape != (n,) or not pos.is_contiguous():
            raise ValueError("pos must be a contiguous int64 tensor of shape [n]")
    if isinstance(style, str):
        style = {"interleaved": ROPE_INTERLEAVED, "half": ROPE_HALF}[style]
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must match x (shape, dtype) and be contiguous")
    _gpu(x, out)
    with torch.cuda.device(x.device):
        _raise(lib().ra_permute_rope(_ptr(x), _ptr(out), _ptr(pos), BH, n, d, _dtype_code(x.dtype), int(P),
                                     _layout(layout), float(base), int(style), 1 if inverse else 0,
                                     _vp(_stream(x.device))), "ra_permute_rope")
    return out


# The C entry points' own names, for callers who follow include/ra.h (ra_last_error is reported
# inside the exceptions instead).
ra_abi_version = abi_version
ra_check = check
ra_tile_shape = tile_shape
ra_permute = permute
ra_permute_ids = permute_ids
ra_permute_rope = permute_rope
ra_round = round
ra_merge = merge
ra_forward = forward
ra_bwd_delta = bwd_delta
ra_backward_round = backward_round
ra_backward = backward
__all__ += ["ra_abi_version", "ra_check", "ra_tile_shape", "ra_permute", "ra_permute_ids", "ra_permute_rope",
            "ra_round", "ra_merge", "ra_forward", "ra_bwd_delta", "ra_backward_round", "ra_backward"]
