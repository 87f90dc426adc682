"""CPU-only checks of the C ABI: the library loads, exports every declared symbol, and rejects
bad arguments on the host before anything is launched (no GPU is touched)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ra.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def ra():
    import striped_blockwise_amd as m
    try:
        m.lib()
    except m.RaError as e:
        pytest.fail(f"libra.so is not built: {e}")
    return m


def test_header_declares_the_boundary():
    names = _declared()
    for want in ("ra_abi_version", "ra_last_error", "ra_check", "ra_tile_shape", "ra_permute",
                 "ra_permute_ids", "ra_round", "ra_merge", "ra_forward", "ra_bwd_delta",
                 "ra_backward_round", "ra_backward", "ra_permute_rope"):
        assert want in names


def test_library_exports_every_declared_symbol(ra):
    L = ra.lib()
    for name in _declared():
        assert hasattr(L, name), name
        assert isinstance(getattr(L, name), ctypes._CFuncPtr)


def test_abi_version_and_tiles(ra):
    assert ra.abi_version() == 5
    tq, tk = ra.tile_shape(ra.BF16, 128)
    assert tq > 0 and tk > 0 and tq % 32 == 0 and tk % 16 == 0
    assert ra.tile_shape(ra.F32, 64)[0] > 0
    with pytest.raises(NotImplementedError):
        ra.tile_shape(ra.BF16, 64)
    with pytest.raises(ValueError):
        ra.tile_shape(7, 128)


@pytest.mark.parametrize("kw,exc,msg", [
    (dict(n=10, P=4), ValueError, "multiple of P"),
    (dict(P=0), ValueError, "P must be"),
    (dict(p=4), ValueError, "p=4"),
    (dict(kv=-1), ValueError, "kv=-1"),
    (dict(d=96), NotImplementedError, "head dim 96"),
    (dict(d=0), ValueError, "head dim d"),
    (dict(dtype=5), ValueError, "dtype"),
    (dict(layout=3), ValueError, "layout"),
    (dict(layout=2, n=1 << 17, P=1 << 17), ValueError, "P <= 65536"),
    (dict(scale=float("nan")), ValueError, "scale"),
    (dict(B=-1), ValueError, ">= 0"),
    (dict(n=1 << 40, P=1), ValueError, "too large"),
])
def test_check_rejects(ra, kw, exc, msg):
    args = dict(B=1, H=8, n=8192, d=128, P=4, dtype=ra.BF16, layout=ra.STRIPED, causal=True,
                scale=0.0, p=0, kv=0)
    args.update(kw)
    with pytest.raises(exc, match=re.escape(msg)):
        ra.check(**args)


def test_check_accepts_every_workload(ra):
    import workloads
    for w in workloads.WORKLOADS.values():
        dt = ra.F32 if w.dtype == "f32" else ra.BF16
        for layout in (ra.CONTIGUOUS, ra.STRIPED, ra.STRIPED_TOKENS):
            ra.check(w.B, w.H, w.n, w.d, w.P, dt, layout, True, 0.0, p=w.P - 1, kv=0)
    ra.check(0, 8, 0, 128, 4)            # empty problems are valid


def test_raw_abi_rejects_null_and_bad_sizes_without_gpu(ra):
    L = ra.lib()
    assert L.ra_permute(None, None, 1, 16, 256, 4, 0, None) == -1
    assert b"NULL" in L.ra_last_error()
    assert L.ra_permute(None, None, 1, 18, 256, 4, 0, None) == -1       # n % P
    assert L.ra_permute(None, None, 1, 16, 6, 4, 0, None) == -1         # row_bytes % 4
    assert L.ra_permute(None, None, 0, 16, 256, 4, 0, None) == 0        # empty: no-op
    assert L.ra_last_error() == b""
    assert L.ra_merge(None, None, None, None, 0, 128, None) == 0        # empty: no-op
    assert L.ra_merge(None, None, None, None, 4, 128, None) == -1
    pr = ra._problem(1, 1, 256, 64, 4, ra.F32, ra.CONTIGUOUS, True, 0.0)
    assert L.ra_round(ctypes.byref(pr), None, None, None, 0, 0, 0, 0, None, None, None, None) == -1
    assert L.ra_forward(ctypes.byref(pr), None, None, None, 0, 4, None, ra.F32, None, None, None) == -1
    assert L.ra_forward(ctypes.byref(pr), None, None, None, 2, 1, None, ra.F32, None, None, None) == -1
    assert b"device range" in L.ra_last_error()
    empty = ra._problem(1, 1, 0, 64, 4, ra.F32, ra.CONTIGUOUS, True, 0.0)
    assert L.ra_forward(ctypes.byref(empty), None, None, None, 0, 4, None, ra.F32, None, None, None) == 0
    bad = ra._problem(1, 1, 256, 64, 4, ra.F32, ra.CONTIGUOUS, True, 0.0)
    bad.causal = 2
    assert L.ra_check(ctypes.byref(bad), 0, 0) == -1 and b"causal" in L.ra_last_error()
    # misaligned pointer (never dereferenced: validation fails first)
    assert L.ra_permute(ctypes.c_void_p(2), ctypes.c_void_p(4096), 1, 16, 8, 4, 0, None) == -1


def test_backward_host_validation(ra):
    """The backward entry points validate on the host and enqueue nothing on bad input."""
    L = ra.lib()
    N = None
    assert L.ra_bwd_delta(N, ra.BF16, N, ra.BF16, 0, 128, N, N) == 0            # empty: no-op
    assert L.ra_bwd_delta(N, ra.BF16, N, ra.BF16, 4, 128, N, N) == -1
    assert L.ra_bwd_delta(N, 7, N, ra.BF16, 4, 128, N, N) == -1 and b"dtype" in L.ra_last_error()
    assert L.ra_bwd_delta(N, ra.BF16, N, ra.BF16, 4, 0, N, N) == -1
    pr = ra._problem(1, 1, 256, 128, 4, ra.BF16, ra.STRIPED, True, 0.0)
    args13 = (N,) * 6
    assert L.ra_backward(ctypes.byref(pr), *args13, 0, 4, N, N, N, N) == -1         # NULL pointers
    assert L.ra_backward(ctypes.byref(pr), *args13, 3, 3, N, N, N, N) == -1
    assert b"device range" in L.ra_last_error()
    assert L.ra_backward_round(ctypes.byref(pr), *args13, 0, 0, 0, 0, 4, 0, N, N, N, N) == -1   # p = 4
    assert L.ra_backward_round(ctypes.byref(pr), *args13, 0, 0, 0, 0, 1, 0, N, N, N, N) == -1   # NULL
    bad_d = ra._problem(1, 1, 256, 64, 4, ra.BF16, ra.STRIPED, True, 0.0)
    assert L.ra_backward(ctypes.byref(bad_d), *args13, 0, 4, N, N, N, N) == -2       # bf16 d=64
    empty = ra._problem(1, 0, 256, 128, 4, ra.BF16, ra.STRIPED, True, 0.0)
    assert L.ra_backward(ctypes.byref(empty), *args13, 0, 4, N, N, N, N) == 0
    assert L.ra_backward_round(ctypes.byref(empty), *args13, 0, 0, 0, 0, 1, 0, N, N, N, N) == 0


def test_token_order_layout_host_validation(ra):
    """RA_STRIPED_TOKENS is accepted by ra_forward's and ra_backward's validation and refused
    (unsupported, nothing launched) by the per-round entry points."""
    L = ra.lib()
    N = None
    pr = ra._problem(1, 1, 256, 128, 4, ra.BF16, ra.STRIPED_TOKENS, True, 0.0)
    assert L.ra_check(ctypes.byref(pr), 3, 1) == 0
    assert L.ra_forward(ctypes.byref(pr), N, N, N, 0, 4, N, ra.BF16, N, N, N) == -1     # NULL, not layout
    assert b"NULL" in L.ra_last_error()
    assert L.ra_round(ctypes.byref(pr), N, N, N, 0, 0, 0, 0, N, N, N, N) == -2
    assert b"layout order" in L.ra_last_error()
    assert L.ra_backward(ctypes.byref(pr), *(N,) * 6, 0, 4, N, N, N, N) == -1        # NULL, not layout
    assert b"NULL" in L.ra_last_error()
    assert L.ra_backward_round(ctypes.byref(pr), *(N,) * 6, 0, 0, 0, 0, 1, 0, N, N, N, N) == -2


def test_rope_host_validation(ra):
    L = ra.lib()
    N = None
    args = lambda **kw: [kw.get(k, v) for k, v in (("src", N), ("dst", N), ("pos", N), ("BH", 1), ("n", 16),
                                                   ("d", 8), ("dtype", ra.BF16), ("P", 4), ("layout", ra.STRIPED),
                                                   ("base", 10000.0), ("style", ra.ROPE_INTERLEAVED),
                                                   ("inverse", 0), ("stream", N))]
    assert L.ra_permute_rope(*args(n=0)) == 0                       # empty: no-op
    assert L.ra_permute_rope(*args()) == -1 and b"NULL" in L.ra_last_error()
    assert L.ra_permute_rope(*args(d=7)) == -1 and b"even" in L.ra_last_error()
    assert L.ra_permute_rope(*args(style=5)) == -1 and b"style" in L.ra_last_error()
    assert L.ra_permute_rope(*args(n=18)) == -1 and b"multiple of P" in L.ra_last_error()
    assert L.ra_permute_rope(*args(base=-1.0)) == -1
    assert L.ra_permute_rope(*args(dtype=9)) == -1
    assert L.ra_permute_rope(*args(layout=3)) == -1 and b"layout" in L.ra_last_error()
    assert L.ra_permute_rope(*args(layout=ra.STRIPED_TOKENS)) == -1 and b"NULL" in L.ra_last_error()


def test_binding_refuses_cpu_tensors(ra):
    x = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        ra.forward(x, x, x, 4)
    with pytest.raises(ValueError, match="GPU"):
        ra.permute(x, 4)
    with pytest.raises(ValueError, match="GPU"):
        ra.backward(x, x, x, x, torch.zeros((1, 1, 64)), 4, delta=torch.zeros((1, 1, 64)))


def test_product_package_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "striped_blockwise_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), f
                assert "oracle/" not in text and "import workloads" not in text, f


def test_header_is_plain_c_and_links(tmp_path, ra):
    """include/ra.h compiles as C99, and a C program links against libra.so and runs the
    host-only entry points (no GPU needed): the boundary is usable without C++ or Python."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "use_ra.c"
    src.write_text(r'''
#include <stdio.h>
#include <string.h>
#include "ra.h"
int main(void) {
  ra_problem_t pr;
  memset(&pr, 0, sizeof pr);
  pr.B = 1; pr.H = 8; pr.n = 8192; pr.d = 128; pr.P = 4;
  pr.dtype = RA_BF16; pr.layout = RA_STRIPED_TOKENS; pr.causal = 1; pr.scale = 0.0f;
  if (ra_abi_version() != RA_ABI_VERSION) return 1;
  if (ra_check(&pr, 3, 0) != RA_OK) return 2;
  pr.n = 8190;                                   /* not a multiple of P */
  if (ra_check(&pr, 0, 0) != RA_E_INVAL) return 3;
  if (strstr(ra_last_error(), "multiple of P") == NULL) return 4;
  int32_t tq = 0, tk = 0;
  if (ra_tile_shape(RA_BF16, 128, &tq, &tk) != RA_OK || tq <= 0 || tk <= 0) return 5;
  if (ra_tile_shape(RA_BF16, 96, &tq, &tk) != RA_E_UNSUPPORTED) return 6;
  printf("ok %d %d\n", tq, tk);
  return 0;
}
''')
    exe = tmp_path / "use_ra"
    libdir = os.path.join(ROOT, "striped_blockwise_amd")
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                    "-L", libdir, "-lra", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, (out.returncode, out.stdout, out.stderr)
    assert out.stdout.startswith("ok ")


def test_binding_offers_every_c_entry_point_by_name(ra):
    """Every function the header declares has a binding of the same name (ra_last_error's text
    arrives in the exceptions)."""
    import re as _re
    names = _re.findall(r"^\S.*?\b(ra_\w+)\(", open(os.path.join(ROOT, "include", "ra.h")).read(), _re.M)
    assert names, "no declarations found"
    for name in names:
        if name == "ra_last_error":
            continue
        assert callable(getattr(ra, name, None)), name
        assert name in ra.__all__, name


def test_outputs_may_not_alias_inputs(ra):
    """Every attention and gradient entry point refuses outputs that overlap an input or another
    output, on the host, before anything is launched.  The addresses are never dereferenced:
    each call fails validation first."""
    L = ra.lib()
    V = ctypes.c_void_p
    MB = 1 << 20
    base = [V(0x40000000 + i * 64 * MB) for i in range(12)]      # disjoint 64 MB ranges
    q, k, v, o, lse, st, do, de, dq, dk, dv, x = base
    inside = lambda p, off=4096: V(p.value + off)
    pr = ra._problem(1, 2, 256, 128, 4, ra.BF16, ra.STRIPED, True, 0.0)
    c, d = 64, 128
    # ra_round: o_part inside q, lse_part inside v, stats inside k, o_part over lse_part
    assert L.ra_round(ctypes.byref(pr), q, k, v, c * d, c * d, 1, 0, inside(q), lse, None, None) == -1
    assert b"o_part overlaps input q" in L.ra_last_error()
    assert L.ra_round(ctypes.byref(pr), q, k, v, c * d, c * d, 1, 0, o, inside(v), None, None) == -1
    assert b"lse_part overlaps input v" in L.ra_last_error()
    assert L.ra_round(ctypes.byref(pr), q, k, v, c * d, c * d, 1, 0, o, lse, inside(k, 256), None) == -1
    assert b"stats overlaps input k" in L.ra_last_error()
    assert L.ra_round(ctypes.byref(pr), q, k, v, c * d, c * d, 1, 0, o, inside(o, 1024), None, None) == -1
    assert b"outputs o_part and lse_part overlap" in L.ra_last_error()
    # ra_forward: o inside k; lse inside q; stats inside o; q == k == v is allowed (checked on a
    # failing call: the only error left is the stats overlap)
    assert L.ra_forward(ctypes.byref(pr), q, k, v, 0, 4, inside(k), ra.BF16, lse, None, None) == -1
    assert b"o overlaps input k" in L.ra_last_error()
    assert L.ra_forward(ctypes.byref(pr), q, k, v, 0, 4, o, ra.BF16, inside(q, 64 * 1024 - 4), None, None) == -1
    assert b"lse overlaps input q" in L.ra_last_error()
    assert L.ra_forward(ctypes.byref(pr), q, q, q, 0, 4, o, ra.BF16, lse, inside(o, 8), None) == -1
    assert b"outputs o and stats overlap" in L.ra_last_error()
    tok = ra._problem(1, 2, 256, 128, 4, ra.BF16, ra.STRIPED_TOKENS, True, 0.0)
    assert L.ra_forward(ctypes.byref(tok), q, k, v, 3, 4, inside(v, 2 * 256 * 128 * 2 - 8), ra.BF16, lse,
                        None, None) == -1                        # token order: o spans all n rows
    assert b"o overlaps input v" in L.ra_last_error()
    # ra_backward: dq inside dout, dk inside lse, dv inside q
    args = lambda **kw: [kw.get(n, dflt) for n, dflt in (("q", q), ("k", k), ("v", v), ("do", do), ("lse", lse),
                                                          ("de", de))]
    assert L.ra_backward(ctypes.byref(pr), *args(), 0, 4, inside(do), dk, dv, None) == -1
    assert b"dq overlaps input dout" in L.ra_last_error()
    assert L.ra_backward(ctypes.byref(pr), *args(), 0, 4, dq, inside(lse, 0), dv, None) == -1
    assert b"dk overlaps input lse" in L.ra_last_error()
    assert L.ra_backward(ctypes.byref(pr), *args(), 0, 4, dq, dk, inside(q), None) == -1
    assert b"dv overlaps input q" in L.ra_last_error()
    # ra_backward_round: dv_acc inside k, dq_acc inside delta
    assert L.ra_backward_round(ctypes.byref(pr), *args(), c * d, c * d, c * d, c, 1, 0, dq, dk, inside(k),
                               None) == -1
    assert b"dv_acc overlaps input k" in L.ra_last_error()
    assert L.ra_backward_round(ctypes.byref(pr), *args(), c * d, c * d, c * d, c, 1, 0, inside(de, 0), dk, dv,
                               None) == -1
    assert b"dq_acc overlaps input delta" in L.ra_last_error()


def test_bench_imports_the_oracle_only_in_cpu_baseline():
    """bench.py measures the product; the oracle is only timed, in the cpu_baseline leg."""
    import ast
    src = open(os.path.join(ROOT, "bench.py"), encoding="utf-8").read()
    tree = ast.parse(src)
    top = [n for n in tree.body if isinstance(n, (ast.Import, ast.ImportFrom))]
    for n in top:
        mods = [a.name for a in n.names] if isinstance(n, ast.Import) else [n.module or ""]
        assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), "module-level oracle import"
    for fn in ast.walk(tree):
        if not isinstance(fn, ast.FunctionDef):
            continue
        for n in ast.walk(fn):
            mods = []
            if isinstance(n, ast.Import):
                mods = [a.name for a in n.names]
            elif isinstance(n, ast.ImportFrom):
                mods = [n.module or ""]
            if any(m == "oracle" or m.startswith("oracle.") for m in mods):
                assert fn.name == "cpu_baseline", f"{fn.name} imports the oracle"
