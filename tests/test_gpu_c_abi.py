"""A C program drives the striped forward through the C ABI alone (HIP runtime C API for memory,
include/ra.h for the work) and its output is compared with the fp64 oracle.

The program reads bf16 Q, K, V from files written here, permutes them into the striped layout
with ra_permute, runs ra_forward for every device, un-permutes O and LSE with ra_permute, and
writes them back; no Python or PyTorch is in that path.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from oracle import attention as OA
from tests._gpu_util import compare, need_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SRC = r'''
#include <stdio.h>
#include <stdlib.h>
#include <hip/hip_runtime_api.h>
#include "ra.h"

static int rd(const char* path, void* buf, size_t n) {
  FILE* f = fopen(path, "rb"); if (!f) return 1;
  size_t got = fread(buf, 1, n, f); fclose(f); return got != n;
}
static int wr(const char* path, const void* buf, size_t n) {
  FILE* f = fopen(path, "wb"); if (!f) return 1;
  size_t put = fwrite(buf, 1, n, f); fclose(f); return put != n;
}
#define CK(x) do { if ((x) != 0) { fprintf(stderr, "failed: %s (%s)\n", #x, ra_last_error()); return 1; } } while (0)

int main(int argc, char** argv) {
  if (argc != 6) return 2;
  const char* dir = argv[1];
  const int64_t H = atoll(argv[2]), n = atoll(argv[3]), d = atoll(argv[4]);
  const int32_t P = atoi(argv[5]);
  const size_t elems = (size_t)H * n * d, bytes = elems * 2;
  char path[4096];
  void* host = malloc(bytes);
  void *q, *k, *v, *qs, *ks, *vs, *os_, *o, *ls, *l;
  CK(hipMalloc(&q, bytes)); CK(hipMalloc(&k, bytes)); CK(hipMalloc(&v, bytes));
  CK(hipMalloc(&qs, bytes)); CK(hipMalloc(&ks, bytes)); CK(hipMalloc(&vs, bytes));
  CK(hipMalloc(&os_, elems * 4)); CK(hipMalloc(&o, elems * 4));
  CK(hipMalloc(&ls, (size_t)H * n * 4)); CK(hipMalloc(&l, (size_t)H * n * 4));
  const char* names[3] = {"q.bin", "k.bin", "v.bin"};
  void* dev[3] = {q, k, v};
  void* per[3] = {qs, ks, vs};
  for (int i = 0; i < 3; ++i) {
    snprintf(path, sizeof path, "%s/%s", dir, names[i]);
    CK(rd(path, host, bytes));
    CK(hipMemcpy(dev[i], host, bytes, hipMemcpyHostToDevice));
    CK(ra_permute(dev[i], per[i], H, n, d * 2, P, 0, NULL));
  }
  ra_problem_t pr = {1, H, n, d, P, RA_BF16, RA_STRIPED, 1, 0.0f};
  CK(ra_forward(&pr, qs, ks, vs, 0, P, os_, RA_F32, (float*)ls, NULL, NULL));
  CK(ra_permute(os_, o, H, n, d * 4, P, 1, NULL));
  CK(ra_permute(ls, l, H, n, 4, P, 1, NULL));
  CK(hipDeviceSynchronize());
  float* out = (float*)malloc(elems * 4);
  CK(hipMemcpy(out, o, elems * 4, hipMemcpyDeviceToHost));
  snprintf(path, sizeof path, "%s/o.bin", dir); CK(wr(path, out, elems * 4));
  CK(hipMemcpy(out, l, (size_t)H * n * 4, hipMemcpyDeviceToHost));
  snprintf(path, sizeof path, "%s/lse.bin", dir); CK(wr(path, out, (size_t)H * n * 4));
  printf("ok\n");
  return 0;
}
'''


def test_c_program_drives_the_striped_forward(tmp_path):
    need_gpu()
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    H, P, c, d = 2, 4, 300, 128
    n = P * c
    g = torch.Generator().manual_seed(31)
    q, k, v = (torch.randn((1, H, n, d), generator=g).mul(0.5).to(torch.bfloat16) for _ in range(3))
    for name, t in (("q", q), ("k", k), ("v", v)):
        t.contiguous().view(torch.int16).numpy().tofile(tmp_path / f"{name}.bin")
    src = tmp_path / "drive.c"
    src.write_text(C_SRC)
    exe = tmp_path / "drive"
    libdir = os.path.join(ROOT, "striped_blockwise_amd")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    subprocess.run([gcc, "-std=c99", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(rocm, "include"), str(src), "-L", libdir, "-lra",
                    "-L", os.path.join(rocm, "lib"), "-lamdhip64",
                    f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-o", str(exe)], check=True)
    print("[c-abi] running the C program", flush=True)
    out = subprocess.run([str(exe), str(tmp_path), str(H), str(n), str(d), str(P)], capture_output=True,
                         text=True, timeout=120)
    assert out.returncode == 0, (out.returncode, out.stdout, out.stderr)
    o = np.fromfile(tmp_path / "o.bin", dtype=np.float32).reshape(1, H, n, d)
    lse = np.fromfile(tmp_path / "lse.bin", dtype=np.float32).reshape(1, H, n)
    o_ref, l_ref = OA.attention(q, k, v, True)
    compare(o, lse, o_ref, l_ref, "bf16", "C program, striped, token order after un-permute")
