#!/usr/bin/env python3
"""Benchmark: causal blockwise attention TFLOP/s on one MI355X, striped vs contiguous (ring).

Workload (default ``share_n256k``): one device's share of a 262144-token sequence split over
P = 8 (virtual) devices -- the query block of device 7 (c = 32768 tokens) against all 8 K/V
blocks, B = 1, H = 32, d = 128, bf16, causal.

One timed step = the striped hot path over that share: ra_forward for device 7 on the
token-order Q, K, V with layout RA_STRIPED_TOKENS (all 8 ring rounds fused, GetMask per round,
tile skipping; the striped permutation applied in the kernel's addressing: row y of block k is
token y*P + k, and O / LSE are written back to token rows y*P + 7).
``value`` is useful causal TFLOP/s of the step: 4 * d * (unmasked query-key pairs) * B * H
flops divided by the step time (masked halves of diagonal tiles and softmax work excluded).

Also measured in the same run (reported as extra fields, never as ``value``):
  * ring: the contiguous-layout forward for device 7 (most causal work of that layout);
  * per-round ra_round times for device 7 in both layouts and their ratio;
  * the same share through an explicit permutation pass: ra_permute of Q, K, V and of the
    position IDs, then ra_forward on the permuted tensors (RA_STRIPED);
  * the streamed path: 8 x (ra_round + ra_merge), with merge and permute GB/s;
  * backward: ra_backward (dQ, dK, dV) of the same share in both layouts, useful TFLOP/s;
  * the 8K-token sequence (P = 4): every (device, round) ra_round, and per round the slowest
    device's time in both layouts (the emulated ring's round time) and their ratio;
  * roofline of the dominant kernel (the fused bf16 forward) against the bf16 MFMA peak;
  * cpu_baseline: the fp64 CPU oracle on a bounded sample of the same share.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
       python bench.py --sweep      (striped/ring speedup vs sequence length; its own JSON line)
       python bench.py --backward   (backward of the device share, both layouts; its own JSON line)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal blockwise-attn TFLOP/s and % bf16 MFMA peak, ring vs striped, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, published
PMC_FILE = os.path.join(ROOT, "profiles", "k_attn_bf16_share_n256k_pmc.json")
# the fused forward's sources: the counters in PMC_FILE are used only while these are unchanged
KERNEL_SRCS = [os.path.join(ROOT, "striped_blockwise_amd", "csrc", f)
               for f in ("k_attn_bf16.hip", "bf16_tile.h", "tile_deal.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class ClockSampler:
    """Graphics clocks and socket power of the GPU while a kernel runs, from the driver's metrics
    table (amdsmi).  The table refreshes about once a second, so the sampler polls it from a host
    thread while the caller keeps the kernel running for a few seconds, and keeps only the fresh
    entries (a new accumulation counter) that arrive inside that window.  Best effort: ``result()``
    is None when amdsmi is missing or refuses access."""

    def __init__(self, torch, dev, period_s: float = 0.005):
        import threading
        self.samples = []
        self.period = period_s
        self.stop_ev = threading.Event()
        self.thread = None
        self.handle = None
        self.err = None
        self.window = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.smi = amdsmi
            handles = amdsmi.amdsmi_get_processor_handles()
            bus = getattr(torch.cuda.get_device_properties(dev), "pci_bus_id", None)
            for h in handles:
                try:
                    bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
                    if bus is not None and int(bdf.split(":")[1], 16) == int(bus):
                        self.handle = h
                        break
                except Exception:
                    continue
            if self.handle is None and len(handles) == 1:
                self.handle = handles[0]
            try:
                cap = amdsmi.amdsmi_get_power_cap_info(self.handle).get("power_cap")
                self.cap_w = cap / 1e6 if isinstance(cap, (int, float)) and cap > 1e5 else cap
            except Exception:
                self.cap_w = None
        except Exception as e:  # pragma: no cover - depends on the box
            self.err = repr(e)

    def _read(self):
        m = self.smi.amdsmi_get_gpu_metrics_info(self.handle)
        clks = [x for x in (m.get("current_gfxclks") or []) if isinstance(x, (int, float)) and 0 < x < 10000]
        if not clks and isinstance(m.get("current_gfxclk"), (int, float)):
            clks = [m["current_gfxclk"]]
        pw = m.get("current_socket_power")
        return m.get("accumulation_counter"), clks, pw if isinstance(pw, (int, float)) and 0 < pw < 100000 else None

    def _run(self):
        import time as _t
        last = None
        while not self.stop_ev.is_set():
            try:
                acc, clks, pw = self._read()
            except Exception as e:  # pragma: no cover
                self.err = repr(e)
                return
            if acc != last:
                self.samples.append((_t.perf_counter(), clks, pw))
                last = acc
            self.stop_ev.wait(self.period)

    def run_while(self, torch, fn, seconds: float = 3.0):
        """Keep calling fn() (enqueueing GPU work) for about `seconds`, sampling meanwhile."""
        import threading
        import time as _t
        if self.handle is None:
            return self
        self.thread = threading.Thread(target=self._run, daemon=True)
        self.thread.start()
        fn()
        torch.cuda.synchronize()
        t0 = _t.perf_counter()                 # the GPU has been busy since just before here
        while _t.perf_counter() - t0 < seconds:
            fn()
            fn()
            torch.cuda.synchronize()
        t1 = _t.perf_counter()
        self.stop_ev.set()
        self.thread.join()
        self.window = (t0, t1)
        return self

    def result(self, cus: int):
        if self.window is None:
            return None if self.err is None else {"error": self.err}
        t0, t1 = self.window
        fresh = [(c, p) for t, c, p in self.samples if t0 < t < t1 and c]
        if not fresh:
            return {"error": "no fresh metrics entry inside the window"}
        mhz = sum(sum(c) / len(c) for c, _ in fresh) / len(fresh)
        pw = [p for _, p in fresh if p]
        return {"sclk_mhz_mean": round(mhz, 1), "fresh_samples": len(fresh),
                "xcd_mhz_last": fresh[-1][0],
                "socket_power_w_mean": round(sum(pw) / len(pw), 1) if pw else None, "power_cap_w": self.cap_w,
                "peak_at_sclk_tflops": round(cus * mhz * 1e6 * 4096 / 1e12, 1),
                "source": "amdsmi gpu_metrics current_gfxclks (per XCD) and current_socket_power: the entries "
                          "refreshed while the measured launch ran back to back for ~3 s after its timed runs"}


def useful_pairs(layout: str, P: int, c: int, p: int, causal: bool = True) -> list:
    """Unmasked pairs of device p per ring round (closed form of the Striped Attention review's
    work formulas, with the diagonal block's c(c+1)/2)."""
    out = []
    for r in range(P):
        k = (p - r) % P
        if not causal:
            out.append(c * c)
        elif layout == "contiguous":
            out.append(c * c if k < p else (c * (c + 1) // 2 if k == p else 0))
        else:
            out.append(c * (c + 1) // 2 if k <= p else c * (c - 1) // 2)
    return out


def source_hash(paths) -> str:
    """sha256 of the files' bytes, concatenated in the given order."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from_profile(workload: str):
    """HBM bytes per launch of the fused forward from committed rocprofv3 --pmc counters, or
    None when the counters are missing, were taken on another workload or on a different
    kernel source."""
    try:
        with open(PMC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload_name") != workload:
        return None
    if rec.get("kernel_source_sha256") != source_hash(KERNEL_SRCS):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, layout: str, budget_s: float = 12.0):
    """Time the fp64 oracle on sampled query rows of device w.device (whole heads of keys)."""
    import numpy as np

    import workloads
    from oracle import attention as OA
    from oracle import ring as OR
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    P, c, p, d = w.P, w.c, w.device, w.d
    order = OR.layout_order(w.n, P, layout)
    rows = np.linspace(0, c - 1, 256).round().astype(np.int64)
    pos_q = order[p * c + rows]
    flops = 0.0
    elapsed = 0.0
    heads = 0
    for h in range(w.H):
        q, k, v = workloads.qkv(w, heads=[h])
        ql = OR.to_layout(q.double().numpy(), order)[:, :, p * c + rows]
        kl = OR.to_layout(k.double().numpy(), order)
        vl = OR.to_layout(v.double().numpy(), order)
        t0 = time.perf_counter()
        OA.attention(ql, kl, vl, True, pos_q=pos_q, pos_k=order)
        elapsed += time.perf_counter() - t0
        flops += 4.0 * d * float((pos_q + 1).sum())          # visible keys = position + 1
        heads += 1
        if elapsed >= budget_s:
            break
    full = 4.0 * d * w.B * w.H * sum(OR.work_closed_form(layout, p, OR.kv_block(p, r, P), c, True) for r in range(P))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    return {
        "value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "sample": f"{heads} head(s) x 256 evenly spaced query rows of device {p} ({layout}) against "
                  f"all {w.n} keys, fp64 NumPy; {flops:.3e} useful flops in {elapsed:.2f} s",
        "extrapolated_full_share_s": round(full / (flops / elapsed), 1),
        "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": model,
    }


def per_round_all_devices(torch, ra, dev, name: str = "seq_n8k", reps: int = 5):
    """Emulated ring rounds of a whole small sequence: every (device p, round r) ra_round timed
    alone (HIP events, a 512 MB write between reps so that no K/V block is served from cache),
    median over reps; a round of the emulated ring lasts as long as its slowest device."""
    import statistics

    import workloads
    w = workloads.get(name)
    P, c = w.P, w.c
    q, k, v = (t.to(dev) for t in workloads.qkv(w))
    lay = {"contiguous": (q, k, v), "striped": tuple(ra.permute(t, P) for t in (q, k, v))}
    flush = torch.empty(128 * 2 ** 20, dtype=torch.float32, device=dev)
    out = (torch.empty((w.B, w.H, c, w.d), dtype=torch.float32, device=dev),
           torch.empty((w.B, w.H, c), dtype=torch.float32, device=dev))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for layout, (qq, kk, vv) in lay.items():
        tmax = []
        for r in range(P):
            per_dev = []
            for p in range(P):
                kb = (p - r) % P                            # ring schedule: block of device p - r
                args_r = (qq[:, :, p * c:(p + 1) * c], kk[:, :, kb * c:(kb + 1) * c], vv[:, :, kb * c:(kb + 1) * c],
                          P, p, kb, layout, True)
                ts = []
                for _ in range(reps + 1):
                    flush.fill_(1.0)
                    a.record()
                    ra.round(*args_r, out=out)
                    b.record()
                    torch.cuda.synchronize()
                    ts.append(a.elapsed_time(b))
                per_dev.append(statistics.median(ts[1:]))
            tmax.append(max(per_dev))
        res[layout] = tmax
    ideal = []
    for r in range(P):
        pc = max(useful_pairs("contiguous", P, c, p)[r] for p in range(P))
        ps = max(useful_pairs("striped", P, c, p)[r] for p in range(P))
        ideal.append(round(pc / ps, 5))
    del flush, lay, q, k, v
    return {"workload": name, "n": w.n, "P": P, "H": w.H, "reps": reps,
            "round_max_ms_contiguous": [round(x, 4) for x in res["contiguous"]],
            "round_max_ms_striped": [round(x, 4) for x in res["striped"]],
            "speedup_striped_over_ring": [round(x / y, 4) for x, y in zip(res["contiguous"], res["striped"])],
            "ideal_speedup": ideal}


def sweep(torch, ra, dev, P: int = 8, H: int = 8, d: int = 128,
          lengths=(16384, 32768, 65536, 131072, 262144, 524288, 1048576)) -> int:
    """Fused-forward and backward time of the last device (most causal work under the
    contiguous layout) for both layouts as the sequence grows: the attention-only version of
    the Striped Attention review's speedup-vs-length table (which measures whole training
    steps).  The backward is ra_backward with D precomputed, as in the default line's field."""
    rows = []
    for n in lengths:
        c = n // P
        p = P - 1
        gen = torch.Generator(device=dev).manual_seed(n)
        q, k, v = (torch.randn((1, H, n, d), generator=gen, device=dev).mul_(0.5).to(torch.bfloat16)
                   for _ in range(3))
        qs, ks, vs = (ra.permute(t, P) for t in (q, k, v))
        o = torch.empty((1, H, c, d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((1, H, c), dtype=torch.float32, device=dev)
        dout = torch.randn((1, H, c, d), generator=gen, device=dev).to(torch.bfloat16)
        grads = (torch.empty((1, H, c, d), dtype=torch.float32, device=dev),
                 torch.empty((1, H, n, d), dtype=torch.float32, device=dev),
                 torch.empty((1, H, n, d), dtype=torch.float32, device=dev))
        res = {"n": n, "c": c}
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def timed(fn, reps):
            fn()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        for layout, args_ in (("contiguous", (q, k, v)), ("striped", (qs, ks, vs))):
            pairs = sum(useful_pairs(layout, P, c, p))
            reps = max(2, min(20, int(2e13 / (4.0 * d * H * pairs))))
            ms = timed(lambda: ra.forward(*args_, P, layout, True, p_begin=p, p_end=p + 1, out=(o, lse)), reps)
            res[layout + "_ms"] = round(ms, 4)
            res[layout + "_tflops"] = round(4.0 * d * H * pairs / (ms * 1e-3) / 1e12, 1)
            delta = ra.bwd_delta(o, dout)
            ms = timed(lambda: ra.backward(*args_, dout, lse, P, layout, True, p, p + 1, delta=delta, out=grads),
                       max(2, reps // 3))
            res["bwd_" + layout + "_ms"] = round(ms, 4)
            res["bwd_" + layout + "_tflops"] = round(10.0 * d * H * pairs / (ms * 1e-3) / 1e12, 1)
        res["speedup"] = round(res["contiguous_ms"] / res["striped_ms"], 4)
        res["bwd_speedup"] = round(res["bwd_contiguous_ms"] / res["bwd_striped_ms"], 4)
        res["ideal_speedup"] = round(sum(useful_pairs("contiguous", P, c, p)) / sum(useful_pairs("striped", P, c, p)), 5)
        log(f"[sweep] n={n}: forward contiguous {res['contiguous_ms']:.3f} ms, striped {res['striped_ms']:.3f} ms, "
            f"speedup {res['speedup']:.3f}; backward {res['bwd_contiguous_ms']:.3f} / {res['bwd_striped_ms']:.3f} ms, "
            f"speedup {res['bwd_speedup']:.3f} (ideal {res['ideal_speedup']})")
        rows.append(res)
        del q, k, v, qs, ks, vs, o, lse, dout, grads
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "striped/ring attention-only speedup vs sequence length (forward, backward), 1 GPU",
                      "config": {"P": P, "device": P - 1, "B": 1, "H": H, "d": d, "dtype": "bf16",
                                 "data": "synthetic N(0,1)*0.5 (GPU generator)"},
                      "sweep": rows}), flush=True)
    return 0


def backward_leg(torch, ra, w, striped_qkv, contiguous_qkv, flops_s, flops_c, p, reps=3):
    """Backward of one device share (training), both layouts.

    D = rowsum(O dO) is computed first (ra_bwd_delta), then ra_backward (the dK/dV kernel and
    the dQ kernel) is timed with HIP events.  Useful flops: 5 matrix products of 2 d flops per
    unmasked pair (S, dP, dV, dK, dQ), 2.5x the forward's.
    """
    dev = striped_qkv[0].device
    B, H, n, d = striped_qkv[0].shape
    P = w.P
    c = n // P
    gen = torch.Generator(device=dev).manual_seed(4)
    dout = torch.randn((B, H, c, d), device=dev, generator=gen).to(torch.bfloat16)
    o = torch.empty((B, H, c, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, c), dtype=torch.float32, device=dev)
    dq = torch.empty((B, H, c, d), dtype=torch.float32, device=dev)
    dk = torch.empty((B, H, n, d), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for layout, (qq, kk, vv), fl in (("striped", striped_qkv, flops_s), ("contiguous", contiguous_qkv, flops_c)):
        ra.forward(qq, kk, vv, P, layout, True, p_begin=p, p_end=p + 1, out=(o, lse))
        delta = ra.bwd_delta(o, dout)
        ra.backward(qq, kk, vv, dout, lse, P, layout, True, p, p + 1, delta=delta, out=(dq, dk, dv))
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            ra.backward(qq, kk, vv, dout, lse, P, layout, True, p, p + 1, delta=delta, out=(dq, dk, dv))
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        tf = 2.5 * fl / (ms * 1e-3) / 1e12
        out[layout] = {"ms": round(ms, 3), "useful_flops": 2.5 * fl, "tflops": round(tf, 3),
                       "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}
        log(f"[bench] backward {layout}: {ms:.2f} ms ({tf:.1f} TFLOP/s useful)")
    out["share_speedup_striped_over_ring"] = round(out["contiguous"]["ms"] / out["striped"]["ms"], 4)
    out["kernels"] = "k_bwd_dkv_bf16 then k_bwd_dq_bf16 (ra_backward); D precomputed by ra_bwd_delta"
    return out


def stress_leg(torch, ra, dev, name: str = "stress_n1m", reps: int = 5):
    """The million-token stress share (device 31 of P = 32, H = 8, 1% of key rows x8): the fused
    striped forward on token-order tensors, and the streamed form (32 x ra_round + ra_merge on
    the permuted blocks)."""
    import workloads
    w = workloads.get(name)
    P, c, d, H, B = w.P, w.c, w.d, w.H, w.B
    p = w.device if w.device is not None else P - 1
    log(f"[bench] generating inputs for {w.name} (n={w.n}, P={P}, H={H}) on the CPU")
    q, k, v = (t.to(dev) for t in workloads.qkv(w))
    flops = 4.0 * d * B * H * sum(useful_pairs("striped", P, c, p))
    o_t = torch.empty((B, H, w.n, d), dtype=torch.bfloat16, device=dev)
    lse_t = torch.empty((B, H, w.n), dtype=torch.float32, device=dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fwd = lambda: ra.forward(q, k, v, P, "striped_tokens", True, p_begin=p, p_end=p + 1, out=(o_t, lse_t))
    fwd()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a.record()
        fwd()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    ts.sort()
    f_ms = ts[len(ts) // 2]
    qs, ks, vs = (ra.permute(t, P) for t in (q, k, v))
    del q, k, v, o_t, lse_t
    po = torch.empty((B, H, c, d), dtype=torch.float32, device=dev)
    pl = torch.empty((B, H, c), dtype=torch.float32, device=dev)
    acc_o, acc_l = torch.empty_like(po), torch.empty_like(pl)

    def streamed():
        acc_o.zero_()
        acc_l.fill_(float("-inf"))
        for r in range(P):
            kb = (p - r) % P
            ra.round(qs[:, :, p * c:(p + 1) * c], ks[:, :, kb * c:(kb + 1) * c], vs[:, :, kb * c:(kb + 1) * c],
                     P, p, kb, "striped", True, out=(po, pl))
            ra.merge(acc_o, acc_l, po, pl)

    streamed()
    torch.cuda.synchronize()
    a.record()
    streamed()
    b.record()
    torch.cuda.synchronize()
    s_ms = a.elapsed_time(b)
    del qs, ks, vs, po, pl, acc_o, acc_l
    torch.cuda.empty_cache()
    out = {"workload": name, "n": w.n, "P": P, "c": c, "device": p, "H": H, "useful_flops": flops,
           "forward_ms": round(f_ms, 4), "forward_tflops": round(flops / (f_ms * 1e-3) / 1e12, 3),
           "forward_pct_peak": round(100 * flops / (f_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 3),
           "forward_timing": f"median of {reps}, ra_forward RA_STRIPED_TOKENS",
           "streamed_ms": round(s_ms, 4), "streamed_tflops": round(flops / (s_ms * 1e-3) / 1e12, 3),
           "streamed": "32 x (ra_round + ra_merge) on ra_permute'd blocks, one timed pass"}
    log(f"[bench] {name}: fused forward {f_ms:.2f} ms ({out['forward_tflops']:.1f} TFLOP/s); "
        f"streamed {s_ms:.2f} ms")
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="share_n256k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed striped steps (no other legs, no clock window): for profiler runs")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the default line: backward (dQ, dK, dV) of the device share, both layouts")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the default line: striped/ring speedup and TFLOP/s vs sequence length")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the ring's devices are emulated on a single MI355X "
              "(rounds run in order on one stream); --gpus must be 1.", file=sys.stderr)
        return 2

    import torch

    import striped_blockwise_amd as ra
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    ra.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.sweep:
        return sweep(torch, ra, dev)
    w = workloads.get(args.workload)
    P, c, d, H, B = w.P, w.c, w.d, w.H, w.B
    p = w.device if w.device is not None else P - 1
    BH = B * H

    log(f"[bench] generating inputs for {w.name} (n={w.n}, P={P}, H={H}, d={d}) on the CPU")
    t0 = time.perf_counter()
    q, k, v = (t.to(dev) for t in workloads.qkv(w))
    ids = workloads.positions(w.n).to(dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s")

    qs, ks, vs = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ids_s = torch.empty_like(ids)
    o = torch.empty((B, H, c, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, c), dtype=torch.float32, device=dev)
    o_t = torch.empty((B, H, w.n, d), dtype=torch.bfloat16, device=dev)     # token order: rows t = p mod P written
    lse_t = torch.empty((B, H, w.n), dtype=torch.float32, device=dev)

    pairs_s = useful_pairs("striped", P, c, p)
    pairs_c = useful_pairs("contiguous", P, c, p)
    flops_s = 4.0 * d * BH * sum(pairs_s)
    flops_c = 4.0 * d * BH * sum(pairs_c)

    if args.backward:
        for src, dst in ((q, qs), (k, ks), (v, vs)):
            ra.permute(src, P, out=dst)
        res = backward_leg(torch, ra, w, (qs, ks, vs), (q, k, v), flops_s, flops_c, p, reps=max(1, args.steps))
        print(json.dumps({"metric": "causal blockwise-attn backward TFLOP/s (useful: 10 d flops per unmasked pair), 1 GPU",
                          "config": {"workload": w.name, "n": w.n, "P": P, "c": c, "device": p, "B": B, "H": H,
                                     "d": d, "causal": True, "dout": "seeded N(0,1) bf16 (GPU generator)"},
                          "backward": res}), flush=True)
        return 0

    def step():
        e_f0.record()
        ra.forward(q, k, v, P, "striped_tokens", True, p_begin=p, p_end=p + 1, out=(o_t, lse_t))
        e_f1.record()

    def permuted_step(ev_fwd=None):
        ra.permute(q, P, out=qs)
        ra.permute(k, P, out=ks)
        ra.permute(v, P, out=vs)
        ra.permute_ids(ids, P, out=ids_s)
        if ev_fwd:
            ev_fwd[0].record()
        ra.forward(qs, ks, vs, P, "striped", True, p_begin=p, p_end=p + 1, out=(o, lse))
        if ev_fwd:
            ev_fwd[1].record()

    e_f0, e_f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps")

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    s0.record()
    for i in range(args.steps):
        e_f0, e_f1 = ev[i]
        step()
    s1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_mean = s0.elapsed_time(s1) / args.steps
    # the step is the one forward launch: its per-step event times, median over the K steps
    fwd_ms = sorted(a.elapsed_time(b) for a, b in ev)
    step_ms = fwd_ms[len(fwd_ms) // 2] if len(fwd_ms) % 2 else 0.5 * (fwd_ms[len(fwd_ms) // 2 - 1] + fwd_ms[len(fwd_ms) // 2])
    fwd_avg = sum(fwd_ms) / len(fwd_ms)
    value = flops_s / (step_ms * 1e-3) / 1e12
    achieved = flops_s / (fwd_avg * 1e-3) / 1e12
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    # clocks and power while the same launch runs (outside the timed steps)
    clock = None if args.no_extras else ClockSampler(torch, dev).run_while(torch, lambda: ra.forward(
        q, k, v, P, "striped_tokens", True, p_begin=p, p_end=p + 1, out=(o_t, lse_t))).result(cus)
    log(f"[bench] striped step median {step_ms:.2f} ms ({value:.1f} TFLOP/s), mean {step_mean:.2f} ms; forward "
        f"kernel mean {fwd_avg:.2f} ms ({achieved:.1f} TFLOP/s, {100 * achieved / PEAK_BF16_TFLOPS:.1f}% of bf16 peak)")
    if clock and "sclk_mhz_mean" in clock:
        log(f"[bench] sclk {clock['sclk_mhz_mean']:.0f} MHz ({clock['fresh_samples']} samples), socket power "
            f"{clock['socket_power_w_mean']} W of {clock['power_cap_w']} W: peak at that clock "
            f"{clock['peak_at_sclk_tflops']:.0f} TFLOP/s")
    else:
        log(f"[bench] clock: {clock}")

    result = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "ms_per_step_mean": round(step_mean, 4), "step_time": "median of the K steps' own HIP-event times",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)*0.5 bf16 Q/K/V, generated on the host)",
        "config": {"workload": w.name, "n": w.n, "P": P, "c": c, "device": p, "B": B, "H": H, "d": d,
                   "layout": "striped_tokens", "causal": True,
                   "step": "ra_forward(device p, all P rounds, RA_STRIPED_TOKENS: permutation in the addressing)",
                   "useful_flops_per_step": flops_s},
        "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 3),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 5),
                     "traffic": traffic_from_profile(w.name), "kernel": "k_attn_bf16 (ra_forward)",
                     "kernel_ms": round(fwd_avg, 4), "algorithmic_flops_per_launch": flops_s,
                     "clock": clock,
                     "frac_of_peak_at_sclk": (round(achieved / clock["peak_at_sclk_tflops"], 5)
                                              if clock and clock.get("peak_at_sclk_tflops") else None)},
        "wall_s_timed": round(wall, 3),
    }

    permuted_step()                                    # qs, ks, vs: the permuted inputs for the extras
    torch.cuda.synchronize()
    if not args.no_extras:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # ---- the same share through an explicit permutation pass (RA_STRIPED)
        reps = max(3, args.steps // 2)
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        a.record()
        for i in range(reps):
            permuted_step(pev[i])
        b.record()
        torch.cuda.synchronize()
        pstep_ms = a.elapsed_time(b) / reps
        pfwd_ms = sum(x.elapsed_time(y) for x, y in pev) / reps
        result["permuted_step"] = {"step": "ra_permute Q,K,V,pos -> ra_forward(RA_STRIPED)",
                                   "ms": round(pstep_ms, 4),
                                   "tflops": round(flops_s / (pstep_ms * 1e-3) / 1e12, 3),
                                   "forward_ms": round(pfwd_ms, 4)}
        log(f"[bench] permute + forward step {pstep_ms:.2f} ms ({flops_s / (pstep_ms * 1e-3) / 1e12:.1f} TFLOP/s)")

        # ---- ring (contiguous) forward for the same device
        reps = max(3, args.steps // 2)
        ra.forward(q, k, v, P, "contiguous", True, p_begin=p, p_end=p + 1, out=(o, lse))
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            ra.forward(q, k, v, P, "contiguous", True, p_begin=p, p_end=p + 1, out=(o, lse))
        b.record()
        torch.cuda.synchronize()
        ring_ms = a.elapsed_time(b) / reps
        result["ring"] = {"forward_ms": round(ring_ms, 4),
                          "tflops": round(flops_c / (ring_ms * 1e-3) / 1e12, 3),
                          "useful_flops": flops_c,
                          "striped_forward_ms": round(fwd_avg, 4),
                          "share_speedup_striped_over_ring": round(ring_ms / fwd_avg, 4),
                          "ideal_share_speedup": round(sum(pairs_c) / sum(pairs_s), 5)}
        log(f"[bench] ring forward {ring_ms:.2f} ms; share speedup {ring_ms / fwd_avg:.3f}x")

        # ---- per-round ra_round, both layouts, device p
        per = {}
        for layout, (qq, kk_, vv) in (("contiguous", (q, k, v)), ("striped", (qs, ks, vs))):
            times = []
            for r in range(P):
                kb = (p - r) % P
                args_r = (qq[:, :, p * c:(p + 1) * c], kk_[:, :, kb * c:(kb + 1) * c], vv[:, :, kb * c:(kb + 1) * c],
                          P, p, kb, layout, True)
                ra.round(*args_r)
                a.record()
                for _ in range(3):
                    ra.round(*args_r)
                b.record()
                torch.cuda.synchronize()
                times.append(a.elapsed_time(b) / 3)
            per[layout] = times
        ratios = [tc / ts for tc, ts in zip(per["contiguous"], per["striped"])]
        result["per_round"] = {
            "device": p, "round_ms_contiguous": [round(x, 4) for x in per["contiguous"]],
            "round_ms_striped": [round(x, 4) for x in per["striped"]],
            "speedup_striped_over_ring": [round(x, 4) for x in ratios],
            "ideal_speedup": [round(a_ / b_, 5) if b_ else None for a_, b_ in zip(pairs_c, pairs_s)],
            "slowest_round_speedup": round(max(per["contiguous"]) / max(per["striped"]), 4),
        }
        log("[bench] per-round speedup " + " ".join(f"{x:.3f}" for x in ratios))

        # ---- streamed striped path: rounds + merges, and the HBM-bound kernels' bandwidth
        acc_o = torch.empty((B, H, c, d), dtype=torch.float32, device=dev)
        acc_l = torch.empty((B, H, c), dtype=torch.float32, device=dev)
        po = torch.empty_like(acc_o)
        pl = torch.empty_like(acc_l)
        m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        merge_ms = []
        acc_o.zero_()
        acc_l.fill_(float("-inf"))
        torch.cuda.synchronize()
        a.record()
        for r in range(P):
            kb = (p - r) % P
            ra.round(qs[:, :, p * c:(p + 1) * c], ks[:, :, kb * c:(kb + 1) * c], vs[:, :, kb * c:(kb + 1) * c],
                     P, p, kb, "striped", True, out=(po, pl))
            m0.record()
            ra.merge(acc_o, acc_l, po, pl)
            m1.record()
            torch.cuda.synchronize()
            merge_ms.append(m0.elapsed_time(m1))
        b.record()
        torch.cuda.synchronize()
        stream_ms = a.elapsed_time(b)
        merge_bytes = 3.0 * BH * c * (4 * d + 4)
        # merge bandwidth on its own: a 512 MB write before each timed merge, so that neither
        # operand is still in the 256 MB Infinity Cache from the round that produced it
        flush = torch.empty(128 * 2 ** 20, dtype=torch.float32, device=dev)
        merge_ms = []
        for _ in range(5):
            flush.fill_(1.0)
            m0.record()
            ra.merge(acc_o, acc_l, po, pl)
            m1.record()
            torch.cuda.synchronize()
            merge_ms.append(m0.elapsed_time(m1))
        del flush
        merge_ms.sort()
        mavg = merge_ms[len(merge_ms) // 2]
        # permute bandwidth
        a.record()
        for _ in range(3):
            ra.permute(k, P, out=ks)
        b.record()
        torch.cuda.synchronize()
        perm_ms = a.elapsed_time(b) / 3
        perm_bytes = 2.0 * k.numel() * k.element_size()
        # rotary embedding fused into the same permutation (one read, one write per element)
        ra.permute_rope(q, P, "striped", out=qs)
        a.record()
        for _ in range(3):
            ra.permute_rope(q, P, "striped", out=qs)
        b.record()
        torch.cuda.synchronize()
        rope_ms = a.elapsed_time(b) / 3
        ra.permute(q, P, out=qs)                       # restore the plain permuted Q
        result["streamed"] = {"rounds_plus_merges_ms": round(stream_ms, 3),
                              "tflops": round(flops_s / (stream_ms * 1e-3) / 1e12, 3)}
        result["hbm_kernels"] = {
            "merge": {"ms": round(mavg, 4), "bytes": merge_bytes, "timing": "median of 5, cache flushed before each",
                      "GBps": round(merge_bytes / (mavg * 1e-3) / 1e9, 1), "peak_GBps": PEAK_HBM_GBS},
            "permute": {"ms": round(perm_ms, 4), "bytes": perm_bytes,
                        "GBps": round(perm_bytes / (perm_ms * 1e-3) / 1e9, 1), "peak_GBps": PEAK_HBM_GBS},
            "permute_rope": {"ms": round(rope_ms, 4), "bytes": perm_bytes,
                             "GBps": round(perm_bytes / (rope_ms * 1e-3) / 1e9, 1), "peak_GBps": PEAK_HBM_GBS},
        }
        log(f"[bench] streamed {stream_ms:.2f} ms; merge {mavg:.3f} ms "
            f"({merge_bytes / (mavg * 1e-3) / 1e9:.0f} GB/s); permute {perm_ms:.3f} ms "
            f"({perm_bytes / (perm_ms * 1e-3) / 1e9:.0f} GB/s); permute+RoPE {rope_ms:.3f} ms "
            f"({perm_bytes / (rope_ms * 1e-3) / 1e9:.0f} GB/s)")

    if not args.no_extras:
        result["backward"] = backward_leg(torch, ra, w, (qs, ks, vs), (q, k, v), flops_s, flops_c, p)
        result["per_round_all_devices"] = per_round_all_devices(torch, ra, dev)
        log("[bench] seq_n8k per-round speedup (slowest device) "
            + " ".join(f"{x:.3f}" for x in result["per_round_all_devices"]["speedup_striped_over_ring"]))

    if not args.no_extras and w.name != "stress_n1m":
        result["stress_n1m"] = stress_leg(torch, ra, dev)

    if not args.no_extras:
        # context: a plain library GEMM (torch.matmul -> hipBLASLt), bf16, square 8192, on the
        # same box in the same run -- what dense bf16 matrix-core work sustains here
        g = 8192
        ga = torch.randn((g, g), device=dev, dtype=torch.bfloat16)
        gb = torch.randn((g, g), device=dev, dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(ga, gb)
        torch.cuda.synchronize()
        reps = 40
        a.record()
        for _ in range(reps):
            torch.matmul(ga, gb)
        b.record()
        torch.cuda.synchronize()
        gemm_ms = a.elapsed_time(b) / reps
        gclock = ClockSampler(torch, dev).run_while(torch, lambda: [torch.matmul(ga, gb) for _ in range(20)]).result(cus)
        result["context_gemm"] = {"op": "torch.matmul bf16 8192x8192x8192 (hipBLASLt)", "ms": round(gemm_ms, 4),
                                  "tflops": round(2.0 * g ** 3 / (gemm_ms * 1e-3) / 1e12, 1), "clock": gclock}
        if gclock and gclock.get("peak_at_sclk_tflops"):
            result["context_gemm"]["frac_of_peak_at_sclk"] = round(
                result["context_gemm"]["tflops"] / gclock["peak_at_sclk_tflops"], 4)
        log(f"[bench] bf16 GEMM 8192^3: {result['context_gemm']['tflops']} TFLOP/s")
        del ga, gb

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(w, "striped")
        log(f"[bench] cpu oracle {result['cpu_baseline']['value']:.4f} TFLOP/s")
    else:
        result["cpu_baseline"] = None

    props = torch.cuda.get_device_properties(dev)
    result["device"] = {"name": props.name, "cus": props.multi_processor_count,
                        "arch": getattr(props, "gcnArchName", "")}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
