"""Benchmark: 4-bit FlashAttention forward (MXFP4 QK^T and PV, FP16 softmax state) on one MI355X.

One step = one pass of the hot path over one batch of synthetic input resident in HBM:
Smooth-QK + MXFP4 quantization of Q, K, V, then the attention forward with
P-Reordering.  The primary workload is the Qwen3-8B-shaped causal prefill layer
(B=1, Hq=32, Hkv=8, N=4096, d=128; Smooth-QK alpha 0.5 calibrated offline on a
separate 512-token batch).  value = algorithmic TFLOP/s of the whole step
(4 N_q N_kv d Hq B, halved for causal).

Also reported (one JSON line, extra keys): the dominant kernel against the FP4
MFMA roofline, the other prefill shapes, P-Reordering off, the split-KV decode
step in GB/s against HBM, and the CPU oracle timed on a sample of rows.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP4_PEAK_TFLOPS = 10100.0   # MI355X dense FP4 MFMA
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "bit_flashattention_amd", "csrc", f)
                  for f in ("attention.hip", "hifa4_device.hpp")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(kernel: str, flops_per_launch: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when the
    kernel source changed since the counters were taken."""
    try:
        t = json.load(open(TRAFFIC_FILE))[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


class Timer:
    """HIP events on the current stream around each launch of one kernel family."""

    def __init__(self):
        import torch
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, s):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append((s, e))

    def mean_ms(self) -> float:
        return float(np.mean([a.elapsed_time(b) for a, b in self.pairs])) if self.pairs else 0.0


def prepare_prefill(w, hf, torch):
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, k, v = up(w.q), up(w.k), up(w.v)
    s = inv = None
    if w.smooth:
        s, inv = hf.calibrate_smooth(up(w.q_cal), up(w.k_cal), w.alpha)  # offline, untimed
    bufs = (hf.empty_mx4(False, w.B, w.Hq, w.N_q, w.d), hf.empty_mx4(False, w.B, w.Hkv, w.N_kv, w.d),
            hf.empty_mx4(True, w.B, w.Hkv, w.N_kv, w.d))
    out = torch.empty((w.B, w.Hq, w.N_q, w.d), dtype=torch.float16, device="cuda")
    return dict(q=q, k=k, v=v, s=s, inv=inv, bufs=bufs, out=out)


def default_kv_tile(d: int) -> int:
    """Keys per tile: 128 where the kernels support it (d <= 128), else 64."""
    return 128 if d <= 128 else 64


def run_prefill(w, hf, torch, steps, warmup, reorder=True, kv_tile=None):
    """Time `steps` full steps (quantize + attention).  Returns (ms/step, attention kernel ms)."""
    kv_tile = kv_tile or default_kv_tile(w.d)
    st = prepare_prefill(w, hf, torch)
    q4, k4, v4 = st["bufs"]

    def step(timer=None):
        hf.quantize_qkv(st["q"], st["k"], st["v"], Hkv=w.Hkv, smooth=w.smooth, s=st["s"],
                        inv_s=st["inv"], out=st["bufs"])
        ev = timer.start() if timer else None
        hf.attn_fwd(q4, k4, v4, B=w.B, Hq=w.Hq, Hkv=w.Hkv, N_q=w.N_q, N_kv=w.N_kv, d=w.d,
                    causal=w.causal, smooth=w.smooth, reorder=reorder, out=st["out"],
                    kv_tile=kv_tile)
        if timer:
            timer.stop(ev)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    timer = Timer()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timer)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    return ms, timer.mean_ms(), st


def run_decode(w, hf, torch, steps, warmup, copies=2):
    """Decode: KV cache pre-quantized (untimed); the step is the split-KV attention with
    in-kernel Smooth-QK + quantization of q.  Rotates between `copies` caches larger than
    the 256 MB last-level cache so each step reads HBM."""
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    s, inv = hf.calibrate_smooth(up(w.q_cal), up(w.k_cal), w.alpha)
    q = up(w.q)
    k, v = up(w.k), up(w.v)
    caches = []
    for _ in range(copies):
        _, k4, v4 = hf.quantize_qkv(None, k, v, Hkv=w.Hkv, smooth=True, s=s, inv_s=inv)
        caches.append((k4, v4))
    del k, v
    torch.cuda.synchronize()
    out = torch.empty((w.B, w.Hq, 1, w.d), dtype=torch.float16, device="cuda")
    nbytes = hf.hifa4_attn_workspace_bytes(w.B, w.Hq, 1, w.d, w.num_splits)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def step(i, timer=None):
        k4, v4 = caches[i % copies]
        ev = timer.start() if timer else None
        hf.attn_fwd(None, k4, v4, B=w.B, Hq=w.Hq, Hkv=w.Hkv, N_q=1, N_kv=w.N_kv, d=w.d,
                    causal=False, smooth=True, reorder=True, q_f16=q, s=s,
                    num_splits=w.num_splits, out=out, workspace=ws)
        if timer:
            timer.stop(ev)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    timer = Timer()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, timer)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    return ms, timer.mean_ms(), dict(q=q, s=s, caches=caches, out=out)


def sample_rows(w, n, seed=12345):
    rng = np.random.default_rng(seed)
    total = w.B * w.Hq * w.N_q
    return np.sort(rng.choice(total, size=min(n, total), replace=False)).astype(np.int64)


def row_flops(w, rows):
    i = rows % w.N_q
    keys = (i + w.N_kv - w.N_q + 1) if w.causal else np.full_like(i, w.N_kv)
    return float(np.sum(4.0 * w.d * keys))


def parity_sample(w, hf, st, rows, reorder=True):
    """Oracle on sampled rows vs the GPU output of the timed launch configuration."""
    import oracle
    s_ref = inv_ref = None
    if w.smooth:
        s_ref, inv_ref = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    rq = oracle.quantize_rows(w.q, w.Hkv, s_ref)
    rk = oracle.quantize_rows(w.k, w.Hkv, inv_ref)
    rv = oracle.quantize_v(w.v)
    ref = oracle.attn(w.B, w.Hq, w.Hkv, w.N_q, w.N_kv, w.d, causal=w.causal, reorder=int(reorder),
                      kv_tile=default_kv_tile(w.d), q4=rq, k4=rk, v4=rv, rows=rows)
    got = st["out"].reshape(-1, w.d)[rows].cpu().numpy().astype(np.float64)
    exp = ref["out"].view(np.float16).astype(np.float64)
    rowmax = np.abs(exp).max(axis=1, keepdims=True)
    e = np.abs(got - exp) / rowmax
    # error of the 4-bit path against fp64 softmax attention on the binary16 inputs
    exact = oracle.attn_exact(w.q, w.k, w.v, w.causal, rows=rows)
    ex_max = np.abs(exact).max(axis=1, keepdims=True)
    ee = np.abs(got - exact) / ex_max
    return float(e.max()), float(e.mean()), float(ee.max()), float(ee.mean())


def cpu_baseline(w, target_s=12.0, seed=777):
    """The oracle's attention forward (quantized operands given) on a seeded sample of query
    rows, on the host threads this process may use (at most 16).  A first 1024-row pass sizes
    the sample so that the timed pass takes about `target_s` seconds."""
    import oracle
    s_ref = inv_ref = None
    if w.smooth:
        s_ref, inv_ref = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    rq = oracle.quantize_rows(w.q, w.Hkv, s_ref)
    rk = oracle.quantize_rows(w.k, w.Hkv, inv_ref)
    rv = oracle.quantize_v(w.v)
    threads = max(1, min(16, os.cpu_count() or 1))
    total = w.B * w.Hq * w.N_q

    def timed(rows):
        t0 = time.perf_counter()
        oracle.attn(w.B, w.Hq, w.Hkv, w.N_q, w.N_kv, w.d, causal=w.causal, reorder=1,
                    kv_tile=default_kv_tile(w.d), q4=rq, k4=rk, v4=rv, rows=rows, threads=threads)
        return time.perf_counter() - t0

    probe = sample_rows(w, 1024, seed=seed + 1)
    rate = row_flops(w, probe) / timed(probe)
    n = int(min(total, max(1024, 1024 * target_s * rate / row_flops(w, probe))))
    rows = sample_rows(w, n, seed=seed)
    dt = timed(rows)
    return row_flops(w, rows) / dt / 1e12, dt, threads, len(rows)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true", help="primary workload only (profiling runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-check", type=int, default=0, metavar="MIB",
                    help="first run one plain device copy of MIB MiB (a known-size reference "
                         "for hardware byte counters)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported (this build has no "
              "multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_flashattention_amd as hf
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    hf.load()
    torch.cuda.set_device(0)
    if a.copy_check:
        src = torch.empty(a.copy_check << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] reference copy of {a.copy_check} MiB done")
        del src, dst

    # ---- primary: Qwen3-8B-shaped causal prefill, P-Reordering on
    w = synth.qwen3_8b()
    log(f"[bench] {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N_q} d={w.d} causal")
    ms, attn_ms, st = run_prefill(w, hf, torch, a.steps, a.warmup, reorder=True)
    value = w.flops / (ms * 1e-3) / 1e12
    attn_tflops = w.flops / (attn_ms * 1e-3) / 1e12
    log(f"[bench] step {ms:.4f} ms ({value:.1f} TFLOP/s); attention kernel {attn_ms:.4f} ms "
        f"({attn_tflops:.1f} TFLOP/s, {100 * attn_tflops / FP4_PEAK_TFLOPS:.2f} % of FP4 peak)")
    traffic = measured_traffic("attn_prefill_qwen3_8b", w.flops)
    result = {
        "metric": "4-bit flash-attn prefill TFLOP/s & % of FP4 MFMA peak; decode KV GB/s",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic (seeded SplitMix64/Box-Muller, RoPE, outlier channels; no model weights)",
        "config": {"workload": "qwen3_8b_prefill", "B": 1, "Hq": 32, "Hkv": 8, "N": 4096, "d": 128,
                   "causal": True, "smooth_alpha": 0.5, "reorder": True,
                   "kv_tile": default_kv_tile(w.d),
                   "step": "quantize_qkv + attn_fwd"},
        "roofline": {"bound": "mfma",
                     "kernel": f"attn_prefill_kernel<{w.d},{default_kv_tile(w.d)},causal,reorder>",
                     "achieved": round(attn_tflops, 3), "peak": FP4_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / FP4_PEAK_TFLOPS, 5),
                     "traffic": traffic, "kernel_ms": round(attn_ms, 5)},
    }
    extra = {}
    if not a.quick:
        rows = sample_rows(w, 256)
        emax, emean, xmax, xmean = parity_sample(w, hf, st, rows, reorder=True)
        extra["parity_sample"] = {"rows": len(rows), "err_max": emax, "err_mean": emean,
                                  "vs_fp64_exact_max": xmax, "vs_fp64_exact_mean": xmean}
        log(f"[bench] parity on {len(rows)} sampled rows: max {emax:.2e} mean {emean:.2e}; "
            f"vs fp64 exact attention: max {xmax:.2e} mean {xmean:.2e}")
        del st
        ms0, attn0, st0 = run_prefill(w, hf, torch, a.steps, a.warmup, reorder=False)
        extra["qwen3_8b_reorder_off"] = {"ms_per_step": ms0, "attn_ms": attn0,
                                         "attn_tflops": w.flops / (attn0 * 1e-3) / 1e12}
        log(f"[bench] reorder off: attention {attn0:.4f} ms")
        del st0
        for name, fn in (("gemma2_9b_prefill", synth.gemma2_9b),
                         ("llama_batched_prefill", synth.llama_batched)):
            wx = fn()
            for reorder in ((True, False) if name.startswith("llama") else (True,)):
                msx, attnx, stx = run_prefill(wx, hf, torch, a.steps, a.warmup, reorder=reorder)
                key = name + ("" if reorder else "_reorder_off")
                extra[key] = {"ms_per_step": msx, "attn_ms": attnx,
                              "step_tflops": wx.flops / (msx * 1e-3) / 1e12,
                              "attn_tflops": wx.flops / (attnx * 1e-3) / 1e12,
                              "attn_frac_fp4_peak": wx.flops / (attnx * 1e-3) / 1e12 / FP4_PEAK_TFLOPS}
                log(f"[bench] {key}: step {msx:.4f} ms, attention {attnx:.4f} ms "
                    f"({extra[key]['attn_tflops']:.1f} TFLOP/s)")
                del stx
        wd = synth.decode()
        msd, attnd, std = run_decode(wd, hf, torch, a.steps, a.warmup)
        gbs = wd.kv_bytes / (attnd * 1e-3) / 1e9
        extra["decode"] = {"workload": "decode B=64 Hq=32 Hkv=8 d=128 N_kv=8192 splits=16",
                           "kv_bytes": wd.kv_bytes, "ms_per_step": msd, "kernel_ms": attnd,
                           "kv_gbs": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS}
        log(f"[bench] decode: {attnd:.4f} ms, {gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f} % of HBM)")
        del std
        torch.cuda.empty_cache()
    if not a.no_cpu:
        tf, dt, thr, nrows = cpu_baseline(w)
        result["cpu_baseline"] = {"value": tf, "unit": "TFLOP/s", "cores": thr, "kind": "oracle",
                                  "sample": f"qwen3_8b_prefill attention (quantized operands given), "
                                            f"{nrows} seeded random query rows of "
                                            f"{w.B * w.Hq * w.N_q}, {dt:.1f} s"}
        log(f"[bench] cpu oracle: {tf:.6f} TFLOP/s on {thr} threads ({dt:.1f} s)")
    if extra:
        result["extra"] = extra
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
