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

Each measurement first runs its workload untimed for --device-warmup-ms (default 100 ms) so
that the GPU clocks have ramped up, then W untimed warmup steps, then exactly K timed steps.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu] [--decode-only]
                       [--prefill-only]
                       [--append-only] [--device-warmup-ms MS]
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


def default_kv_tile(d: int, n_kv: int) -> int:
    """Keys per tile: 128 over long key ranges (N_kv >= 4096), else 64.  Measured (attention
    kernel, one box, three runs each): the Qwen3-8B shape (d 128, N 4096) 75.2 us at 128 against
    78.8 at 64; Gemma2-9B (d 256, N 4096) 72.9 us at 128 against 76.6 at 64; the Llama batch
    (d 128, N 2048) 160.7 us at 64 against 167.7 at 128 (its causal diagonal tiles are a larger
    share of its work)."""
    return 128 if n_kv >= 4096 else 64


DEVICE_WARMUP_MS = 100.0


def device_warmup(fn, torch, ms=None):
    """Run fn untimed for at least `ms` milliseconds of wall clock before the warmup steps:
    the GPU raises its clocks over the first tens of milliseconds of sustained work (measured:
    the Qwen3-8B step goes from 102 to 89 us over the first ~300 steps), and the timed steps
    should see the sustained rate."""
    ms = DEVICE_WARMUP_MS if ms is None else ms
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()


def launch_stats(fn, torch, n=100):
    """Median, p10 and p90 (ms) of `n` launches of fn, each bracketed by its own pair of events
    on the launch stream (the events add a little to each launch)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return {"median_ms": float(np.median(t)), "p10_ms": float(np.percentile(t, 10)),
            "p90_ms": float(np.percentile(t, 90)), "launches": n}


def run_prefill(w, hf, torch, steps, warmup, reorder=True, kv_tile=None, raw_q=False,
                scale_rule=0, phat_mode=0):
    """Time `steps` full steps, then `steps` attention launches alone.  A step runs the
    Smooth-QK + quantize pass over Q, K and V, then the attention kernel; with raw_q the
    quantize pass covers K and V only and the attention kernel smooths and quantizes the
    binary16 Q itself.
    Returns (ms/step, attention kernel ms from the back-to-back launches, state)."""
    kv_tile = kv_tile or default_kv_tile(w.d, w.N_kv)
    st = prepare_prefill(w, hf, torch)
    q4, k4, v4 = st["bufs"]
    qin = None if raw_q else st["q"]
    qarg = dict(q_f16=st["q"], s=st["s"]) if raw_q else {}
    q4a = None if raw_q else q4

    def attn():
        hf.attn_fwd(q4a, k4, v4, B=w.B, Hq=w.Hq, Hkv=w.Hkv, N_q=w.N_q, N_kv=w.N_kv, d=w.d,
                    causal=w.causal, smooth=w.smooth, reorder=reorder, out=st["out"],
                    kv_tile=kv_tile, scale_rule=scale_rule, phat_mode=phat_mode, **qarg)

    def step():
        hf.quantize_qkv(qin, st["k"], st["v"], Hkv=w.Hkv, smooth=w.smooth, s=st["s"],
                        inv_s=st["inv"], out=(None if raw_q else q4, k4, v4),
                        scale_rule=scale_rule)
        attn()

    device_warmup(step, torch)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    # the attention kernel alone: `steps` back-to-back launches between two events on the
    # launch stream (no per-launch event overhead inside the bracket)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        attn()
    e1.record()
    torch.cuda.synchronize()
    st["launch_stats"] = launch_stats(attn, torch)
    return ms, e0.elapsed_time(e1) / steps, st


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

    def step(i):
        k4, v4 = caches[i % copies]
        hf.attn_fwd(None, k4, v4, B=w.B, Hq=w.Hq, Hkv=w.Hkv, N_q=1, N_kv=w.N_kv, d=w.d,
                    causal=False, smooth=True, reorder=True, q_f16=q, s=s,
                    num_splits=w.num_splits, out=out, workspace=ws)

    cnt0 = [0]

    def warm():
        step(cnt0[0])
        cnt0[0] += 1
    device_warmup(warm, torch)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # back-to-back launches between two events on the launch stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    cnt = [0]

    def one():
        step(cnt[0])
        cnt[0] += 1
    stats = launch_stats(one, torch)
    return ms, e0.elapsed_time(e1) / steps, dict(q=q, s=s, caches=caches, out=out,
                                                 launch_stats=stats)


def append_bytes(w, T, pos):
    """Algorithmic HBM bytes of one append of T tokens at `pos` (every (b, g)): read the new K
    and V rows and the staged V of the first touched block, the RoPE table rows and inv_s; write
    the K_hat rows, every touched V_hat block (d codes of 16 B + d scale bytes) and the staging
    rows of a block left filling."""
    d, bg = w.d, w.B * w.Hkv
    blocks = (pos + T - 1) // 32 - pos // 32 + 1
    staged_in = pos % 32
    staged_out = (pos + T) % 32 if (pos + T) // 32 > pos // 32 else ((pos + T) % 32 - pos % 32
                                                                     if (pos + T) % 32 else 0)
    per_bg = (2 * T * d * 2 + staged_in * d * 2 + T * (d // 2 + d // 32) + blocks * d * 17
              + staged_out * d * 2)
    return bg * per_bg + T * d * 4 + w.Hkv * d * 4


APPEND_CALLS = 1000


def run_append(w, hf, torch, steps, warmup, T):
    """Decode-time KV append: a cache of N-1 tokens built by one append (untimed), then
    back-to-back appends of the tokens [N-T, N) at position N-T (each rewrites the same rows and
    blocks, so every launch does the same work) between two events, eagerly and replayed from a
    graph.  At least APPEND_CALLS calls each: a one-token append is host-bound, and the first
    few dozen launches after a synchronization enqueue faster than a sustained stream of them
    (measured on one box: 3.2 us per call over 50 calls, 4.2 over 200, 4.65 over 1000)."""
    steps = max(steps, APPEND_CALLS)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    s, inv = hf.calibrate_smooth(up(w.q_cal), up(w.k_cal), w.alpha)
    cos, sin = up(w.cos), up(w.sin)
    cache = hf.empty_kv_cache(w.B, w.Hkv, hf.padded(w.N + 1), w.d)
    k_all, v_all = up(w.k_raw), up(w.v)
    pos = w.N - T
    hf.kv_append(cache, k_all[:, :, :pos].contiguous(), v_all[:, :, :pos].contiguous(), pos=0,
                 rope_cos=cos, rope_sin=sin, smooth=True, inv_s=inv)
    kn, vn = k_all[:, :, pos:].contiguous(), v_all[:, :, pos:].contiguous()
    del k_all, v_all

    def step():
        hf.kv_append(cache, kn, vn, pos=pos, rope_cos=cos, rope_sin=sin, smooth=True, inv_s=inv)

    device_warmup(step, torch, ms=20.0)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (cache.k4.codes, cache.k4.scales, cache.v4.codes, cache.v4.scales)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # the same appends replayed from a captured graph: GPU time without the per-call host
    # cost (argument checks, ctypes), checked against the eager cache after every replay
    graph_ms = None
    try:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for _ in range(steps):
                    step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        times = []
        for _ in range(3):
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / steps)
            got = (cache.k4.codes, cache.k4.scales, cache.v4.codes, cache.v4.scales)
            if not all(torch.equal(a, b) for a, b in zip(got, ref)):
                raise RuntimeError("graph replay changed the cache")
        graph_ms = min(times)
        del g
    except RuntimeError as e:
        log(f"[bench] kv_append graph timing skipped: {e}")
    return ms, append_bytes(w, T, pos), graph_ms


def sample_rows(w, n, seed=12345):
    rng = np.random.default_rng(seed)
    total = w.B * w.Hq * w.N_q
    return np.sort(rng.choice(total, size=min(n, total), replace=False)).astype(np.int64)


def accuracy_rows(w, seed):
    """Query rows on which the error against fp64 exact attention is reported: every row of a
    workload of at most 4096 rows (the single head, the decode step), else a seeded 1/16 sample
    of all rows (every head)."""
    total = w.B * w.Hq * w.N_q
    if total <= 4096:
        return np.arange(total, dtype=np.int64)
    return sample_rows(w, total // 16, seed=seed)


def rows_to_host(out, rows, d, torch):
    """The given flat query rows of a [B][Hq][N_q][d] binary16 output, as a numpy array."""
    idx = torch.from_numpy(np.ascontiguousarray(rows)).cuda()
    return out.reshape(-1, d)[idx].cpu().numpy()


def rel_error(got, ref):
    """(max, mean) of |got - ref| / max_row |ref| (rows of the last axis; fp64)."""
    g = np.asarray(got, dtype=np.float64).reshape(-1, ref.shape[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    rm = np.abs(r).max(axis=1, keepdims=True)
    rm[rm == 0] = 1.0
    e = np.abs(g - r) / rm
    return float(e.max()), float(e.mean())


def row_flops(w, rows):
    i = rows % w.N_q
    keys = (i + w.N_kv - w.N_q + 1) if w.causal else np.full_like(i, w.N_kv)
    return float(np.sum(4.0 * w.d * keys))


E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def phat_tile_sums(codes, scales, kv_tile):
    """Sum of P_hat per (row, tile) from a dumped [rows][Npad/2] codes / [rows][Npad/32] scales
    pair: E2M1 value (sign in bit 3) times 2^(scale byte - 127) per 32-key block."""
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], -1)
    val = E2M1_MAGNITUDES[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    blk = val.reshape(codes.shape[0], -1, 32).sum(axis=2) * np.exp2(scales.astype(np.float64) - 127)
    return blk.reshape(codes.shape[0], -1, kv_tile // 32).sum(axis=2)


def eps_bar_tiles(sum_p, sum_phat, n_heads, N_q, rows_per_tile=64):
    """Per-tile mass change of the P-Reordering diagnostic.  sum_p / sum_phat: [n_heads * N_q][T]
    per-(row, key tile) sums of P and of P_hat (NaN where the row has no valid key in the tile),
    rows of each head contiguous.  A tile is rows_per_tile query rows x one key tile; over its
    rows with at least one valid key (sum P > 0):
        eps_bar = mean_i (sum P_hat_i - sum P_i) / sum P_i
        mass-weighted = (sum_i sum P_hat_i - sum_i sum P_i) / sum_i sum P_i
    Returns (eps_bar, mass_weighted), one entry per tile that has such a row."""
    T = sum_p.shape[1]
    valid = np.isfinite(sum_phat) & np.isfinite(sum_p) & (sum_p > 0)
    shape = (n_heads, N_q // rows_per_tile, rows_per_tile, T)
    spv = np.where(valid, sum_p, 0.0).reshape(shape)
    sphv = np.where(valid, sum_phat, 0.0).reshape(shape)
    val = valid.reshape(shape)
    eps = np.where(val, (sphv - spv) / np.where(val, spv, 1.0), 0.0)
    cnt = val.sum(axis=2)
    tiles = cnt > 0
    eb = (eps.sum(axis=2) / np.maximum(cnt, 1))[tiles]
    mw = ((sphv - spv).sum(axis=2) / np.maximum(spv.sum(axis=2), 1e-300))[tiles]
    return eb, mw


def eps_bar_summary(eb, mw, workload):
    hist, edges = np.histogram(eb, bins=16, range=(-0.2, 0.2))
    return {"workload": workload, "tiles": int(eb.size),
            "median": float(np.median(eb)), "mean": float(eb.mean()),
            "p10": float(np.percentile(eb, 10)), "p90": float(np.percentile(eb, 90)),
            "fraction_negative": float(np.mean(eb < 0)),
            "mass_weighted_median": float(np.median(mw)),
            "histogram": {"edges": [round(x, 4) for x in edges.tolist()], "counts": hist.tolist(),
                          "below": int(np.sum(eb < -0.2)), "above": int(np.sum(eb > 0.2))}}


def eps_bar_gpu_dump(w, hf, torch, kv_tile=64, scale_rule=0):
    """GPU half of the epsilon-bar diagnostic: one P_hat-dumping launch of the whole workload
    (off the timed path); returns the dump (device tensors, [rows][Npad/2] codes and
    [rows][Npad/32] scale bytes)."""
    st = prepare_prefill(w, hf, torch)
    q4, k4, v4 = st["bufs"]
    hf.quantize_qkv(st["q"], st["k"], st["v"], Hkv=w.Hkv, smooth=w.smooth, s=st["s"],
                    inv_s=st["inv"], out=st["bufs"], scale_rule=scale_rule)
    total = w.B * w.Hq * w.N_q
    npk = (w.N_kv + 127) // 128 * 128
    phat = hf.MX4(torch.zeros((total, npk // 2), dtype=torch.uint8, device="cuda"),
                  torch.zeros((total, npk // 32), dtype=torch.uint8, device="cuda"))
    hf.attn_fwd(q4, k4, v4, B=w.B, Hq=w.Hq, Hkv=w.Hkv, N_q=w.N_q, N_kv=w.N_kv, d=w.d,
                causal=w.causal, smooth=w.smooth, reorder=True, out=st["out"], kv_tile=kv_tile,
                phat=phat, scale_rule=scale_rule)
    torch.cuda.synchronize()
    codes, scales = phat.codes.cpu().numpy(), phat.scales.cpu().numpy()
    del st, phat
    torch.cuda.empty_cache()
    return codes, scales


def cpu_info():
    """Host CPU model and counts (the oracle baseline reports the threads it used)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count() or 1
    return {"cpu_model": model, "host_logical_cpus": os.cpu_count(), "cpus_available": affinity}


def cpu_leg(w, gpu_out, eps_inputs, acc_inputs, target_s=12.0, seed=777):
    """Everything that runs the CPU oracle, after the GPU measurements:

    * the baseline: the oracle's attention forward (quantized operands given, same tile
      size as the GPU) on a seeded sample of query rows of the primary workload, on this
      process's share of the host CPUs (the CPUs it may run on, at most 16: the share one
      GPU gets on a shared box); a first 1024-row pass sizes the sample so that the timed
      pass takes about `target_s` seconds;
    * parity of the GPU output on those rows (error relative to each row's max |O_oracle|);
    * for every workload in `acc_inputs`, the error of the GPU output and of the oracle's
      against fp64 softmax attention on the binary16 inputs, on all rows of the small
      workloads and a seeded 1/16 of the rows of the others, per P-Reordering setting;
    * the epsilon-bar diagnostic: per tile of 64 query rows x 64 keys, the mean over its rows
      of (sum P_hat - sum P) / sum P, from the oracle's per-tile sums over every head, with
      the GPU's dumped P_hat checked to give the same sum P_hat."""
    import oracle
    import synth
    res = {}

    def quant(wk, rule=0):
        s_ref = inv_ref = None
        if wk.smooth:
            s_ref, inv_ref = oracle.calibrate(wk.q_cal, wk.k_cal, wk.alpha)
        return (oracle.quantize_rows(wk.q, wk.Hkv, s_ref, rule),
                oracle.quantize_rows(wk.k, wk.Hkv, inv_ref, rule), oracle.quantize_v(wk.v, rule))

    rq, rk, rv = quant(w)
    threads = oracle.cpu_share()
    total = w.B * w.Hq * w.N_q
    kt = default_kv_tile(w.d, w.N_kv)

    def timed(rows):
        t0 = time.perf_counter()
        r = oracle.attn(w.B, w.Hq, w.Hkv, w.N_q, w.N_kv, w.d, causal=w.causal, reorder=1,
                        kv_tile=kt, q4=rq, k4=rk, v4=rv, rows=rows, threads=threads)
        return time.perf_counter() - t0, r

    probe = sample_rows(w, 1024, seed=seed + 1)
    dt0, _ = timed(probe)
    rate = row_flops(w, probe) / dt0
    n = int(min(total, max(1024, 1024 * target_s * rate / row_flops(w, probe))))
    rows = sample_rows(w, n, seed=seed)
    dt, ref = timed(rows)
    res["cpu_baseline"] = dict(
        value=row_flops(w, rows) / dt / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
        sample=f"{w.name} attention (quantized operands given, kv_tile {kt}), {len(rows)} "
               f"seeded random query rows of {total}, {dt:.1f} s", **cpu_info())

    got = gpu_out.reshape(-1, w.d)[rows]
    emax, emean = rel_error(got, ref["out"].view(np.float16))
    res["parity_sample"] = {"workload": w.name, "rows": len(rows), "err_max": emax,
                            "err_mean": emean}

    # error against fp64 exact attention, every workload
    acc = {}
    for name, wk, arows, outs, kw in acc_inputs:
        q3, k3, v3 = quant(wk, kw.get("scale_rule", 0))
        exact = oracle.attn_exact(wk.q, wk.k, wk.v, wk.causal, rows=arows, threads=threads)
        entry = {"rows": int(len(arows)), "rows_total": int(wk.B * wk.Hq * wk.N_q)}
        for reorder, gout in outs.items():
            r3 = oracle.attn(wk.B, wk.Hq, wk.Hkv, wk.N_q, wk.N_kv, wk.d, causal=wk.causal,
                             reorder=reorder, q4=q3, k4=k3, v4=v3, rows=arows, threads=threads,
                             **kw)
            o3 = r3["out"].view(np.float16)
            tag = "reorder_on" if reorder else "reorder_off"
            gm, ga = rel_error(gout, exact)
            om, oa = rel_error(o3, exact)
            pm, pa = rel_error(gout, o3)
            entry[tag] = {"gpu_vs_fp64_exact_max": gm, "gpu_vs_fp64_exact_mean": ga,
                          "oracle_vs_fp64_exact_max": om, "oracle_vs_fp64_exact_mean": oa,
                          "gpu_vs_oracle_max": pm, "gpu_vs_oracle_mean": pa}
        acc[name] = entry
    res["error_vs_fp64_exact"] = acc

    # the oracle on one thread: the single-head case whole, and 4 of the 64 sequences of the
    # decode step (same per-row work)
    single = {}
    for name, wk in (("single_head", synth.single_head()), ("decode_4_of_64_sequences",
                                                           synth.decode(B=4))):
        q3, k3, v3 = quant(wk)
        t0 = time.perf_counter()
        oracle.attn(wk.B, wk.Hq, wk.Hkv, wk.N_q, wk.N_kv, wk.d, causal=wk.causal, reorder=1,
                    kv_tile=wk.kv_tile, num_splits=wk.num_splits, q4=q3, k4=k3, v4=v3, threads=1)
        dt3 = time.perf_counter() - t0
        single[name] = {"seconds": dt3, "tflops": wk.flops / dt3 / 1e12,
                        "kv_gbs": wk.kv_bytes / dt3 / 1e9}
    res["cpu_oracle_single_thread"] = single

    # eps_inputs: (label, workload, dumped P_hat codes, scales, block-exponent rule) per run
    for label, we, codes, scales, rule in (eps_inputs or []):
        q2, k2, v2 = quant(we, rule)
        heads = we.B * we.Hq
        chunk = 8  # heads per oracle call
        ebs, mws, dev_max = [], [], 0.0
        for h0 in range(0, heads, chunk):
            h1 = min(heads, h0 + chunk)
            erows = np.arange(h0 * we.N_q, h1 * we.N_q, dtype=np.int64)
            r2 = oracle.attn(we.B, we.Hq, we.Hkv, we.N_q, we.N_kv, we.d, causal=we.causal,
                             reorder=1, kv_tile=64, q4=q2, k4=k2, v4=v2, rows=erows,
                             want_sums=True, threads=threads, scale_rule=rule)
            sp, sph = r2["sum_p"], r2["sum_phat"]
            T = sp.shape[1]
            gph = phat_tile_sums(codes[erows], scales[erows], 64)[:, :T]
            seen = np.isfinite(sph)
            if seen.any():
                dev = np.abs(gph[seen] - sph[seen]) / np.maximum(sph[seen], 1e-300)
                dev_max = max(dev_max, float(dev.max()))
            eb, mw = eps_bar_tiles(sp, sph, h1 - h0, we.N_q)
            ebs.append(eb)
            mws.append(mw)
        eb, mw = np.concatenate(ebs), np.concatenate(mws)
        res[label] = eps_bar_summary(
            eb, mw, f"{we.name}: all {heads} (b, h) heads, tiles of 64 rows x 64 keys, "
                    f"{'no-clipping' if rule else 'OCP'} block-exponent rule")
        res[label]["gpu_dump_sum_phat_max_rel_dev"] = dev_max
    return res


def main():
    global DEVICE_WARMUP_MS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true", help="primary workload only (profiling runs)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="the three prefill shapes only, no CPU leg (profiling runs); prints its "
                         "own line")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the split-KV decode step (profiling runs); prints its own line")
    ap.add_argument("--device-warmup-ms", type=float, default=DEVICE_WARMUP_MS,
                    help="untimed sustained work before the warmup steps of each measurement, "
                         "so that the GPU clocks have ramped up (0: none)")
    ap.add_argument("--append-only", action="store_true",
                    help="only the KV-cache appends (profiling runs); prints its own line")
    ap.add_argument("--copy-check", type=int, default=0, metavar="MIB",
                    help="first run one plain device copy of MIB MiB (a known-size reference "
                         "for hardware byte counters)")
    a = ap.parse_args()
    DEVICE_WARMUP_MS = a.device_warmup_ms
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported (the library has no "
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

    if a.decode_only:
        wd = synth.decode()
        msd, attnd, _ = run_decode(wd, hf, torch, a.steps, a.warmup)
        gbs = wd.kv_bytes / (attnd * 1e-3) / 1e9
        log(f"[bench] decode: {attnd:.4f} ms, {gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f} % of HBM)")
        print(json.dumps({"metric": "decode KV GB/s", "value": round(gbs, 3), "unit": "GB/s",
                          "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
                          "ms_per_step": round(msd, 5), "kernel_ms": round(attnd, 5),
                          "config": {"workload": "decode B=64 Hq=32 Hkv=8 d=128 N_kv=8192 "
                                                 "splits=16"}}), flush=True)
        return

    if a.append_only:
        wa = synth.kv_append()
        lines = {}
        for T in (1, 128):
            ms, nb, gms = run_append(wa, hf, torch, a.steps, a.warmup, T)
            lines[f"T{T}"] = {"us": round(ms * 1e3, 3), "bytes": nb, "gbs": round(nb / ms / 1e6, 1),
                              "calls": max(a.steps, APPEND_CALLS),
                              "graph_us": None if gms is None else round(gms * 1e3, 3)}
            log(f"[bench] kv_append T={T}: {ms * 1e3:.2f} us per call ({nb / ms / 1e6:.1f} GB/s)"
                + ("" if gms is None else f"; from a graph {gms * 1e3:.2f} us "
                                          f"({nb / gms / 1e6:.1f} GB/s)"))
        print(json.dumps({"metric": "KV append us", "value": lines["T1"]["us"], "unit": "us",
                          "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
                          "higher_is_better": False, "appends": lines,
                          "config": {"workload": "kv_append B=64 Hkv=8 d=128 cache 8192 tokens"}}),
              flush=True)
        return

    if a.prefill_only:
        lines = {}
        for fn in (synth.qwen3_8b, synth.gemma2_9b, synth.llama_batched):
            wx = fn()
            msx, attnx, stx = run_prefill(wx, hf, torch, a.steps, a.warmup, reorder=True)
            lines[wx.name] = {"kernel": f"attn_prefill_kernel<{wx.d},{default_kv_tile(wx.d, wx.N_kv)},"
                                        f"causal,reorder>", "attn_ms": attnx, "ms_per_step": msx,
                              "attn_frac_fp4_peak": wx.flops / (attnx * 1e-3) / 1e12 / FP4_PEAK_TFLOPS}
            log(f"[bench] {wx.name}: attention {attnx:.4f} ms ({100 * lines[wx.name]['attn_frac_fp4_peak']:.2f} "
                f"% of FP4 peak)")
            del stx
            torch.cuda.empty_cache()
        print(json.dumps({"metric": "prefill attention ms", "steps": a.steps, "warmup": a.warmup,
                          "workloads": lines}), flush=True)
        return

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
        "device_warmup_ms": DEVICE_WARMUP_MS,
        "config": {"workload": "qwen3_8b_prefill", "B": 1, "Hq": 32, "Hkv": 8, "N": 4096, "d": 128,
                   "causal": True, "smooth_alpha": 0.5, "reorder": True,
                   "kv_tile": default_kv_tile(w.d, w.N_kv),
                   "step": "quantize_qkv + attn_fwd"},
        "roofline": {"bound": "mfma",
                     "kernel": f"attn_prefill_kernel<{w.d},{default_kv_tile(w.d, w.N_kv)},causal,reorder>",
                     "achieved": round(attn_tflops, 3), "peak": FP4_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / FP4_PEAK_TFLOPS, 5),
                     "traffic": traffic, "kernel_ms": round(attn_ms, 5)},
    }
    extra = {"qwen3_8b_attention_per_launch": st["launch_stats"]}
    gpu_out = None if a.no_cpu else st["out"].reshape(-1, w.d).cpu().numpy()
    # per workload: (name, workload, rows, {reorder: GPU output rows}, oracle tile settings),
    # the error against fp64 exact attention is computed on these rows in the CPU leg
    acc_inputs = []
    acc_rows = accuracy_rows(w, seed=2)
    acc_q = {1: gpu_out[acc_rows] if gpu_out is not None else None}
    del st
    eps_inputs = None
    if not a.quick:
        # the single-head workload: latency-bound, reported for its error and time
        w1h = synth.single_head()
        ms1h, attn1h, st1h = run_prefill(w1h, hf, torch, a.steps, a.warmup, reorder=True, kv_tile=64)
        extra["single_head"] = {"ms_per_step": ms1h, "attn_ms": attn1h,
                                "attn_tflops": w1h.flops / (attn1h * 1e-3) / 1e12}
        log(f"[bench] single head 256x256 d128: step {ms1h * 1e3:.1f} us, attention "
            f"{attn1h * 1e3:.1f} us")
        if not a.no_cpu:
            r1h = accuracy_rows(w1h, seed=1)
            acc_inputs.append(("single_head", w1h, r1h,
                               {1: rows_to_host(st1h["out"], r1h, w1h.d, torch)}, dict(kv_tile=64)))
        del st1h
        msq, attnq, stq = run_prefill(w, hf, torch, a.steps, a.warmup, reorder=True, raw_q=True)
        extra["qwen3_8b_q_in_kernel"] = {"ms_per_step": msq, "attn_ms": attnq,
                                         "step_tflops": w.flops / (msq * 1e-3) / 1e12}
        log(f"[bench] Q smoothed and quantized inside the attention kernel instead: step "
            f"{msq:.4f} ms, attention {attnq:.4f} ms")
        del stq
        ms0, attn0, st0 = run_prefill(w, hf, torch, a.steps, a.warmup, reorder=False)
        extra["qwen3_8b_reorder_off"] = {"ms_per_step": ms0, "attn_ms": attn0,
                                         "attn_tflops": w.flops / (attn0 * 1e-3) / 1e12}
        log(f"[bench] reorder off: attention {attn0:.4f} ms")
        # exp-free P_hat (codes from the log-domain value, no v_exp_f32 per score)
        msx, attnx, stx = run_prefill(w, hf, torch, a.steps, a.warmup, reorder=True, phat_mode=1)
        extra["qwen3_8b_expfree_phat"] = {"ms_per_step": msx, "attn_ms": attnx,
                                          "attn_tflops": w.flops / (attnx * 1e-3) / 1e12}
        log(f"[bench] exp-free P_hat: attention {attnx:.4f} ms")
        del stx
        if not a.no_cpu:
            acc_q[0] = rows_to_host(st0["out"], acc_rows, w.d, torch)
            acc_inputs.append(("qwen3_8b_prefill", w, acc_rows, acc_q,
                               dict(kv_tile=default_kv_tile(w.d, w.N_kv))))
        del st0
        for name, fn in (("gemma2_9b_prefill", synth.gemma2_9b),
                         ("llama_batched_prefill", synth.llama_batched)):
            wx = fn()
            xrows = accuracy_rows(wx, seed=3 if name.startswith("gemma") else 4)
            xouts = {}
            for reorder in ((True, False) if name.startswith("llama") else (True,)):
                msx, attnx, stx = run_prefill(wx, hf, torch, a.steps, a.warmup, reorder=reorder)
                if not a.no_cpu:
                    xouts[int(reorder)] = rows_to_host(stx["out"], xrows, wx.d, torch)
                key = name + ("" if reorder else "_reorder_off")
                extra[key] = {"ms_per_step": msx, "attn_ms": attnx,
                              "step_tflops": wx.flops / (msx * 1e-3) / 1e12,
                              "attn_tflops": wx.flops / (attnx * 1e-3) / 1e12,
                              "attn_frac_fp4_peak": wx.flops / (attnx * 1e-3) / 1e12 / FP4_PEAK_TFLOPS}
                log(f"[bench] {key}: step {msx:.4f} ms, attention {attnx:.4f} ms "
                    f"({extra[key]['attn_tflops']:.1f} TFLOP/s)")
                del stx
            if not a.no_cpu:
                acc_inputs.append((name, wx, xrows, xouts,
                                   dict(kv_tile=default_kv_tile(wx.d, wx.N_kv))))
            if name.startswith("llama"):
                # the no-clipping block-exponent rule on the same batch (every 4-bit block)
                nouts = {}
                for reorder in (True, False):
                    msn, attnn, stn = run_prefill(wx, hf, torch, a.steps, a.warmup,
                                                  reorder=reorder, scale_rule=1)
                    key = name + "_noclip" + ("" if reorder else "_reorder_off")
                    extra[key] = {"ms_per_step": msn, "attn_ms": attnn,
                                  "attn_tflops": wx.flops / (attnn * 1e-3) / 1e12}
                    log(f"[bench] {key}: step {msn:.4f} ms, attention {attnn:.4f} ms")
                    if not a.no_cpu:
                        nouts[int(reorder)] = rows_to_host(stn["out"], xrows, wx.d, torch)
                    del stn
                if not a.no_cpu:
                    acc_inputs.append((name + "_noclip", wx, xrows, nouts,
                                       dict(kv_tile=default_kv_tile(wx.d, wx.N_kv), scale_rule=1)))
                    eps_inputs = [("eps_bar", wx) + eps_bar_gpu_dump(wx, hf, torch) + (0,),
                                  ("eps_bar_noclip", wx) + eps_bar_gpu_dump(wx, hf, torch,
                                                                            scale_rule=1) + (1,)]
        wd = synth.decode()
        msd, attnd, std = run_decode(wd, hf, torch, a.steps, a.warmup)
        gbs = wd.kv_bytes / (attnd * 1e-3) / 1e9
        extra["decode"] = {"workload": "decode B=64 Hq=32 Hkv=8 d=128 N_kv=8192 splits=16",
                           "kv_bytes": wd.kv_bytes, "ms_per_step": msd, "kernel_ms": attnd,
                           "kv_gbs": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS,
                           "per_launch": std["launch_stats"]}
        log(f"[bench] decode: {attnd:.4f} ms, {gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f} % of HBM)")
        if not a.no_cpu:
            drows = accuracy_rows(wd, seed=5)
            acc_inputs.append(("decode", wd, drows, {1: rows_to_host(std["out"], drows, wd.d, torch)},
                               dict(kv_tile=wd.kv_tile, num_splits=wd.num_splits)))
        del std
        torch.cuda.empty_cache()
        # one long sequence: 8 KV heads are too few for the fused decode kernel, so this runs
        # the split kernel (one wavefront per chunk) and the merge kernel; eight cache copies
        # (285 MB, more than the last-level cache) so that every launch reads HBM
        w1 = synth.decode(B=1, N_kv=32768, num_splits=64, n_cal=128)
        ms1, attn1, st1 = run_decode(w1, hf, torch, a.steps, a.warmup, copies=8)
        gbs1 = w1.kv_bytes / (attn1 * 1e-3) / 1e9
        extra["decode_one_sequence"] = {
            "workload": "decode B=1 Hq=32 Hkv=8 d=128 N_kv=32768 splits=64 kv_tile=64",
            "kv_bytes": w1.kv_bytes, "ms_per_step": ms1, "kernel_ms": attn1, "kv_gbs": gbs1,
            "frac_hbm_peak": gbs1 / HBM_PEAK_GBS, "per_launch": st1["launch_stats"]}
        log(f"[bench] decode, one 32768-token sequence (64 splits): {attn1 * 1e3:.1f} us, "
            f"{gbs1:.1f} GB/s ({100 * gbs1 / HBM_PEAK_GBS:.1f} % of HBM)")
        del st1, w1
        torch.cuda.empty_cache()
        wa = synth.kv_append()
        extra["kv_append"] = {"workload": "kv_append B=64 Hkv=8 d=128: RoPE + Smooth-QK + MXFP4 of "
                                          "the new K rows, V blocks re-quantized, cache of 8192 "
                                          "tokens"}
        for T in (1, 128):
            msa, nba, gma = run_append(wa, hf, torch, a.steps, a.warmup, T)
            best = msa if gma is None else min(msa, gma)
            extra["kv_append"][f"T{T}"] = {"us_per_call": msa * 1e3, "alg_bytes": nba,
                                           "calls": max(a.steps, APPEND_CALLS),
                                           "us_graph": None if gma is None else gma * 1e3,
                                           "gbs": nba / best / 1e6,
                                           "frac_hbm_peak": nba / best / 1e6 / HBM_PEAK_GBS}
            log(f"[bench] kv_append T={T}: {msa * 1e3:.2f} us per call"
                + ("" if gma is None else f", {gma * 1e3:.2f} us from a graph")
                + f" ({nba / best / 1e6:.1f} GB/s)")
        del wa
        torch.cuda.empty_cache()
    if not a.no_cpu:
        if a.quick:
            acc_inputs.append(("qwen3_8b_prefill", w, acc_rows, {1: acc_q[1]},
                               dict(kv_tile=default_kv_tile(w.d, w.N_kv))))
        cl = cpu_leg(w, gpu_out, eps_inputs, acc_inputs)
        result["cpu_baseline"] = cl.pop("cpu_baseline")
        log(f"[bench] cpu oracle: {result['cpu_baseline']['value']:.6f} TFLOP/s on "
            f"{result['cpu_baseline']['cores']} threads ({result['cpu_baseline']['sample']})")
        ps = cl["parity_sample"]
        log(f"[bench] parity on {ps['rows']} sampled rows: max {ps['err_max']:.2e} mean "
            f"{ps['err_mean']:.2e}")
        for k, v in cl.get("error_vs_fp64_exact", {}).items():
            for tag in ("reorder_on", "reorder_off"):
                if tag in v:
                    e = v[tag]
                    log(f"[bench] {k} {tag}, {v['rows']} rows vs fp64 exact: GPU max "
                        f"{e['gpu_vs_fp64_exact_max']:.3f} mean {e['gpu_vs_fp64_exact_mean']:.4f}; "
                        f"oracle max {e['oracle_vs_fp64_exact_max']:.3f} mean "
                        f"{e['oracle_vs_fp64_exact_mean']:.4f}; GPU vs oracle max "
                        f"{e['gpu_vs_oracle_max']:.1e}")
        for k, v in cl.get("cpu_oracle_single_thread", {}).items():
            log(f"[bench] cpu oracle, one thread, {k}: {v['seconds']:.2f} s")
        for key in ("eps_bar", "eps_bar_noclip"):
            if key in cl:
                eb = cl[key]
                log(f"[bench] {key} over {eb['tiles']} tiles: median {eb['median']:.4f}, "
                    f"{100 * eb['fraction_negative']:.1f} % negative")
        extra.update(cl)
    if extra:
        result["extra"] = extra
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
