"""Host-side checks of bench.py and its workloads (CPU only, no HIP device needed).

* The benchmark measures one GPU: any other --gpus value is refused before torch or the
  device is touched, with exit status 2 and a message that says why.
* The synthetic workloads the benchmark times have the shapes of the five configurations
  (single head 256 x 256; Qwen3-8B-shaped B1 Hq32 Hkv8 N4096 d128 causal; Gemma2-9B-shaped
  Hq16 Hkv8 d256; Llama-shaped B8 N2048; decode B64 Hq32 Hkv8 N_kv 8192), and their
  algorithmic units equal the figures worked out by hand from the problem statement's
  definitions: 4 * N_q * N_kv * d * Hq * B FLOPs, halved when causal (33,554,432 for the
  single head, 137,438,953,472 for the two 4096-token prefills, 274,877,906,944 for the
  Llama batch), and B * Hkv * N_kv * (d + d/16) KV-cache bytes for decode (570,425,344:
  4-bit K and V codes, d/2 bytes each per token, plus one scale byte per 32 elements).
"""
import inspect
import os
import subprocess
import sys

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [0, 2, 8])
def test_bench_refuses_other_gpu_counts(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("name,shape,flops", [
    ("single_head", (1, 1, 1, 256, 256, 128, False), 33_554_432),
    ("qwen3_8b", (1, 32, 8, 4096, 4096, 128, True), 137_438_953_472),
    ("gemma2_9b", (1, 16, 8, 4096, 4096, 256, True), 137_438_953_472),
    ("llama_batched", (8, 32, 8, 2048, 2048, 128, True), 274_877_906_944),
])
def test_prefill_workload_shapes_and_flops(name, shape, flops):
    w = getattr(synth, name)()
    assert (w.B, w.Hq, w.Hkv, w.N_q, w.N_kv, w.d, w.causal) == shape
    assert w.flops == flops
    assert w.q.shape == (w.B, w.Hq, w.N_q, w.d) and w.k.shape == (w.B, w.Hkv, w.N_kv, w.d)


def test_decode_workload_shape_and_bytes():
    # the defaults bench.py uses (generating the 570 MB cache here would only take time)
    p = inspect.signature(synth.decode).parameters
    shape = tuple(p[k].default for k in ("B", "Hq", "Hkv", "N_kv", "d", "num_splits"))
    assert shape == (64, 32, 8, 8192, 128, 16)
    w = synth.Workload("decode", 64, 32, 8, 1, 8192, 128, False, True, 0.5, 64, 16, (1,))
    assert w.kv_bytes == 570_425_344
    assert w.flops == 4 * 8192 * 128 * 32 * 64


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def test_eps_bar_tiles_hand_example():
    """Two heads of 64 query rows, two key tiles.  Head 0, tile 0: rows with sum P = 2 and
    sum P_hat = 1.8 (relative change -0.1) except row 5, whose sum P_hat is 2.2 (+0.1); tile 1
    is masked (NaN) for rows 0..31 and has sum P = 4, sum P_hat = 3 (-0.25) for rows 32..63.
    Head 1: sum P = 0 in tile 0 (no mass: left out) and -0.5 for every row of tile 1."""
    import numpy as np
    b = _bench()
    sp = np.full((128, 2), 2.0)
    sph = np.full((128, 2), 1.8)
    sph[5, 0] = 2.2
    sp[:32, 1] = np.nan
    sph[:32, 1] = np.nan
    sp[32:64, 1], sph[32:64, 1] = 4.0, 3.0
    sp[64:, 0], sph[64:, 0] = 0.0, 0.0
    sp[64:, 1], sph[64:, 1] = 2.0, 1.0
    eb, mw = b.eps_bar_tiles(sp, sph, n_heads=2, N_q=64)
    # tiles in (head, row tile, key tile) order: (0,0,0), (0,0,1), (1,0,1)
    assert eb.shape == (3,)
    assert np.allclose(eb, [(63 * -0.1 + 0.1) / 64, -0.25, -0.5])
    assert np.allclose(mw, [(63 * 1.8 + 2.2 - 128) / 128, -0.25, -0.5])
    s = b.eps_bar_summary(eb, mw, "hand")
    assert s["tiles"] == 3 and s["fraction_negative"] == 1.0
    assert sum(s["histogram"]["counts"]) + s["histogram"]["below"] + s["histogram"]["above"] == 3


def test_phat_tile_sums_hand_example():
    """One row, 128 keys: block 0 holds code 2 (value 1) at every key with scale byte 127
    (x1), block 1 code 15 (-6) at key 32 with scale 128 (x2), blocks 2-3 code 1 (0.5) with
    scale 125 (x1/4).  Tile sums at kv_tile 64: 32 + (-12) = 20 and 64 * 0.5 / 4 = 8."""
    import numpy as np
    b = _bench()
    nib = np.zeros(128, dtype=np.uint8)
    nib[:32] = 2
    nib[32] = 15
    nib[64:] = 1
    codes = (nib[0::2] | (nib[1::2] << 4)).reshape(1, 64)
    scales = np.array([[127, 128, 125, 125]], dtype=np.uint8)
    t = b.phat_tile_sums(codes, scales, 64)
    assert np.allclose(t, [[20.0, 8.0]])


def test_accuracy_rows_and_rel_error():
    import numpy as np
    b = _bench()
    small = synth.Workload("s", 1, 4, 1, 256, 256, 64, False, False, 0.0, 64, 1, (1,))
    assert np.array_equal(b.accuracy_rows(small, 1), np.arange(1024))
    big = synth.Workload("b", 8, 32, 8, 2048, 2048, 128, True, False, 0.0, 64, 1, (1,))
    r = b.accuracy_rows(big, 4)
    assert len(r) == 8 * 32 * 2048 // 16 and np.all(np.diff(r) > 0)
    ref = np.array([[1.0, -2.0], [0.5, 0.25]])
    got = np.array([[1.0, -1.0], [0.5, 0.0]])
    emax, emean = b.rel_error(got, ref)
    assert emax == 0.5 and emean == (0 + 0.5 + 0 + 0.5) / 4


def test_cpu_info_reports_model_and_counts():
    b = _bench()
    info = b.cpu_info()
    assert info["host_logical_cpus"] >= 1 and info["cpus_available"] >= 1
    assert isinstance(info["cpu_model"], str) and info["cpu_model"]
