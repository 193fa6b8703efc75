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
