"""GPU parity of the exp-free P_hat mode (phat_mode = HIFA4_PHAT_EXPFREE).

HiFA4 (arXiv 2607.04302, Abstract): with P-Reordering only P_hat's codes feed the PV product
and the normalizer.  The exp-free mode makes those codes from the log-domain value without an
exponential (its mapping is checked against E2M1 rounding of 2^u on the CPU in
tests/test_expfree_map.py).  Against the oracle's reference path (P = 2^t, then E2M1): >= 99.9 %
identical P_hat codes and scale bytes over valid keys, output error <= 1e-2 max and <= 1e-3
mean relative to each row's max |O_oracle|; and at the benchmark's Qwen3-8B size every row.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import check_attn, mx4_to_dev, oracle_quant, to_dev, to_host, v_to_dev, valid_keys

pytestmark = pytest.mark.gpu
EXPFREE = 1


@pytest.fixture(scope="module")
def hf():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible HIP device")
    import bit_flashattention_amd as m
    m.load()
    return m


CASES = [
    # name, overrides, kv_tile, raw_q, causal
    ("qwen3_8b", dict(B=1, Hq=4, Hkv=1, N=512, d=128, n_cal=128), 128, False, True),
    ("qwen3_8b", dict(B=1, Hq=2, Hkv=2, N=200, N_kv=330, d=128, n_cal=64), 64, True, True),
    ("gemma2_9b", dict(B=1, Hq=2, Hkv=1, N=384, d=256, n_cal=128), 128, False, True),
    ("gemma2_9b", dict(B=1, Hq=2, Hkv=2, N=130, d=256, n_cal=64), 64, True, True),
    ("llama_batched", dict(B=2, Hq=4, Hkv=2, N=257, d=64), 128, True, True),
    ("llama_batched", dict(B=1, Hq=8, Hkv=2, N=96, N_kv=400, d=128), 64, False, False),
    ("single_head", dict(), 64, False, False),
]


def run_case(hf, w, kv_tile, raw_q, causal, tag, nrows_check=None):
    import torch
    s_ref = inv_ref = None
    if w.smooth:
        s_ref, inv_ref = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    rq, rk, rv = oracle_quant(w, s_ref, inv_ref)
    npk = oracle.padded(w.N_kv)
    phat = hf.MX4(torch.zeros((w.B, w.Hq, w.N_q, npk // 2), dtype=torch.uint8, device="cuda"),
                  torch.zeros((w.B, w.Hq, w.N_q, npk // 32), dtype=torch.uint8, device="cuda"))
    qarg = dict(q_f16=to_dev(w.q), s=None if s_ref is None else to_dev(s_ref)) if raw_q else {}
    out = hf.attn_fwd(None if raw_q else mx4_to_dev(rq), mx4_to_dev(rk), v_to_dev(rv), B=w.B,
                      Hq=w.Hq, Hkv=w.Hkv, N_q=w.N_q, N_kv=w.N_kv, d=w.d, causal=causal,
                      smooth=w.smooth, reorder=True, phat=phat, kv_tile=kv_tile,
                      phat_mode=EXPFREE, **qarg)
    torch.cuda.synchronize()
    ref = oracle.attn(w.B, w.Hq, w.Hkv, w.N_q, w.N_kv, w.d, causal=causal, reorder=1,
                      kv_tile=kv_tile, q4=rq, k4=rk, v4=rv, want_phat=True)
    got = to_host(out).reshape(-1, w.d)
    n = len(got)
    check_attn(tag, got, ref, valid_keys(np.arange(n), w.N_q, w.N_kv, causal),
               phat=(to_host(phat.codes).reshape(n, -1), to_host(phat.scales).reshape(n, -1)))


@pytest.mark.parametrize("name,kw,kv_tile,raw_q,causal", CASES)
def test_expfree_prefill_matches_oracle(hf, name, kw, kv_tile, raw_q, causal):
    tag = f"expfree prefill {name} {kw} kv_tile={kv_tile} raw_q={raw_q} causal={causal}"
    print(f"[{tag}]", flush=True)
    w = synth.WORKLOADS[name](**kw)
    run_case(hf, w, kv_tile, raw_q, causal, tag)


def test_expfree_full_size_qwen3(hf):
    """The benchmark's Qwen3-8B shape (B1 Hq32 Hkv8 N4096 d128, causal, 128-key tiles):
    every row's output and P_hat codes against the oracle."""
    tag = "expfree fullsize qwen3_8b kv_tile=128"
    print(f"[{tag}]", flush=True)
    w = synth.qwen3_8b()
    run_case(hf, w, 128, False, True, tag)
