"""The attention entry point that allocates nothing (hifa4_attn_fwd_noalloc) against
hifa4_attn_fwd with a caller workspace, through the C ABI.

The split-KV path with fewer than 128 KV heads in the batch is the one whose kernels use a
scratch buffer (the partial states between the split kernel and the merge kernel), so the
cases run it: two calls in a row, the second smaller than the first (fewer rows, fewer
splits, a different d), each compared bit for bit with the workspace entry point on the same
inputs, and each also checked against the CPU oracle at the acceptance bar.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import check_attn, mx4_to_dev, oracle_quant, to_dev, to_host, v_to_dev, valid_keys

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hf():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible HIP device")
    import bit_flashattention_amd as m
    m.load()
    return m


def _case(hf, B, Hq, Hkv, N_kv, d, C, kt):
    import torch
    print(f"[noalloc] B={B} Hq={Hq} Hkv={Hkv} N_kv={N_kv} d={d} splits={C} kv_tile={kt}",
          flush=True)
    w = synth.decode(B=B, Hq=Hq, Hkv=Hkv, N_kv=N_kv, d=d, num_splits=C, kv_tile=kt, n_cal=64)
    s_ref, inv_ref = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    rq, rk, rv = oracle_quant(w, s_ref, inv_ref)
    k4, v4, q, s = mx4_to_dev(rk), v_to_dev(rv), to_dev(w.q), to_dev(s_ref)
    kw = dict(B=B, Hq=Hq, Hkv=Hkv, N_q=1, N_kv=N_kv, d=d, causal=False, smooth=True,
              reorder=True, q_f16=q, s=s, num_splits=C, kv_tile=kt)
    assert B * Hkv < 128 and C > 1  # the split kernel + merge kernel: the scratch is used
    ref_out = hf.attn_fwd(None, k4, v4, **kw)
    out = torch.full((B, Hq, 1, d), float("nan"), dtype=torch.float16, device="cuda")
    hf.attn_fwd_noalloc(None, k4, v4, out=out, **kw)
    torch.cuda.synchronize()
    got = to_host(out).reshape(-1, d)
    assert np.array_equal(got.view(np.uint16), to_host(ref_out).reshape(-1, d).view(np.uint16))
    ref = oracle.attn(B, Hq, Hkv, 1, N_kv, d, causal=False, reorder=1, num_splits=C, kv_tile=kt,
                      q4=rq, k4=rk, v4=rv)
    check_attn(f"noalloc B={B} Hq={Hq} N_kv={N_kv} d={d} C={C}", got, ref,
               valid_keys(np.arange(B * Hq), 1, N_kv, False))


def test_noalloc_matches_workspace_entry_two_calls(hf):
    # first call: 4 x 32 query rows over 8192 keys in 64 chunks (4.3 MB of partial states)
    _case(hf, B=4, Hq=32, Hkv=8, N_kv=8192, d=128, C=64, kt=64)
    # second call, smaller: 8 rows over 3000 keys in 5 chunks, d = 64 (stale contents of the
    # first call's larger partial-state area must not leak into it)
    _case(hf, B=1, Hq=8, Hkv=2, N_kv=3000, d=64, C=5, kt=128)
