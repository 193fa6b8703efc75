"""GPU parity of the decode-time KV-cache append (hifa4_kv_append, through the C ABI).

A cache built by appends must hold exactly what quantizing the whole post-RoPE
sequence gives (HiFA4, arXiv 2607.04302, Abstract: Smooth-QK acts on K after
RoPE; K_hat and V_hat are 4-bit block-scaled operands).  The oracle side is
oracle.rope_f16 (RoPE, binary16 result), then oracle.quantize_rows with inv_s
for K and oracle.quantize_v for V, over positions [0, n).  Bar: identical codes
(+0 == -0) and scale bytes everywhere, untouched cache rows still zero, and the
staging rows holding the binary16 V of the block still filling.  A decode and
a prefill attention over an appended cache larger than N_kv (kv_capacity) must
match the oracle's attention over its own quantization of the same tokens.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import ERR_MAX, ERR_MEAN, codes_equal, out_error, tile_v, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hf():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible HIP device")
    import bit_flashattention_amd as m
    m.load()
    return m


def _sync():
    import torch
    torch.cuda.synchronize()


def _calibrate(hf, w, smooth):
    if not smooth:
        return None, None, None, None
    s_ref, inv_ref = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    s, inv = hf.calibrate_smooth(to_dev(w.q_cal), to_dev(w.k_cal), w.alpha)
    assert np.array_equal(to_host(inv), inv_ref)
    return s, inv, s_ref, inv_ref


def _oracle_cache(w, n, inv_ref, rope):
    k = w.k_raw[:, :, :n]
    if rope:
        k = oracle.rope_f16(np.ascontiguousarray(k), w.cos, w.sin)
    k4 = oracle.quantize_rows(np.ascontiguousarray(k), w.Hkv, inv_ref)
    v4 = tile_v(oracle.quantize_v(np.ascontiguousarray(w.v[:, :, :n])))
    return k4, v4


def _check_cache(cache, w, n, inv_ref, rope):
    k4, v4 = _oracle_cache(w, n, inv_ref, rope)
    npad = k4[0].shape[2]
    kc, ks = to_host(cache.k4.codes), to_host(cache.k4.scales)
    vc, vs = to_host(cache.v4.codes), to_host(cache.v4.scales)
    assert codes_equal(kc[:, :, :npad], k4[0]).all()
    assert np.array_equal(ks[:, :, :npad], k4[1])
    assert codes_equal(vc[:, :, : npad // 64], v4[0]).all()
    assert np.array_equal(vs[:, :, : npad // 64], v4[1])
    # rows and tiles never appended are untouched (the cache was allocated zeroed)
    assert not kc[:, :, npad:].any() and not ks[:, :, npad:].any()
    assert not vc[:, :, npad // 64:].any() and not vs[:, :, npad // 64:].any()
    # staging rows: binary16 V of the positions of the block still filling
    if n % 32:
        st = to_host(cache.v_stage)
        first = n // 32 * 32
        assert np.array_equal(st[:, :, : n - first].view(np.uint16),
                              w.v[:, :, first:n].view(np.uint16))


APPEND_CASES = [
    # d, token counts of the successive appends, capacity, smooth, rope
    (128, [1, 1, 30, 1, 33, 100, 1, 1, 64], 384, True, True),
    (64, [37, 1, 1, 27, 64, 1, 5, 2000, 3], 2304, True, True),   # one large multi-chunk append
    (256, [31, 2, 1, 64, 1, 29], 256, True, True),
    (128, [5, 59, 1, 2], 128, False, True),                         # no Smooth-QK
    (128, [40, 1, 23], 256, True, False),                           # K already rotated
]


@pytest.mark.parametrize("d,ts,cap,smooth,rope", APPEND_CASES)
def test_append_sequence_matches_oracle(hf, d, ts, cap, smooth, rope):
    print(f"[append] d={d} appends={ts} capacity={cap} smooth={smooth} rope={rope}", flush=True)
    w = synth.kv_append(B=2, Hkv=2, Hq=4, N=sum(ts), d=d, n_cal=64)
    s, inv, s_ref, inv_ref = _calibrate(hf, w, smooth)
    cache = hf.empty_kv_cache(w.B, w.Hkv, cap, d)
    k_all, v_all = to_dev(w.k_raw), to_dev(w.v)
    cos, sin = (to_dev(w.cos), to_dev(w.sin)) if rope else (None, None)
    pos = 0
    for i, t in enumerate(ts):
        hf.kv_append(cache, k_all[:, :, pos:pos + t].contiguous(), v_all[:, :, pos:pos + t].contiguous(),
                     pos=pos, rope_cos=cos, rope_sin=sin, smooth=smooth, inv_s=inv)
        pos += t
        if i in (0, len(ts) // 2, len(ts) - 1):
            _sync()
            _check_cache(cache, w, pos, inv_ref, rope)


def test_append_k_only_and_v_only(hf):
    """Skipping one tensor leaves its cache and staging rows untouched."""
    w = synth.kv_append(B=1, Hkv=2, Hq=2, N=70, d=128, n_cal=32)
    _, inv, _, inv_ref = _calibrate(hf, w, True)
    cache = hf.empty_kv_cache(w.B, w.Hkv, 128, w.d)
    hf.kv_append(cache, to_dev(w.k_raw), None, pos=0, rope_cos=to_dev(w.cos),
                 rope_sin=to_dev(w.sin), smooth=True, inv_s=inv)
    _sync()
    assert not to_host(cache.v4.codes).any() and not to_host(cache.v_stage).any()
    k4, _ = _oracle_cache(w, 70, inv_ref, True)
    assert codes_equal(to_host(cache.k4.codes), k4[0]).all()
    cache2 = hf.empty_kv_cache(w.B, w.Hkv, 128, w.d)
    hf.kv_append(cache2, None, to_dev(w.v), pos=0)
    _sync()
    assert not to_host(cache2.k4.codes).any() and not to_host(cache2.k4.scales).any()
    _, v4 = _oracle_cache(w, 70, inv_ref, True)
    assert codes_equal(to_host(cache2.v4.codes), v4[0]).all()
    assert np.array_equal(to_host(cache2.v4.scales), v4[1])


@pytest.mark.parametrize("N,cap,splits", [(1000, 1152, 4), (131, 256, 1)])
def test_attention_over_appended_cache(hf, N, cap, splits):
    """Decode (raw q, in-kernel Smooth-QK + quantization, split-KV) and prefill (causal,
    pre-quantized Q) over a cache with more rows than N_kv, against the oracle."""
    print(f"[append+attn] N_kv={N} capacity={cap} splits={splits}", flush=True)
    w = synth.kv_append(B=2, Hkv=2, Hq=8, N=N, d=128, n_cal=64)
    s, inv, s_ref, inv_ref = _calibrate(hf, w, True)
    cache = hf.empty_kv_cache(w.B, w.Hkv, cap, w.d)
    k_all, v_all = to_dev(w.k_raw), to_dev(w.v)
    cos, sin = to_dev(w.cos), to_dev(w.sin)
    cuts = [0, N - 3, N - 2, N - 1, N]
    for a, b in zip(cuts[:-1], cuts[1:]):
        hf.kv_append(cache, k_all[:, :, a:b].contiguous(), v_all[:, :, a:b].contiguous(), pos=a,
                     rope_cos=cos, rope_sin=sin, smooth=True, inv_s=inv)
    k4r, v4r = _oracle_cache(w, N, inv_ref, True)
    v4c = oracle.quantize_v(np.ascontiguousarray(w.v))
    # decode: one query per sequence
    q = synth.tensor(synth.seed_of(6, synth.TAG_QUERY), w.B, w.Hq, 1, w.d)
    q4r = oracle.quantize_rows(q, w.Hkv, s_ref)
    out = hf.attn_fwd(None, cache.k4, cache.v4, B=w.B, Hq=w.Hq, Hkv=w.Hkv, N_q=1, N_kv=N, d=w.d,
                      causal=False, smooth=True, reorder=True, q_f16=to_dev(q), s=s,
                      num_splits=splits, kv_capacity=cap)
    _sync()
    ref = oracle.attn(w.B, w.Hq, w.Hkv, 1, N, w.d, causal=False, reorder=1, num_splits=splits,
                      kv_tile=64, q4=q4r, k4=k4r, v4=v4c)
    emax, emean = out_error(to_host(out).reshape(-1, w.d), ref["out"].view(np.float16))
    print(f"  decode err max {emax:.2e} mean {emean:.2e}", flush=True)
    assert emax <= ERR_MAX and emean <= ERR_MEAN
    # prefill: the last 40 positions as causal queries
    nq = 40
    qp = synth.tensor(synth.seed_of(6, synth.TAG_Q), w.B, w.Hq, nq, w.d)
    q4p = oracle.quantize_rows(qp, w.Hkv, s_ref)
    q4d, _, _ = hf.quantize_qkv(to_dev(qp), None, None, Hkv=w.Hkv, smooth=True, s=s)
    outp = hf.attn_fwd(q4d, cache.k4, cache.v4, B=w.B, Hq=w.Hq, Hkv=w.Hkv, N_q=nq, N_kv=N,
                       d=w.d, causal=True, smooth=True, reorder=True, kv_tile=128,
                       kv_capacity=cap)
    _sync()
    refp = oracle.attn(w.B, w.Hq, w.Hkv, nq, N, w.d, causal=True, reorder=1, kv_tile=128,
                       q4=q4p, k4=k4r, v4=v4c)
    emax, emean = out_error(to_host(outp).reshape(-1, w.d), refp["out"].view(np.float16))
    print(f"  prefill err max {emax:.2e} mean {emean:.2e}", flush=True)
    assert emax <= ERR_MAX and emean <= ERR_MEAN


def test_append_full_size(hf):
    """The benchmark's append: B=64 sequences x 8 KV heads, d=128, a cache of 8191 tokens
    built by one append, then one token at position 8191.  Checked: the new token's K row
    and its V block in every (b, g), and four seeded (b, g) caches in full."""
    import torch
    w = synth.kv_append()
    print(f"[append] full size B={w.B} Hkv={w.Hkv} d={w.d} N={w.N}", flush=True)
    s, inv, s_ref, inv_ref = _calibrate(hf, w, True)
    cap = hf.padded(w.N + 1)
    cache = hf.empty_kv_cache(w.B, w.Hkv, cap, w.d)
    k_all, v_all = to_dev(w.k_raw), to_dev(w.v)
    cos, sin = to_dev(w.cos), to_dev(w.sin)
    n0 = w.N - 1
    hf.kv_append(cache, k_all[:, :, :n0].contiguous(), v_all[:, :, :n0].contiguous(), pos=0,
                 rope_cos=cos, rope_sin=sin, smooth=True, inv_s=inv)
    hf.kv_append(cache, k_all[:, :, n0:].contiguous(), v_all[:, :, n0:].contiguous(), pos=n0,
                 rope_cos=cos, rope_sin=sin, smooth=True, inv_s=inv)
    _sync()
    del k_all, v_all
    # the appended token's K row, every (b, g)
    kr = oracle.rope_f16(np.ascontiguousarray(w.k_raw[:, :, n0:]), w.cos, w.sin, pos0=n0)
    k4 = oracle.quantize_rows(kr, w.Hkv, inv_ref)
    assert codes_equal(to_host(cache.k4.codes[:, :, n0]), k4[0][:, :, 0]).all()
    assert np.array_equal(to_host(cache.k4.scales[:, :, n0]), k4[1][:, :, 0])
    # its 32-position V block (positions 8160..8191 = block 255: tile 127, second half)
    v4 = tile_v(oracle.quantize_v(np.ascontiguousarray(w.v[:, :, n0 - 31:])))
    assert codes_equal(to_host(cache.v4.codes[:, :, 127, :, 16:]), v4[0][:, :, 0, :, :16]).all()
    assert np.array_equal(to_host(cache.v4.scales[:, :, 127, :, 1]), v4[1][:, :, 0, :, 0])
    # four (b, g) caches in full
    rng = np.random.default_rng(606)
    for flat in rng.choice(w.B * w.Hkv, 4, replace=False):
        b, g = divmod(int(flat), w.Hkv)
        sub = synth.AppendWorkload("slice", 1, 1, 1, w.N, w.d, w.theta, w.alpha,
                                   np.ascontiguousarray(w.k_raw[b:b + 1, g:g + 1]),
                                   np.ascontiguousarray(w.v[b:b + 1, g:g + 1]), w.cos, w.sin)
        k4s, v4s = _oracle_cache(sub, w.N, inv_ref[g:g + 1], True)
        assert codes_equal(to_host(cache.k4.codes[b, g, : w.N]), k4s[0][0, 0, : w.N]).all()
        assert np.array_equal(to_host(cache.k4.scales[b, g, : w.N]), k4s[1][0, 0, : w.N])
        assert codes_equal(to_host(cache.v4.codes[b, g, : w.N // 64]), v4s[0][0, 0]).all()
        assert np.array_equal(to_host(cache.v4.scales[b, g, : w.N // 64]), v4s[1][0, 0])
    del cache
    torch.cuda.empty_cache()


def test_binding_stream_is_torch_current_stream(hf):
    """The binding reads torch's current stream through its raw handle (cheaper than a
    torch.cuda.Stream object per call); it must be the same stream, also inside a stream
    context, and an explicit stream argument wins."""
    import torch
    assert hf._stream() == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        assert hf._stream() == side.cuda_stream == torch.cuda.current_stream().cuda_stream
    assert hf._stream(side) == side.cuda_stream
    assert hf._stream() == torch.cuda.current_stream().cuda_stream
