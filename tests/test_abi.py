"""The C-ABI library builds, loads, exports every declared symbol, and rejects bad
arguments on the host before touching a device (CPU only: no compute calls)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hifa4.h")


@pytest.fixture(scope="module")
def hf():
    import bit_flashattention_amd as m
    if not os.path.exists(m.LIB_PATH):
        from bit_flashattention_amd import build
        build.build(verbose=False)
    m.load()
    return m


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = set(re.findall(r"\b(hifa4_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_every_declared_symbol_is_exported(hf):
    names = _declared()
    assert set(hf.EXPORTS) == set(names)
    lib = ctypes.CDLL(hf.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(hf):
    lib = hf.load()
    assert lib.hifa4_version() == 105
    for s in range(6):
        assert lib.hifa4_status_str(s)
    assert b"unknown" in lib.hifa4_status_str(99)


def test_mx4_bytes(hf):
    assert hf.hifa4_mx4_bytes(0, 1, 32, 4096, 128) == (32 * 4096 * 64, 32 * 4096 * 4)
    assert hf.hifa4_mx4_bytes(1, 2, 8, 100, 256) == (2 * 8 * 128 * 128, 2 * 8 * 128 * 8)
    assert hf.hifa4_mx4_bytes(0, 0, 8, 0, 64) == (0, 0)
    with pytest.raises(hf.HiFA4Error) as e:
        hf.hifa4_mx4_bytes(0, 1, 1, 1, 100)
    assert e.value.status == hf.EINVAL


def test_workspace_bytes(hf):
    assert hf.hifa4_attn_workspace_bytes(64, 32, 1, 128, 1) == 0
    assert hf.hifa4_attn_workspace_bytes(64, 32, 1, 128, 16) == 64 * 32 * 16 * 130 * 4
    with pytest.raises(hf.HiFA4Error):
        hf.hifa4_attn_workspace_bytes(1, 1, 1, 128, 0)


def _args(hf, **kw):
    a = hf.AttnArgs()
    fake = 0x1000  # never dereferenced: every case below fails validation first
    a.q_codes = a.q_scales = a.k_codes = a.k_scales = a.v_codes = a.v_scales = fake
    a.out_f16 = fake
    a.num_splits = 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("case,status", [
    (dict(Hq=6, Hkv=4), "EINVAL"),
    (dict(N_kv=0), "EINVAL"),
    (dict(N_kv=40000), "EINVAL"),
    (dict(N_q=300, N_kv=256, causal=1), "EINVAL"),
    (dict(d=100), "EINVAL"),
    (dict(d=96), "EUNSUPPORTED"),
    (dict(args=dict(kv_tile=128, num_splits=2), d=256, N_q=4), "EUNSUPPORTED"),  # split-KV, d = 256
    (dict(args=dict(kv_tile=96)), "EUNSUPPORTED"),
    (dict(args=dict(num_splits=0)), "EINVAL"),
    (dict(args=dict(q_f16=0x2000)), "EINVAL"),          # both Q forms given
    (dict(args=dict(k_codes=None)), "EINVAL"),
    (dict(args=dict(out_f16=None)), "EINVAL"),
    (dict(args=dict(phat_codes=0x1000)), "EINVAL"),      # codes without scales
    (dict(args=dict(num_splits=4), N_q=16), "EUNSUPPORTED"),  # 16 rows x 4 heads > 32
    (dict(args=dict(k_codes=0x1008)), "EINVAL"),         # misaligned
    (dict(args=dict(kv_capacity=200)), "EINVAL"),        # not a multiple of 128
    (dict(args=dict(kv_capacity=128)), "EINVAL"),        # below N_kv = 256
    (dict(args=dict(scale_rule=2)), "EINVAL"),           # no such block-exponent rule
    (dict(args=dict(phat_mode=2)), "EINVAL"),            # no such P_hat mode
    (dict(args=dict(phat_mode=1), reorder=0), "EINVAL"),  # exp-free P_hat without P-Reordering
    (dict(args=dict(phat_mode=1, num_splits=2), N_q=4), "EUNSUPPORTED"),  # exp-free, split-KV
])
def test_attn_validation(hf, case, status):
    shape = dict(B=1, Hq=8, Hkv=2, N_q=64, N_kv=256, d=128, causal=0, reorder=1)
    argkw = case.pop("args", {})
    shape.update(case)
    a = _args(hf, **argkw)
    with pytest.raises(hf.HiFA4Error) as e:
        hf.hifa4_attn_fwd(shape["B"], shape["Hq"], shape["Hkv"], shape["N_q"], shape["N_kv"],
                          shape["d"], shape["causal"], 0, shape["reorder"], a, None)
    assert e.value.status == getattr(hf, status)
    assert hf.load().hifa4_last_error()


def test_attn_empty_is_noop(hf):
    a = _args(hf)
    hf.hifa4_attn_fwd(1, 8, 2, 0, 256, 128, 0, 0, 1, a, None)
    hf.hifa4_attn_fwd(0, 8, 2, 64, 256, 128, 0, 0, 1, a, None)


def test_device_checks_after_validation(hf):
    """Valid sizes with host pointers: ENODEV without a GPU, EINVAL (not device memory) with one."""
    host = np.zeros(1 << 16, dtype=np.uint8)
    p = host.ctypes.data
    p = (p + 255) // 256 * 256
    a = _args(hf, q_codes=p, q_scales=p, k_codes=p, k_scales=p, v_codes=p, v_scales=p, out_f16=p)
    with pytest.raises(hf.HiFA4Error) as e:
        hf.hifa4_attn_fwd(1, 8, 2, 64, 256, 128, 1, 0, 1, a, None)
    assert e.value.status in (hf.ENODEV, hf.EINVAL)
    with pytest.raises(hf.HiFA4Error) as e:
        hf.hifa4_quantize_qkv(p, None, None, 1, 8, 2, 64, 0, 128, 0, None, None, p, p, None, None,
                              None, None, 0, None)
    assert e.value.status in (hf.ENODEV, hf.EINVAL)


@pytest.mark.parametrize("call", ["quant_smooth_no_s", "quant_bad_d", "quant_missing_out",
                                  "quant_bad_rule", "calib_alpha", "calib_null"])
def test_quantize_calibrate_validation(hf, call):
    p = 0x10000
    with pytest.raises(hf.HiFA4Error) as e:
        if call == "quant_smooth_no_s":
            hf.hifa4_quantize_qkv(p, None, None, 1, 8, 2, 64, 0, 128, 1, None, None, p, p, None,
                                  None, None, None, 0, None)
        elif call == "quant_bad_d":
            hf.hifa4_quantize_qkv(p, None, None, 1, 8, 2, 64, 0, 100, 0, None, None, p, p, None,
                                  None, None, None, 0, None)
        elif call == "quant_missing_out":
            hf.hifa4_quantize_qkv(None, p, None, 1, 8, 2, 0, 64, 128, 0, None, None, None, None,
                                  None, None, None, None, 0, None)
        elif call == "quant_bad_rule":
            hf.hifa4_quantize_qkv(p, None, None, 1, 8, 2, 64, 0, 128, 0, None, None, p, p, None,
                                  None, None, None, 2, None)
        elif call == "calib_alpha":
            hf.hifa4_calibrate_smooth(p, p, 1, 8, 2, 16, 128, 1.5, p, p, None)
        else:
            hf.hifa4_calibrate_smooth(p, None, 1, 8, 2, 16, 128, 0.5, p, p, None)
    assert e.value.status == hf.EINVAL


@pytest.mark.parametrize("case", ["null", "bad_d", "negative", "misaligned", "overlap"])
def test_v_layout_validation(hf, case):
    """Argument checks of hifa4_v_layout, taken before any device access."""
    p, q = 0x10000, 0x900000
    args = {"null": (1, None, p, q, q + 0x40000, 1, 1, 64, 128),
            "bad_d": (1, p, p + 0x40000, q, q + 0x40000, 1, 1, 64, 96),
            "negative": (0, p, p + 0x40000, q, q + 0x40000, 1, -1, 64, 128),
            "misaligned": (1, p + 8, p + 0x40000, q, q + 0x40000, 1, 1, 64, 128),
            # the output codes start inside the input codes (1 x 1 x 128 tokens x 64 B)
            "overlap": (1, p, p + 0x40000, p + 4096, q, 1, 1, 128, 128)}[case]
    with pytest.raises(hf.HiFA4Error) as e:
        hf.hifa4_v_layout(*args, None)
    assert e.value.status == hf.EINVAL


def test_v_layout_empty_is_noop(hf):
    p = 0x10000
    hf.hifa4_v_layout(1, p, p + 0x40000, 0x900000, 0x940000, 2, 3, 0, 128, None)


def test_binding_fails_loudly_without_library(tmp_path):
    import importlib
    import bit_flashattention_amd as m
    saved = m._lib
    try:
        m._lib = None
        with pytest.raises(OSError):
            m.load(str(tmp_path / "missing.so"))
    finally:
        m._lib = saved


def test_product_path_does_not_reference_the_oracle():
    pkg = os.path.join(ROOT, "bit_flashattention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f
                assert "hifa4_oracle" not in txt, f


def _append(hf, **kw):
    """hifa4_kv_append with plausible (never dereferenced) pointers, overridden by kw."""
    p = 0x10000
    a = dict(k=p, v=p, B=2, Hkv=2, T=3, d=128, pos=61, cap=256, cos=p, sin=p, rows=64, smooth=1,
             inv_s=p, kc=p, ks=p, vc=p, vs=p, stage=p, rule=0)
    a.update(kw)
    hf.hifa4_kv_append(a["k"], a["v"], a["B"], a["Hkv"], a["T"], a["d"], a["pos"], a["cap"],
                       a["cos"], a["sin"], a["rows"], a["smooth"], a["inv_s"], a["kc"], a["ks"],
                       a["vc"], a["vs"], a["stage"], a["rule"], None)


@pytest.mark.parametrize("case,status", [
    (dict(Hkv=0), "EINVAL"),
    (dict(T=-1), "EINVAL"),
    (dict(d=100), "EINVAL"),
    (dict(d=96), "EUNSUPPORTED"),
    (dict(cap=200), "EINVAL"),                  # not a multiple of 128
    (dict(pos=250, T=7), "EINVAL"),             # past the capacity
    (dict(sin=None), "EINVAL"),                 # cos without sin
    (dict(rows=63), "EINVAL"),                  # table shorter than pos + T
    (dict(inv_s=None), "EINVAL"),               # smooth without inv_s
    (dict(kc=None), "EINVAL"),
    (dict(stage=None), "EINVAL"),
    (dict(vc=0x10008), "EINVAL"),               # misaligned
    (dict(rule=2), "EINVAL"),                   # no such block-exponent rule
])
def test_kv_append_validation(hf, case, status):
    with pytest.raises(hf.HiFA4Error) as e:
        _append(hf, **case)
    assert e.value.status == getattr(hf, status)
    assert hf.load().hifa4_last_error()


def test_kv_append_empty_is_noop(hf):
    _append(hf, T=0)
    _append(hf, B=0)
    _append(hf, k=None, v=None)
    # skipped tensors need none of their buffers
    with pytest.raises(hf.HiFA4Error) as e:
        _append(hf, v=None, vc=None, vs=None, stage=None)
    assert e.value.status in (hf.ENODEV, hf.EINVAL)  # valid sizes: fails only at the device check


def test_attn_noalloc_rejects_oversized_scratch_on_host(hf):
    """The no-allocation entry point validates like hifa4_attn_fwd, and a split-KV call whose
    partial states exceed the static scratch (B=64, Hq=32, one query, 16 splits at d=128:
    64*32*16*130*4 = 17,039,360 bytes > 16 MiB) fails with ENOSPACE before any device work."""
    a = _args(hf, num_splits=16)
    need = hf.hifa4_attn_workspace_bytes(64, 32, 1, 128, 16)
    assert need == 17_039_360 > (16 << 20)
    with pytest.raises(hf.HiFA4Error) as e:
        hf.hifa4_attn_fwd_noalloc(64, 32, 8, 1, 8192, 128, 0, 0, 1, a, None)
    assert e.value.status == hf.ENOSPACE
    assert b"static scratch" in hf.load().hifa4_last_error()
    with pytest.raises(hf.HiFA4Error) as e:
        hf.hifa4_attn_fwd_noalloc(1, 8, 2, 64, 256, 96, 0, 0, 1, _args(hf), None)
    assert e.value.status == hf.EUNSUPPORTED
    hf.hifa4_attn_fwd_noalloc(1, 8, 2, 0, 256, 128, 0, 0, 1, _args(hf), None)  # empty: no-op
