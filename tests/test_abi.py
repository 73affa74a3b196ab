"""The C-ABI library loads, exports what include/*.h declares, and rejects
malformed arguments on the host (these paths return before any HIP call)."""
import ctypes
import glob
import os
import re

import pytest

import fp8_bf16_causal_amd as fbc
from fp8_bf16_causal_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    declared = _declared_functions()
    assert {"attn_fwd", "attn_fwd_ex", "attn_fwd_lse", "attn_quantize_e4m3", "attn_strerror"} <= set(declared)
    for name in declared:
        assert hasattr(lib, name), name


def test_strerror_covers_codes():
    for code in (fbc.ATTN_OK, fbc.ATTN_ERR_INVALID, fbc.ATTN_ERR_UNSUPPORTED, fbc.ATTN_ERR_LAUNCH, 12345):
        assert isinstance(fbc.attn_strerror(code), str) and fbc.attn_strerror(code)
    assert fbc.attn_strerror(fbc.ATTN_OK) != fbc.attn_strerror(fbc.ATTN_ERR_INVALID)


# A fake, 16-byte aligned, never dereferenced address: every call below must be
# rejected before the library touches the device.
P = 1 << 20
GOOD = dict(B=1, Hq=4, Hkv=2, S=128, Dqk=128, Dv=128, causal=1, scale=0.088, dtype=fbc.ATTN_BF16)


def _call(ptrs=(P, P, P, P), descale=None, flags=0, **kw):
    a = dict(GOOD)
    a.update(kw)
    return fbc.attn_fwd_ex(*ptrs, a["B"], a["Hq"], a["Hkv"], a["S"], a["Dqk"], a["Dv"], a["causal"], a["scale"],
                           a["dtype"], descale, None, flags)


@pytest.mark.parametrize("kw", [
    dict(ptrs=(0, P, P, P)), dict(ptrs=(P, P, P, 0)), dict(ptrs=(P + 8, P, P, P)), dict(ptrs=(P, P, P + 4, P)),
    dict(B=0), dict(S=0), dict(S=-3), dict(Hq=0), dict(Hkv=0), dict(Dqk=0), dict(Dv=-1), dict(Hq=6, Hkv=4),
    dict(scale=float("nan")), dict(scale=float("inf")), dict(scale=-0.1),
    dict(descale=(1.0, 0.0, 1.0)), dict(descale=(1.0, 1.0, float("nan"))), dict(descale=(-1.0, 1.0, 1.0)),
    dict(scale=3e38, descale=(8.0, 8.0, 1.0)),  # folded score scale beyond the float range
    dict(flags=8), dict(flags=1 << 31), dict(flags=15, dtype=fbc.ATTN_FP8_E4M3),
    # device-resident descales: a null or misaligned pointer
    dict(flags=fbc.ATTN_FLAG_DESCALE_DEVICE, dtype=fbc.ATTN_FP8_E4M3),
    dict(flags=fbc.ATTN_FLAG_DESCALE_DEVICE, dtype=fbc.ATTN_FP8_E4M3, descale=P + 2),
    dict(B=1 << 20, S=1 << 30, Hq=1 << 10, Hkv=1 << 10), dict(S=1 << 22, Hq=1 << 12, Hkv=1 << 12),
])
def test_invalid_arguments(kw):
    assert _call(**kw) == fbc.ATTN_ERR_INVALID


@pytest.mark.parametrize("kw", [
    dict(causal=0), dict(dtype=2), dict(dtype=-1), dict(Dqk=64, Dv=64), dict(Dqk=128, Dv=64), dict(Dqk=256, Dv=256),
    dict(flags=fbc.ATTN_FLAG_EXACT_P), dict(flags=fbc.ATTN_FLAG_NO_BLOCKSCALE),  # the ablations are FP8-only
    dict(flags=fbc.ATTN_FLAG_DESCALE_DEVICE, descale=P),  # device-resident descales too
])
def test_unsupported_arguments(kw):
    assert _call(**kw) == fbc.ATTN_ERR_UNSUPPORTED


def test_plain_entry_point_validates_too():
    assert fbc.attn_fwd(0, P, P, P, 1, 1, 1, 16, 128, 128, 1, 0.1, fbc.ATTN_BF16) == fbc.ATTN_ERR_INVALID
    assert fbc.attn_fwd(P, P, P, P, 1, 1, 1, 16, 128, 128, 0, 0.1, fbc.ATTN_BF16) == fbc.ATTN_ERR_UNSUPPORTED


def test_binding_has_no_cpu_path():
    """The Python layer only marshals arguments: it refuses CPU tensors rather
    than computing anything itself."""
    import torch
    q = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fbc.flash_attn_func(q, q, q, causal=True)


@pytest.mark.parametrize("args,code", [
    ((0, P, P, 10, 128, 0), fbc.ATTN_ERR_INVALID), ((P, 0, P, 10, 128, 0), fbc.ATTN_ERR_INVALID),
    ((P, P, 0, 10, 128, 0), fbc.ATTN_ERR_INVALID), ((P + 1, P, P, 10, 128, 0), fbc.ATTN_ERR_INVALID),
    ((P, P, P + 2, 10, 128, 0), fbc.ATTN_ERR_INVALID), ((P, P + 8, P, 10, 128, 0), fbc.ATTN_ERR_INVALID), ((P, P, P, 0, 128, 0), fbc.ATTN_ERR_INVALID),
    ((P, P, P, -4, 128, 1), fbc.ATTN_ERR_INVALID), ((P, P, P, 10, 128, 2), fbc.ATTN_ERR_INVALID),
    ((P, P, P, 10, 96, 0), fbc.ATTN_ERR_UNSUPPORTED), ((P, P, P, 10, 512, 1), fbc.ATTN_ERR_UNSUPPORTED),
])
def test_quantize_argument_checks(args, code):
    assert fbc.attn_quantize_e4m3(*args) == code


def _call_lse(lse, ptrs=(P, P, P, P), **kw):
    a = dict(GOOD)
    a.update(kw)
    return fbc.attn_fwd_lse(*ptrs, lse, a["B"], a["Hq"], a["Hkv"], a["S"], a["Dqk"], a["Dv"], a["causal"],
                            a["scale"], a["dtype"], None, None, 0)


@pytest.mark.parametrize("lse,kw,code", [
    (0, {}, fbc.ATTN_ERR_INVALID), (P + 2, {}, fbc.ATTN_ERR_INVALID),  # null or misaligned lse
    (P, dict(ptrs=(0, P, P, P)), fbc.ATTN_ERR_INVALID), (P, dict(S=0), fbc.ATTN_ERR_INVALID),
    (P, dict(causal=0), fbc.ATTN_ERR_UNSUPPORTED), (P, dict(Dqk=64, Dv=64), fbc.ATTN_ERR_UNSUPPORTED),
])
def test_lse_entry_point_argument_checks(lse, kw, code):
    assert _call_lse(lse, **kw) == code


@pytest.mark.parametrize("Sq,Sk,lse,code", [
    (128, 100, P, fbc.ATTN_ERR_INVALID),   # fewer keys than queries
    (0, 100, P, fbc.ATTN_ERR_INVALID), (128, 256, P + 2, fbc.ATTN_ERR_INVALID),
])
def test_prefix_entry_point_argument_checks(Sq, Sk, lse, code):
    a = dict(GOOD)
    assert fbc.attn_fwd_prefix(P, P, P, P, lse, a["B"], a["Hq"], a["Hkv"], Sq, Sk, a["Dqk"], a["Dv"], a["causal"],
                               a["scale"], a["dtype"], None, None, 0) == code


def test_flash_attn_func_refuses_descales_with_bf16():
    """A dequantisation factor other than 1 on bfloat16 inputs would be silently
    ignored by the kernels: the wrapper refuses it (before any device work)."""
    import torch

    q = torch.zeros((1, 4, 2, 128), dtype=torch.bfloat16)
    for kw in (dict(descale_q=0.5), dict(descale_k=2.0), dict(descale_v=0.25)):
        with pytest.raises(ValueError, match="descale"):
            fbc.flash_attn_func(q, q, q, causal=True, **kw)


def test_flash_attn_func_keeps_flash_attention_call_meanings():
    """flash_attn_func takes flash-attention's positional order (q, k, v,
    softmax_scale, causal) and keywords; what the kernels do not implement is
    refused before any device work instead of being computed differently:
    causal=False, dropout, a sliding window, softcap, ALiBi.
    q_descale/k_descale/v_descale are aliases of descale_q/k/v, one factor
    per tensor."""
    import torch

    q = torch.zeros((1, 4, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(NotImplementedError, match="causal"):
        fbc.flash_attn_func(q, q, q, None, False)
    with pytest.raises(NotImplementedError, match="causal"):
        fbc.flash_attn_func(q, q, q, causal=False)
    for kw in (dict(dropout_p=0.1), dict(window_size=(128, 0)), dict(window_size=(-1, 64)), dict(softcap=30.0),
               dict(alibi_slopes=torch.zeros(2))):
        with pytest.raises(NotImplementedError):
            fbc.flash_attn_func(q, q, q, causal=True, **kw)
    with pytest.raises(ValueError, match="not both"):
        fbc.flash_attn_func(q, q, q, causal=True, q_descale=1.0, descale_q=1.0)
    with pytest.raises(ValueError, match="one factor per tensor"):
        fbc.flash_attn_func(q, q, q, causal=True, k_descale=torch.ones(1, 2))
    with pytest.raises(ValueError, match="descale"):  # bfloat16 with a factor, through the alias
        fbc.flash_attn_func(q, q, q, causal=True, v_descale=torch.full((1,), 0.5))
    # accepted options reach the device checks (CPU tensors: refused there, no fallback)
    for kw in (dict(window_size=(-1, -1)), dict(window_size=(-1, 0)), dict(deterministic=True),
               dict(q_descale=torch.ones(1))):
        with pytest.raises(ValueError, match="one GPU"):
            fbc.flash_attn_func(q, q, q, 0.1, True, **kw)


def test_flash_attn_fp8_func_takes_bfloat16_only():
    import torch

    q = torch.zeros((1, 4, 2, 128), dtype=torch.float32)
    with pytest.raises(TypeError, match="bfloat16"):
        fbc.flash_attn_fp8_func(q, q, q)
