"""ctypes binding of libfp8_bf16_causal.so: the C entry points under the same
names, with argument marshalling only (every step of the computation runs in
the library's HIP kernels)."""
from __future__ import annotations

import ctypes
import os

ATTN_BF16 = 0
ATTN_FP8_E4M3 = 1
ATTN_OK = 0
ATTN_ERR_INVALID = -1
ATTN_ERR_UNSUPPORTED = -2
ATTN_ERR_LAUNCH = -3
ATTN_FLAG_EXACT_P = 1
ATTN_FLAG_NO_BLOCKSCALE = 2
ATTN_FLAG_DESCALE_DEVICE = 4

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8_bf16_causal.so")
_lib = None


def load():
    """Load the built library; raises if it has not been built (there is no
    fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; "
                           "g.build()' or python -m fp8_bf16_causal_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_uint
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32]
    lib.attn_fwd.restype = i32
    # descale_qkv: a host float[3] or, with ATTN_FLAG_DESCALE_DEVICE, a device address
    lib.attn_fwd_ex.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp, vp, u32]
    lib.attn_fwd_ex.restype = i32
    lib.attn_fwd_lse.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp, vp, u32]
    lib.attn_fwd_lse.restype = i32
    lib.attn_fwd_prefix.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp, vp,
                                    u32]
    lib.attn_fwd_prefix.restype = i32
    lib.attn_quantize_e4m3.argtypes = [vp, vp, vp, ctypes.c_longlong, i32, i32, vp]
    lib.attn_quantize_e4m3.restype = i32
    lib.attn_strerror.argtypes = [i32]
    lib.attn_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _descale(descale_qkv, flags):
    """The descale_qkv argument: None; a device address (int) with
    ATTN_FLAG_DESCALE_DEVICE; else three host floats, as a float[3] that the
    caller keeps alive through the call."""
    if descale_qkv is None:
        return None
    if flags & ATTN_FLAG_DESCALE_DEVICE:
        return ctypes.c_void_p(int(descale_qkv))
    return (ctypes.c_float * 3)(*[float(x) for x in descale_qkv])


def attn_fwd(q, k, v, out, B, Hq, Hkv, S, Dqk, Dv, causal, scale, dtype) -> int:
    """q, k, v, out: device addresses (ints). Returns the library's code."""
    return load().attn_fwd(q, k, v, out, B, Hq, Hkv, S, Dqk, Dv, causal, scale, dtype)


def attn_fwd_ex(q, k, v, out, B, Hq, Hkv, S, Dqk, Dv, causal, scale, dtype, descale_qkv=None, stream=None,
                flags=0) -> int:
    """descale_qkv: (dq, dk, dv), a device address with ATTN_FLAG_DESCALE_DEVICE,
    or None; stream: a hipStream_t as int, or None."""
    ds = _descale(descale_qkv, flags)
    return load().attn_fwd_ex(q, k, v, out, B, Hq, Hkv, S, Dqk, Dv, causal, scale, dtype, ds, stream, flags)


def attn_fwd_lse(q, k, v, out, lse, B, Hq, Hkv, S, Dqk, Dv, causal, scale, dtype, descale_qkv=None, stream=None,
                 flags=0) -> int:
    """attn_fwd_ex plus lse: the device address of B*Hq*S float32 log-sum-exps."""
    ds = _descale(descale_qkv, flags)
    return load().attn_fwd_lse(q, k, v, out, lse, B, Hq, Hkv, S, Dqk, Dv, causal, scale, dtype, ds, stream, flags)


def attn_fwd_prefix(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, Dqk, Dv, causal, scale, dtype, descale_qkv=None,
                    stream=None, flags=0) -> int:
    """Sq queries (the last Sq positions) over Sk >= Sq keys; lse: device
    address of B*Hq*Sq float32 or None."""
    ds = _descale(descale_qkv, flags)
    return load().attn_fwd_prefix(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, Dqk, Dv, causal, scale, dtype, ds, stream,
                                  flags)


def attn_quantize_e4m3(x, y, scale, rows, dim, hadamard, stream=None) -> int:
    """x, y, scale: device addresses (ints); see attn_quantize_e4m3 in the C header."""
    return load().attn_quantize_e4m3(x, y, scale, rows, dim, hadamard, stream)


def attn_strerror(code: int) -> str:
    return load().attn_strerror(code).decode()
