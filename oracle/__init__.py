"""fp64 CPU oracle for causal prefill attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and its
Python binding) never does, and this package imports nothing from it.

* ``attention`` -- exact causal attention in fp64 (``attn_oracle.c``), on the
  same raw BF16 / e4m3fn element codes the GPU receives, decoded from the
  format definitions.
* ``probs`` -- the probability matrix of one head, for tiny sizes.
* ``leanp`` -- a step-by-step fp64 model of the pages' FP8 softmax, for
  pinning the encoding (diagnostic, not the pass/fail target).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import leanp  # noqa: F401  (re-exported)

BF16 = 0
FP8_E4M3 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from .build import build
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_bf16.restype = f64
    lib.oracle_decode_e4m3fn.argtypes = [ctypes.c_uint8]
    lib.oracle_decode_e4m3fn.restype = f64
    lib.oracle_num_threads.argtypes = [i32]
    lib.oracle_num_threads.restype = i32
    lib.oracle_attn_f64.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f64, f64, f64, f64, vp, i64,
                                    vp, i32]
    lib.oracle_attn_f64.restype = i32
    lib.oracle_attn_lse_f64.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f64, f64, f64, f64, vp, i64,
                                        vp, vp, i32]
    lib.oracle_attn_lse_f64.restype = i32
    lib.oracle_attn_prefix_f64.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f64, f64, f64, f64,
                                           vp, i64, vp, vp, i32]
    lib.oracle_attn_prefix_f64.restype = i32
    lib.oracle_attn_probs_f64.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, f64, f64, f64, i32, i32, vp]
    lib.oracle_attn_probs_f64.restype = i32
    _lib = lib
    return lib


def _codes(x: np.ndarray, dtype: int) -> np.ndarray:
    want = np.uint16 if dtype == BF16 else np.uint8
    x = np.ascontiguousarray(x)
    if x.dtype != want:
        raise TypeError(f"expected raw {want.__name__} element codes, got {x.dtype}")
    return x


def decode_bf16(codes) -> np.ndarray:
    lib = _load()
    c = np.asarray(codes, dtype=np.uint16)
    return np.array([lib.oracle_decode_bf16(int(v)) for v in c.ravel()]).reshape(c.shape)


def decode_e4m3fn(codes) -> np.ndarray:
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_decode_e4m3fn(int(v)) for v in c.ravel()]).reshape(c.shape)


def num_threads(requested: int = 0) -> int:
    return _load().oracle_num_threads(requested)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, dtype: int, scale: float, dq: float = 1.0,
              dk: float = 1.0, dv: float = 1.0, rows=None, nthreads: int = 0, return_lse: bool = False):
    """Exact causal attention, fp64.

    q [B,S,Hq,Dqk], k [B,Sk,Hkv,Dqk], v [B,Sk,Hkv,Dv]: raw codes (uint16 bf16
    or uint8 e4m3fn), Sk >= S; the queries are the last S positions, so query
    i sees keys j <= i + Sk - S. rows: None (returns [B,S,Hq,Dv]) or an int
    array [n,3] of (b, h, i) (returns [n,Dv]). With return_lse, also the
    natural log-sum-exp of each row's logits scale*dq*dk*<q_i, k_j> over its
    visible keys ([B,Hq,S], or [n]).
    """
    lib = _load()
    q, k, v = _codes(q, dtype), _codes(k, dtype), _codes(v, dtype)
    B, S, Hq, Dqk = q.shape
    Sk, Hkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    if k.shape != (B, Sk, Hkv, Dqk) or v.shape != (B, Sk, Hkv, Dv) or Sk < S:
        raise ValueError("shape mismatch")
    if rows is None:
        out = np.empty((B, S, Hq, Dv), dtype=np.float64)
        lse = np.empty((B, Hq, S), dtype=np.float64) if return_lse else None
        rp, n = None, 0
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        out = np.empty((rows.shape[0], Dv), dtype=np.float64)
        lse = np.empty((rows.shape[0],), dtype=np.float64) if return_lse else None
        rp, n = rows.ctypes.data, rows.shape[0]
    rc = lib.oracle_attn_prefix_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, dtype, B, Hq, Hkv, S, Sk, Dqk, Dv,
                                    float(scale), float(dq), float(dk), float(dv), rp, n, out.ctypes.data,
                                    lse.ctypes.data if return_lse else None, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_prefix_f64 rejected its arguments")
    return (out, lse) if return_lse else out


def probs(q: np.ndarray, k: np.ndarray, dtype: int, scale: float, b: int = 0, h: int = 0, dq: float = 1.0,
          dk: float = 1.0) -> np.ndarray:
    """P[i, j] of one head (zeros above the diagonal). Tiny S only."""
    lib = _load()
    q, k = _codes(q, dtype), _codes(k, dtype)
    B, S, Hq, Dqk = q.shape
    Hkv = k.shape[2]
    P = np.empty((S, S), dtype=np.float64)
    rc = lib.oracle_attn_probs_f64(q.ctypes.data, k.ctypes.data, dtype, B, Hq, Hkv, S, Dqk, float(scale),
                                   float(dq), float(dk), b, h, P.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_attn_probs_f64 rejected its arguments")
    return P


def dequantize(x: np.ndarray, dtype: int, factor: float = 1.0) -> np.ndarray:
    """fp64 values of raw codes times a per-tensor factor (the oracle's decoders)."""
    tab = _table(dtype)
    return tab[np.asarray(x).astype(np.int64)] * factor


_tables = {}


def _table(dtype: int) -> np.ndarray:
    if dtype not in _tables:
        n = 1 << (16 if dtype == BF16 else 8)
        dec = decode_bf16 if dtype == BF16 else decode_e4m3fn
        _tables[dtype] = dec(np.arange(n))
    return _tables[dtype]
