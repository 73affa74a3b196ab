"""TEST INFRASTRUCTURE ONLY: CPU oracle of the FP8 quantize prologue (per-tensor
e4m3 quantisation of Q, K or V, with an optional Hadamard rotation of the rows
of Q and K). Nothing in the product path imports this module.

What the pages fix [spbcomputers.ru ZYFA article, section "Точность: ошибка
FP8 ниже, чем у AITER" and the FAQ entry on the Hadamard rotation;
captivela.com "Zyphra Luncurkan ZYFA", section "Akurasi Jauh Lebih Baik, Bukan
Cuma Cepat"]: most of a full model's FP8 attention error comes from
quantising Q, K and V; rotating Q and K by a Hadamard transform roughly halves
that input error. A rotation by one orthogonal matrix H leaves Q K^T
unchanged ((Q H)(K H)^T = Q K^T), so the attention result is that of the
unrotated inputs.

Readings where the pages are silent:
  * the rotation is the normalised Walsh-Hadamard transform of each row in
    blocks of n = 128 elements when the row length is a multiple of 128, else
    of n = 64 (a 192-wide row is three 64-blocks);
  * quantisation is per tensor: s = amax / 448 (1 when amax = 0), code =
    e4m3fn(y / s) rounded to nearest, ties to even, saturating at 448.

The codes are integers decided by floating point, so this oracle takes every
decision in the kernel's precision (IEEE fp32) and order: the butterflies of
the fast transform run over index bits 0, 1, ..., log2(n)-1 (pairs (i, i+h)
become (a + b, a - b) for h = 1, 2, 4, ...), then one multiply by the fp32
constant 1/sqrt(n); amax is exact; s and y / s are correctly rounded fp32
divisions. Every step is written out below with numpy float32 arithmetic.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = np.float32(448.0)


def bf16_to_f32(codes: np.ndarray) -> np.ndarray:
    """Exact fp32 values of bfloat16 bit patterns (the top 16 bits of an fp32)."""
    return (np.asarray(codes, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def hadamard_block(dim: int) -> int:
    if dim % 64 != 0:
        raise ValueError("row length must be a multiple of 64")
    return 128 if dim % 128 == 0 else 64


def fwht_f32(x: np.ndarray, n: int) -> np.ndarray:
    """Normalised Walsh-Hadamard transform of consecutive n-element blocks of
    the last axis, in fp32, butterflies over bits 0 .. log2(n)-1 in that order."""
    y = np.array(x, dtype=np.float32, copy=True)
    shape = y.shape
    y = y.reshape(-1, shape[-1] // n, n)
    h = 1
    while h < n:
        y = y.reshape(y.shape[0], y.shape[1], n // (2 * h), 2, h)
        a = y[:, :, :, 0, :].copy()
        b = y[:, :, :, 1, :].copy()
        y[:, :, :, 0, :] = a + b  # fp32 adds: numpy keeps float32
        y[:, :, :, 1, :] = a - b
        y = y.reshape(y.shape[0], y.shape[1], n)
        h *= 2
    y = y * np.float32(1.0 / np.sqrt(n))
    return y.reshape(shape).astype(np.float32)


_POS = None


def _positive_values() -> np.ndarray:
    """The 127 finite non-negative e4m3fn values, in code order (decoded from
    the format definition: 4 exponent bits with bias 7, 3 mantissa bits,
    subnormals m * 2^-9)."""
    global _POS
    if _POS is None:
        v = []
        for c in range(127):
            e, m = c >> 3, c & 7
            v.append(m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
        _POS = np.array(v, dtype=np.float64)
    return _POS


def e4m3_codes(q: np.ndarray) -> np.ndarray:
    """e4m3fn codes of fp32 values: magnitude rounded to nearest, ties to the
    even code, saturating at 448; sign bit from the sign of q (-0 gives 0x80)."""
    q = np.asarray(q, dtype=np.float32)
    pos = _positive_values()
    mag = np.abs(q).astype(np.float64)
    hi = np.clip(np.searchsorted(pos, mag, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    dlo, dhi = mag - pos[lo], pos[hi] - mag
    code = np.where((dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0)), hi, lo)
    code = np.where(mag >= pos[126], 126, code)
    return (code | np.where(np.signbit(q), 0x80, 0)).astype(np.uint8)


def quantize_e4m3(x_bf16: np.ndarray, hadamard: bool) -> tuple[np.ndarray, np.float32, np.float32]:
    """Per-tensor e4m3 quantisation of a bfloat16 tensor [..., dim] (bit
    patterns), rows optionally rotated first. Returns (codes uint8 [..., dim],
    dequantisation factor s, amax), both fp32."""
    x = bf16_to_f32(x_bf16)
    y = fwht_f32(x, hadamard_block(x.shape[-1])) if hadamard else x
    amax = np.float32(np.max(np.abs(y))) if y.size else np.float32(0.0)
    s = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    q = (y / s).astype(np.float32)
    return e4m3_codes(q), s, amax
