"""Diagnostic fp64 model of the pages' FP8 softmax ("Lean P") -- TEST INFRASTRUCTURE.

Only tests, the package smoke check and the benchmark's CPU-baseline leg may
import this module. It shares no code with the HIP kernels.

This is NOT the pass/fail oracle for the GPU FP8 path: that is the exact
attention in ``attn_oracle.c`` (the FP8 path approximates it). This model
spells out, step by step and in the pages' order, the three pieces of the FP8
softmax so that each can be pinned on its own:

1. Lean P encoding.  Read as an unsigned integer, an e4m3 code grows by 8 for
   every doubling of the value it encodes, so the code of 2**x is close to
   ``8*x + C``: one multiply-add and one convert to an integer produce the
   probability's FP8 bits directly, with no exponential.
   [spbcomputers.ru ZYFA article, section on the three techniques ("Три
   приёма"), Lean P; captivela.com "Zyphra Luncurkan ZYFA", section "Tiga Trik
   ZYFA", first trick; ZYFA abstract (airebao.com), technique (1).]
2. Power-of-two scale per 64-key block.  Before rounding, each block of 64
   keys of a row is multiplied by 2**k so that its largest probability sits at
   the top of the e4m3 range; the scaled matrix instruction divides the factor
   back out.  [same sections; abstract technique (3).]
3. Normalisation by the sum of the rounded probabilities.  The row sum is the
   sum of the already-rounded (scaled back) probabilities, so the weights sum
   to one.  [same sections; abstract technique (3).]

Readings where the pages leave a step open:
* x is log2 of the probability relative to the running row max, natural-exp
  softmax being 2**(z*log2(e)).
* C = 55.63 code units (LEANP_C).  The pages give no value; this is the
  minimax choice for round-to-nearest, the only narrow range that meets the
  pages' own error bound of 7.5 percent, and it keeps exact powers of two
  exact: round(8n + 55.63) = 8n + 56.
* The block exponent is k = floor(8 - t_max) with t_max the block's largest x,
  so the block maximum lands in (2**7, 2**8]: its code is at most 120, never
  the NaN code 0x7F.  k is capped at 127 (the range of an E8M0 scale byte);
  weights below 2**-119 of the row max then flush to zero.
* The integer convert rounds half to even and saturates to [0, 255]; codes are
  then capped at 126 (the largest finite e4m3 code).
* Keys are processed in tiles of 128 (the unit the pages cost: 32 queries by
  128 keys); the reference max is updated once per tile and the accumulated
  output and sum are rescaled by 2**(m_old - m_new) exactly when it moves.
  Optionally (lazy_log2 > 0) it moves only when a tile's max exceeds it by
  more than lazy_log2 binades, as the GPU kernels do with 8.
"""
from __future__ import annotations

import math

import numpy as np

LEANP_C = 55.63
BLOCK_KEYS = 64
TILE_KEYS = 128
LOG2E = 1.4426950408889634


def _e4m3fn_table() -> np.ndarray:
    """Values of all 256 e4m3fn codes, written from the format definition."""
    tab = np.empty(256, dtype=np.float64)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 0xF, c & 7
        if e == 0xF and m == 7:
            v = math.nan
        elif e == 0:
            v = m * 2.0 ** -9
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        tab[c] = -v if s else v
    return tab


E4M3FN = _e4m3fn_table()
# positive finite codes 0..126 in increasing value order (the format is monotone)
_POS_VALUES = E4M3FN[:127]


def leanp_code(x, C: float = LEANP_C, rounding: str = "rne") -> np.ndarray:
    """Lean P code of 2**x: convert(8*x + C) to an integer, clamped to [0, 126].

    ``rounding`` is the integer convert's rounding: "rne" (half to even) or
    "trunc" (toward zero). Negative and -inf inputs give code 0 (value 0).
    """
    y = 8.0 * np.asarray(x, dtype=np.float64) + C
    y = np.where(np.isnan(y), -np.inf, y)
    if rounding == "rne":
        r = np.rint(np.clip(y, -1.0, 255.0))
    elif rounding == "trunc":
        r = np.trunc(np.clip(y, -1.0, 255.0))
    else:
        raise ValueError(rounding)
    return np.clip(r, 0, 126).astype(np.int64)


def e4m3_value(code) -> np.ndarray:
    return E4M3FN[np.asarray(code, dtype=np.int64)]


def e4m3_round_rne(x) -> np.ndarray:
    """Exact round-to-nearest-even of non-negative values to e4m3fn codes
    (the comparison softmax of the pages: exponential, then round to FP8).
    Values above 448 saturate to 448."""
    x = np.asarray(x, dtype=np.float64)
    idx = np.searchsorted(_POS_VALUES, x, side="left")  # first value >= x
    idx = np.clip(idx, 0, 126)
    lo = np.clip(idx - 1, 0, 126)
    vlo, vhi = _POS_VALUES[lo], _POS_VALUES[idx]
    dlo, dhi = np.abs(x - vlo), np.abs(vhi - x)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (idx % 2 == 0))
    code = np.where(pick_hi, idx, lo)
    code = np.where(x >= _POS_VALUES[126], 126, code)
    return code.astype(np.int64)


def block_exponent(t_max) -> np.ndarray:
    """k = floor(8 - t_max), kept in [0, 127]; t_max = -inf (an all-masked
    block) gives 127."""
    t = np.asarray(t_max, dtype=np.float64)
    k = np.floor(8.0 - t)
    return np.clip(np.where(np.isfinite(k), k, 127.0), 0.0, 127.0).astype(np.int64)


def leanp_attention_row(z: np.ndarray, vrows: np.ndarray, C: float = LEANP_C, rounding: str = "rne",
                        block_scale: bool = True, exact_p: bool = False,
                        tile_keys: int = TILE_KEYS, lazy_log2: float = 0.0) -> tuple[np.ndarray, float]:
    """One query row of the FP8 softmax model.

    z: log2-domain scores z_j = s_j * log2(e) of the visible keys, in key order
       (masked keys are simply absent).
    vrows: [len(z), Dv] dequantised V rows of those keys.
    Returns (output row before the dv factor, final rounded-probability sum).

    block_scale=False drops step 2: every block keeps k = 0, i.e. the plain
    probabilities in [0, 1] are encoded, as an unscaled FP8 softmax would;
    exact_p=True replaces the Lean P code with exact e4m3 rounding of 2**x.
    tile_keys: keys per running-max update (a multiple of the 64-key block).
    lazy_log2: the reference max moves to a tile's max only when that max
      exceeds it by more than this many binades (0: on every rise). Any value
      gives the same exact output; it changes which rounding each code sees.
    """
    n = z.shape[0]
    dv = vrows.shape[1]
    m = -np.inf
    l = 0.0
    o = np.zeros(dv, dtype=np.float64)
    for t0 in range(0, n, tile_keys):
        zt = z[t0:t0 + tile_keys]
        tmax = float(np.max(zt))
        m_new = tmax if (m == -np.inf or tmax - m > lazy_log2) else m
        alpha = 0.0 if m == -np.inf else 2.0 ** (m - m_new)
        l *= alpha
        o *= alpha
        for b0 in range(0, zt.shape[0], BLOCK_KEYS):
            zb = zt[b0:b0 + BLOCK_KEYS]
            x = zb - m_new
            k = int(block_exponent(np.max(x))) if block_scale else 0
            if exact_p:
                code = e4m3_round_rne(2.0 ** (x + k))
            else:
                code = leanp_code(x + k, C, rounding)
            p = e4m3_value(code) * 2.0 ** (-k)
            l += float(np.sum(p))
            o += p @ vrows[t0 + b0:t0 + b0 + zb.shape[0]]
        m = m_new
    return o / l, l


def leanp_attention(qd: np.ndarray, kd: np.ndarray, vd: np.ndarray, scale: float, dv: float = 1.0,
                    rows=None, **kw) -> np.ndarray:
    """FP8 softmax model over dequantised fp64 inputs.

    qd [B,S,Hq,Dqk], kd [B,S,Hkv,Dqk], vd [B,S,Hkv,Dv] (already multiplied by
    their per-tensor factors, so ``scale`` here is the plain softmax scale).
    rows: None for every row (returns [B,S,Hq,Dv]) or a list of (b, h, i)
    (returns [len(rows), Dv]). Small sizes only: a Python loop per row.
    """
    B, S, Hq, _ = qd.shape
    Hkv = kd.shape[2]
    G = Hq // Hkv
    c = scale * LOG2E
    if rows is None:
        out = np.zeros((B, S, Hq, vd.shape[3]))
        it = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(S)]
    else:
        it = list(rows)
        out = np.zeros((len(it), vd.shape[3]))
    for n, (b, h, i) in enumerate(it):
        g = h // G
        z = (kd[b, :i + 1, g, :] @ qd[b, i, h, :]) * c
        o, _ = leanp_attention_row(z, vd[b, :i + 1, g, :], **kw)
        if rows is None:
            out[b, i, h] = dv * o
        else:
            out[n] = dv * o
    return out


# ---------------------------------------------------------------- fp32 decisions
# The code is an integer decided by floating point, so a bit-level comparison
# with a GPU takes the decision in the GPU's precision: with the score scale c
# (base 2, per raw score unit), the reference max m and the block exponent k,
# the pages' 8 x + C with x = c (s - m) + k is formed as one fp32 fused
# multiply-add of the raw score s with 8c onto a per-(row, block) bias
# C + 8k - 8c m (itself one fp32 fused multiply-add), then rounded half to
# even and saturated to [0, 255] by the integer convert.

from fractions import Fraction  # noqa: E402


def round_f32(x: Fraction) -> float:
    """x rounded to the nearest float32 (ties to even), returned as a Python
    float holding that float32 value. Overflow gives +-inf."""
    if x == 0:
        return 0.0
    sign = -1.0 if x < 0 else 1.0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()  # 2^e <= a < 2^(e+2)
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)  # subnormals share the exponent of the smallest normal
    q = a / Fraction(2) ** (e - 23)  # 24-bit significand scale
    n, rem = divmod(q.numerator, q.denominator)
    half = Fraction(rem, q.denominator)
    if half > Fraction(1, 2) or (half == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = math.ldexp(float(n), e - 23)
    if v > 3.4028234663852886e38:
        return sign * math.inf
    return sign * v


def fma_f32(a: float, b: float, c: float) -> float:
    """fp32 fused multiply-add: a*b + c exactly, rounded once to float32
    (a, b, c are float32 values; infinities follow IEEE rules)."""
    if not (math.isfinite(a) and math.isfinite(b) and math.isfinite(c)):
        return float(np.float32(a) * np.float32(b) + np.float32(c))
    return round_f32(Fraction(a) * Fraction(b) + Fraction(c))


def cvt_u8_rne(f: float) -> int:
    """The integer convert of a code: round half to even, saturate to [0, 255];
    -inf and NaN give 0."""
    if math.isnan(f) or f <= 0.0:
        return 0
    if f >= 255.0:
        return 255
    return int(round(f))  # Python rounds half to even


def tile_codes_fp32(s, c: float, C: float = LEANP_C):
    """Codes of one query row's first 128-key tile, every decision in fp32.

    s: the 128 raw scores of the tile (float32 values; -inf for masked keys),
    c: the base-2 score scale (a float32 value). On the first tile the
    reference max m is the tile's max. Each 64-key block b gets
    k_b = clamp(floor(8 - c (max_b - m)), 0, 127) and the bias
    C + 8 k_b - 8c m; code_j = convert(8c s_j + bias). Returns
    (codes [128] int, [k_a, k_b], m)."""
    f32 = lambda v: float(np.float32(v))  # noqa: E731  one fp32 rounding
    s = [f32(v) for v in s]
    c = f32(c)
    c8 = 8.0 * c
    blocks = [s[0:BLOCK_KEYS], s[BLOCK_KEYS:2 * BLOCK_KEYS]]
    mx = [max(b) for b in blocks]
    m = max(mx)
    codes, ks = [], []
    for b, bmax in zip(blocks, mx):
        t = f32(f32(bmax - m) * c) if math.isfinite(bmax) else -math.inf
        kf = math.floor(f32(8.0 - t)) if math.isfinite(t) else math.inf
        k = int(min(max(kf, 0.0), 127.0))
        bias = fma_f32(-c8, m, f32(f32(C) + 8.0 * k))
        codes += [cvt_u8_rne(fma_f32(v, c8, bias)) for v in b]
        ks.append(k)
    return np.array(codes, dtype=np.int64), ks, m
