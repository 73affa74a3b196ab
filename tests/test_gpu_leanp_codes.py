"""GPU: the Lean P codes themselves, read back through the output.

The pages' FP8 softmax writes each probability's e4m3 bits with one
multiply-add and one integer convert, after a power-of-two scale per 64-key
block [spbcomputers.ru ZYFA article, section "Три приёма, которые дали
ускорение", Lean P; captivela.com "Zyphra Luncurkan ZYFA", section "Tiga Trik
ZYFA Biar Cepat dan Akurat", first and third tricks].

Construction (no test-only kernel): one 128-key tile (S = 128), V one-hot
(V[j] = e_j, dv = 1), so that output column d of row i is p_d / l with p_d
the rounded probability of key d. Q and K are e4m3 powers of two chosen so
that every score Q.K_j is a prescribed value on a 2^-12 lattice, exact in the
matrix core's fp32 sums. The softmax scale makes the base-2 score scale c a
power of two, so the reference max, the block exponents and the biases are
exact, and every code decision can be predicted in fp32
(oracle.leanp.tile_codes_fp32). For each row, the codes are recovered from
the ratios of its outputs to that of its row-max key (code 120, exponent 8)
and compared with the prediction, key by key: scores on a fine grid over
20 binades, exact ties of the convert (half to even), saturation at 0,
equal scores, a row max in either block and masked keys (output exactly 0).
"""
import sys

import numpy as np
import pytest
import torch

from oracle import leanp

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634
LATTICE = 2.0 ** -12
S = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_bf16_causal_amd._lib as L
    L.load()
    torch.cuda.set_device(0)


def _scale_for(c_target):
    """A float32 softmax scale whose base-2 score scale, as the library folds
    it (float32 of scale * log2(e) in double), is exactly c_target."""
    s = np.float32(c_target / LOG2E)
    for _ in range(64):
        c = np.float32(np.float64(s) * LOG2E)
        if c == np.float32(c_target):
            return float(s)
        s = np.nextafter(s, np.float32(np.inf) if c < c_target else np.float32(0))
    raise AssertionError("no exact scale")


def _exp_of_dim(d):
    """Score bit b = d - 12 (2^-12 .. 2^11) is the product of Q[d] = 2^qe and
    K[d] = 2^(b - qe), both normal e4m3 values."""
    b = d - 12
    qe = -6 if b <= -1 else (0 if b <= 8 else 3)
    return b, qe, b - qe


def _e4m3_pow2(e, neg=False):
    assert -6 <= e <= 8
    return ((e + 7) << 3) | (0x80 if neg else 0)


def _inputs(t):
    """t: [H][128] target scores (multiples of 2^-12, |t| < 2^12). Returns Q,
    K, V codes [1, S, H, 128] (uint8): every query row of head h holds the
    same Q, so s_ij = t[h][j] for every row i."""
    H = len(t)
    q = np.zeros((1, S, H, 128), dtype=np.uint8)
    k = np.zeros((1, S, H, 128), dtype=np.uint8)
    v = np.zeros((1, S, H, 128), dtype=np.uint8)
    for d in range(24):
        _, qe, _ = _exp_of_dim(d)
        q[0, :, :, d] = _e4m3_pow2(qe)
    for h in range(H):
        for j in range(S):
            a = t[h][j] / LATTICE
            assert a == int(a) and abs(a) < 2 ** 24, (h, j, t[h][j])
            a, neg = abs(int(a)), t[h][j] < 0
            for d in range(24):
                if (a >> d) & 1:
                    k[0, j, h, d] = _e4m3_pow2(_exp_of_dim(d)[2], neg)
            v[0, j, h, j] = 0x38  # e4m3 1.0
    return q, k, v


def _run(q, k, v, scale):
    import fp8_bf16_causal_amd as fbc
    dev = torch.device("cuda", 0)
    t = [torch.from_numpy(x).to(dev).view(torch.float8_e4m3fn) for x in (q, k, v)]
    o = fbc.flash_attn_func(*t, softmax_scale=scale, causal=True)
    torch.cuda.synchronize()
    return o.float().cpu().numpy()[0]  # [S, H, 128]


_POS = leanp.E4M3FN[1:127]


def _nearest_code(value):
    if value == 0.0:
        return 0
    return 1 + int(np.argmin(np.abs(np.log2(_POS) - np.log2(value))))


def _check(t, c, label):
    q, k, v = _inputs(t)
    out = _run(q, k, v, _scale_for(c))
    H = len(t)
    bad, n = [], 0
    for h in range(H):
        for i in range(S):
            s = np.array([t[h][j] if j <= i else -np.inf for j in range(S)])
            codes, ks, m = leanp.tile_codes_fp32(s, c)
            o = out[i, h]
            assert np.all(o[i + 1:] == 0.0), f"{label} h{h} row {i}: masked keys carry weight"
            r = int(np.argmax(s))  # a key at the row max: code 120 under exponent 8
            assert codes[r] == 120 and ks[r // 64] == 8
            for d in range(i + 1):
                kd = ks[d // 64]
                val = o[d] / o[r] * 256.0 * 2.0 ** (kd - 8)
                got = _nearest_code(val)
                n += 1
                if got != codes[d]:
                    bad.append((h, i, d, int(codes[d]), got))
    print(f"{label}: {n} codes compared, {len(bad)} differ {bad[:8]}", flush=True)
    sys.stdout.flush()
    assert not bad


def test_codes_on_a_fine_grid_over_twenty_binades():
    c = 2.0 ** -4  # x = c (s - m) binades: 16 score units per binade
    rng = np.random.default_rng(21)
    t = [
        [-2.25 * j for j in range(S)],  # 0 .. -18 binades, max at key 0
        [80.0 - 5.375 * j for j in range(64)] + [100.0 - 7.5 * j for j in range(64)],  # max moves to block 1
        [-3.0] * 40 + [64.0] + [-300.0 - j for j in range(23)] + [-250.0] * 50 + [-250.5] * 7 + [-251.0] * 7,
        list(np.round(rng.standard_normal(S) * 40.0 / LATTICE) * LATTICE),
    ]
    _check(t, c, "grid")


def test_codes_at_exact_ties_of_the_convert():
    """The bias of a block with reference max 0 and exponent k is
    B_k = fl32(C + 8k); a score 32 (n + 1/2 - B_k) makes the code argument
    exactly n + 1/2 (c = 2^-8, 8c = 2^-5): the convert must round to the even
    neighbour. Neighbours one lattice step away test the other side."""
    c = 2.0 ** -8
    f32 = lambda x: float(np.float32(x))  # noqa: E731
    Bk = lambda kk: f32(f32(leanp.LEANP_C) + 8.0 * kk)  # noqa: E731
    t0 = [0.0]
    for j in range(1, 64):
        n = 119 - 2 * ((j - 1) // 2) - (j % 3)
        tie = 32.0 * (n + 0.5 - Bk(8))
        t0.append(tie if j % 2 == 0 else tie + (LATTICE if j % 4 == 1 else -LATTICE))
    t0.append(-768.0)  # block 1 max: x = -3, exponent 11
    for j in range(65, 128):
        n = 118 - (j - 65) - (j % 2)
        tie = 32.0 * (n + 0.5 - Bk(11))
        t0.append(tie if j % 3 else tie - LATTICE)
    # the same ties relative to a reference max of 1000 (bias -31.25 + B_k)
    t1 = [1000.0] + [x + 1000.0 for x in t0[1:]]
    n_ties = sum(1 for x in t0[1:64] if (x / 32.0 + Bk(8)) % 1.0 == 0.5)
    assert n_ties >= 30
    _check([t0, t1], c, "ties")
