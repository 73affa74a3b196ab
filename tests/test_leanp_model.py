"""Pins of the FP8-softmax model (oracle/leanp.py) against the pages' printed
figures (tests/golden/page_figures.json), torch's float8 cast, closed forms
and the exact fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from oracle import leanp
from fp8_bf16_causal_amd import synth


def _rel_err_leanp(C, rounding="rne"):
    x = np.linspace(-6.0, 8.0, 200001)  # the e4m3 normal range after block scaling
    p = 2.0 ** x
    return np.abs(leanp.e4m3_value(leanp.leanp_code(x, C, rounding)) / p - 1.0)


def test_exact_rounding_matches_torch_cast():
    x = np.concatenate([np.linspace(0.0, 448.0, 100003), 2.0 ** np.linspace(-12, 8.8, 50001)])
    ours = leanp.e4m3_round_rne(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    assert np.array_equal(ours, ref)


def test_exact_rounding_error_is_the_pages_figure(golden):
    x = 2.0 ** np.linspace(-6.0, 8.0, 400001)
    err = np.abs(leanp.e4m3_value(leanp.e4m3_round_rne(x)) / x - 1.0).max()
    assert abs(err - 1.0 / 17.0) < 1e-4  # half a mantissa step at the bottom of a binade
    assert round(err * 100, 1) == round(golden["exact_rounding_max_rel_err"]["value"] * 100, 1)


def test_leanp_error_bound_and_constant(golden):
    bound = golden["leanp_max_rel_err"]["value"]
    err = _rel_err_leanp(leanp.LEANP_C).max()
    assert err <= bound
    assert err > golden["exact_rounding_max_rel_err"]["value"]  # an approximation, coarser than exact rounding
    # the naive constant 8 * exponent-bias = 56 misses the pages' bound: the constant is a real choice
    assert _rel_err_leanp(56.0).max() > bound
    # and the bound only holds in a narrow window around the chosen constant
    assert _rel_err_leanp(55.55).max() > bound and _rel_err_leanp(55.70).max() > bound


def test_leanp_ratio_range_and_subnormal_error():
    """The two facts the log-sum-exp bound of the FP8 path rests on: over the
    e4m3 normal range a Lean P code decodes to between 0.9273 and 1.0727 times
    its probability (so |ln ratio| <= 0.0755), and below it (probabilities
    under 2^-6 after block scaling, subnormal or zero codes) it is off by less
    than 0.0085 in absolute terms."""
    x = np.linspace(-6.0, 8.0, 400001)
    r = leanp.e4m3_value(leanp.leanp_code(x)) / 2.0 ** x
    assert 0.9273 <= r.min() and r.max() <= 1.0727
    assert max(-np.log(r.min()), np.log(r.max())) <= 0.0755
    xs = np.linspace(-40.0, -6.0, 400001)[:-1]
    d = np.abs(leanp.e4m3_value(leanp.leanp_code(xs)) - 2.0 ** xs)
    assert d.max() < 0.0085
    # exact rounding: at most half a subnormal step, 2^-10
    de = np.abs(leanp.e4m3_value(leanp.e4m3_round_rne(2.0 ** xs)) - 2.0 ** xs)
    assert de.max() <= 2.0 ** -10


def test_code_grows_by_eight_per_doubling(golden):
    step = golden["fp8_e4m3_code_step_per_doubling"]["value"]
    x = np.linspace(-5.0, 6.9, 1191)
    assert np.all(leanp.leanp_code(x + 1.0) - leanp.leanp_code(x) == step)
    n = np.arange(-6, 9)
    assert np.array_equal(leanp.leanp_code(n.astype(float)), 8 * n + 56)  # exact powers of two stay exact
    assert np.array_equal(leanp.e4m3_value(8 * n + 56), 2.0 ** n)


def test_leanp_code_monotone_and_saturating():
    x = np.linspace(-30.0, 9.0, 100001)
    c = leanp.leanp_code(x)
    assert np.all(np.diff(c) >= 0)
    assert c.min() == 0 and c.max() <= 126
    assert leanp.leanp_code(-np.inf) == 0 and leanp.leanp_code(np.nan) == 0


def test_block_shift_identity():
    """decode(code + 8k) = 2**k decode(code) for normal codes: shifting a code
    by 8k is the power-of-two block scale, which an E8M0 factor of 2**-k undoes
    exactly."""
    for code in range(8, 127):
        for k in range(0, (126 - code) // 8 + 1):
            assert leanp.e4m3_value(code + 8 * k) == 2.0 ** k * leanp.e4m3_value(code)


def test_block_exponent_reading():
    # the block max lands in (2**7, 2**8]: its code is at most 120, never NaN
    t = np.linspace(-100.0, 0.0, 10001)
    k = leanp.block_exponent(t)
    assert np.all(t + k > 7.0) and np.all(t + k <= 8.0)
    assert np.all(leanp.leanp_code(t + k) <= 120)
    assert leanp.block_exponent(-np.inf) == 127 and leanp.block_exponent(-500.0) == 127


def _dequant(inp):
    dt = oracle.BF16 if inp.dtype == "bf16" else oracle.FP8_E4M3
    dq, dk, dv = inp.descale
    return (oracle.dequantize(synth.raw_codes(inp.q), dt, dq), oracle.dequantize(synth.raw_codes(inp.k), dt, dk),
            oracle.dequantize(synth.raw_codes(inp.v), dt, 1.0), dv)


def _exact(inp, rows):
    dq, dk, dv = inp.descale
    return oracle.attention(synth.raw_codes(inp.q), synth.raw_codes(inp.k), synth.raw_codes(inp.v),
                            oracle.FP8_E4M3, inp.scale, dq, dk, dv, rows=np.array(rows))


def test_rounded_sum_normalisation_gives_weights_summing_to_one():
    """V = 1 everywhere: dividing by the sum of the rounded probabilities
    returns exactly 1 (up to fp64 rounding), whatever the rounding did."""
    inp = synth.make_inputs(B=1, S=300, Hq=1, Hkv=1, Dqk=128, Dv=8, dtype="fp8", seed=21)
    qd, kd, _, _ = _dequant(inp)
    vd = np.ones((1, 300, 1, 8))
    out = leanp.leanp_attention(qd, kd, vd, inp.scale)
    assert np.max(np.abs(out - 1.0)) <= 1e-14


def _err(a, ref, vmax):
    rel_rms = np.sqrt(np.sum((a - ref) ** 2) / np.sum(ref ** 2))
    return rel_rms, np.max(np.abs(a - ref)) / vmax


def _rows(S, H, n, seed):
    rng = np.random.default_rng(seed)
    rows = [(0, h, i) for h in range(H) for i in (0, 1, 63, 64, 127, 128, S - 1)]
    rows += [(0, int(rng.integers(H)), int(rng.integers(S))) for _ in range(n)]
    return rows


def test_model_within_fp8_tolerance_of_exact_attention():
    inp = synth.make_inputs(B=1, S=1024, Hq=2, Hkv=2, Dqk=128, Dv=128, dtype="fp8", seed=3)
    qd, kd, vd, dv = _dequant(inp)
    rows = _rows(1024, 2, 120, 0)
    ref = _exact(inp, rows)
    vmax = np.abs(vd).max() * dv
    lean = leanp.leanp_attention(qd, kd, vd, inp.scale, dv, rows=rows)
    exact_p = leanp.leanp_attention(qd, kd, vd, inp.scale, dv, rows=rows, exact_p=True)
    rr_lean, ma_lean = _err(lean, ref, vmax)
    rr_exact, _ = _err(exact_p, ref, vmax)
    assert rr_lean <= 4e-2 and ma_lean <= 0.1  # the FP8 parity bar
    assert rr_exact < rr_lean  # exact rounding is the finer of the two
    assert rr_lean > 5e-3  # the approximation is visible: the model is not the exact oracle


def test_block_scaling_matters_on_peaked_inputs():
    """Without the per-64-key power of two (plain probabilities in [0, 1]),
    blocks far below the row max fall into e4m3 subnormals or zero and the
    output error grows."""
    inp = synth.make_inputs(B=1, S=2048, Hq=2, Hkv=1, Dqk=128, Dv=128, dtype="fp8", seed=2, structure="peaked")
    qd, kd, vd, dv = _dequant(inp)
    rows = _rows(2048, 2, 100, 1)
    ref = _exact(inp, rows)
    vmax = np.abs(vd).max() * dv
    with_bs = _err(leanp.leanp_attention(qd, kd, vd, inp.scale, dv, rows=rows), ref, vmax)
    without = _err(leanp.leanp_attention(qd, kd, vd, inp.scale, dv, rows=rows, block_scale=False), ref, vmax)
    assert with_bs[0] <= 4e-2 and with_bs[1] <= 0.1
    assert without[0] > 1.5 * with_bs[0] and without[1] > 1.5 * with_bs[1]


def test_roofline_figures(golden):
    # one 32-query x 128-key FP8 tile at head dim 128: 2*32*128*(128+128) flop at
    # 2048 FP8 flop per clock per SIMD (datasheet dense peak / (256 CU * 4 SIMD * 2.4 GHz))
    flop = 2 * 32 * 128 * (128 + 128)
    per_clk = 5.0e15 / (256 * 4 * 2.4e9)
    assert abs(per_clk - 2048) / 2048 < 0.02
    assert flop / 2048 == golden["mfma_cycles_32q_128k_hd128"]["value"]
    # a 16-wide ones operand for the row sum costs 16 / (Dqk + Dv) extra matrix work
    assert round(16 / (128 + 128), 2) == golden["rowsum_extra_matrix_work"]["value"]
    assert golden["block_keys"]["value"] == leanp.BLOCK_KEYS


def test_lazy_reference_max_keeps_the_result():
    """Moving the reference max only on rises of more than 8 binades changes
    which rounding each code sees, not the attention being approximated: both
    variants meet the FP8 bar against exact attention, codes stay <= 120."""
    inp = synth.make_inputs(B=1, S=900, Hq=2, Hkv=1, Dqk=128, Dv=128, dtype="fp8", seed=17, structure="peaked")
    qd, kd, vd, dv = _dequant(inp)
    rows = _rows(900, 2, 80, 3)
    ref = _exact(inp, rows)
    vmax = np.abs(vd).max() * dv
    eager = _err(leanp.leanp_attention(qd, kd, vd, inp.scale, dv, rows=rows), ref, vmax)
    lazy = _err(leanp.leanp_attention(qd, kd, vd, inp.scale, dv, rows=rows, lazy_log2=8.0), ref, vmax)
    assert eager[0] <= 4e-2 and lazy[0] <= 4e-2 and lazy[1] <= 0.1
    assert abs(lazy[0] - eager[0]) < 0.5 * eager[0]
    # with a stale reference the block max sits up to 8 binades above it; the
    # block exponent is then >= 0 and the code still <= 120
    t = np.linspace(0.0, 8.0, 1001)
    k = leanp.block_exponent(t)
    assert np.all(k >= 0) and np.all(leanp.leanp_code(t + k) <= 120)


# ---------------------------------------------------------------- fp32 decisions

def test_round_f32_matches_numpy_single_rounding():
    """round_f32 of a double equals numpy's float64 -> float32 cast (one
    correctly rounded step), over normal and subnormal float32 ranges."""
    from fractions import Fraction

    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 38, 3000),
                        rng.standard_normal(500) * 1e-42, [0.0, 1.0, -2.5, 3.4e38, 1.17549435e-38]])
    for v in x:
        assert leanp.round_f32(Fraction(float(v))) == float(np.float32(v)), v


def test_fma_f32_single_rounding():
    """fma_f32 rounds a*b + c once: where a*b + c is exact in float64 (operands
    of close magnitude) it equals the float32 cast of that double; ties go to
    even; and it differs from a two-step (rounded product) evaluation where
    the product's low bits decide."""
    from fractions import Fraction

    rng = np.random.default_rng(6)
    a = rng.standard_normal(2000).astype(np.float32)
    b = rng.standard_normal(2000).astype(np.float32)
    c = rng.standard_normal(2000).astype(np.float32)
    n_exact = 0
    for x, y, z in zip(a, b, c):
        d = float(x) * float(y) + float(z)
        if Fraction(d) == Fraction(float(x)) * Fraction(float(y)) + Fraction(float(z)):
            n_exact += 1
            assert leanp.fma_f32(float(x), float(y), float(z)) == float(np.float32(d))
    assert n_exact > 1500
    assert leanp.fma_f32(1.0, 1.0, 2.0 ** -24) == 1.0  # tie, even
    assert leanp.fma_f32(1.0, 1.0, 3 * 2.0 ** -24) == 1.0 + 2.0 ** -22  # tie, even (up)
    x = 1.0 + 2.0 ** -12
    # (1 + 2^-12)^2 - 1 = 2^-11 + 2^-24 exactly; a rounded product would lose the 2^-24
    assert leanp.fma_f32(x, x, -1.0) == 2.0 ** -11 + 2.0 ** -24
    assert float(np.float32(np.float32(x) * np.float32(x)) - np.float32(1.0)) == 2.0 ** -11
    assert leanp.fma_f32(-np.inf, 0.5, 3.0) == -np.inf


def test_tile_codes_fp32_agree_with_the_model_away_from_ties():
    """The fp32 code decisions of one tile equal the fp64 model's codes
    (leanp_code(x + k) with the same reference max and block exponents)
    wherever 8(x + k) + C is not within 1e-3 of a half-integer; masked keys
    give code 0 and a fully masked block exponent 127."""
    rng = np.random.default_rng(8)
    c = float(np.float32(0.1275))
    for trial in range(40):
        s = (rng.standard_normal(128) * rng.uniform(2, 60)).astype(np.float32).astype(np.float64)
        nvis = int(rng.integers(1, 129))
        s[nvis:] = -np.inf
        codes, ks, m = leanp.tile_codes_fp32(s, c)
        assert codes[nvis:].sum() == 0
        if nvis <= 64:
            assert ks[1] == 127
        for blk in range(2):
            sl = slice(64 * blk, 64 * blk + 64)
            vis = np.isfinite(s[sl])
            if not vis.any():
                continue
            x = (s[sl][vis] - m) * c
            assert ks[blk] == int(leanp.block_exponent(np.max(x)))
            y = 8.0 * (x + ks[blk]) + leanp.LEANP_C
            far = np.abs(y - np.floor(y) - 0.5) > 1e-3
            assert np.array_equal(codes[sl][vis][far], leanp.leanp_code(x + ks[blk])[far])
