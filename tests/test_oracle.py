"""Pins of the fp64 CPU oracle against things other than itself.

Every check here is independent of the oracle's own code path: a library
routine (torch's casts, torch's scaled_dot_product_attention), a brute-force
materialised computation written differently (log-sum-exp over a full masked
matrix, math.fsum), closed forms, or invariants of causal softmax attention.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from fp8_bf16_causal_amd import synth


def _decoded(inp):
    """fp64 tensors of the inputs, decoded by torch's own casts (independent of
    the oracle's decoders), times their dequantisation factors."""
    dq, dk, dv = inp.descale
    return (inp.q.to(torch.float64) * dq, inp.k.to(torch.float64) * dk, inp.v.to(torch.float64) * dv)


def _oracle(inp, rows=None, nthreads=2):
    dt = oracle.BF16 if inp.dtype == "bf16" else oracle.FP8_E4M3
    dq, dk, dv = inp.descale
    return oracle.attention(synth.raw_codes(inp.q), synth.raw_codes(inp.k), synth.raw_codes(inp.v), dt,
                            inp.scale, dq, dk, dv, rows=rows, nthreads=nthreads)


# ---------------------------------------------------------------- decoders

def test_e4m3fn_decoder_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.nanmax(ours) == 448.0 and ours[0x7F] != ours[0x7F]  # 0x7F is NaN, 448 is the largest value


def test_bf16_decoder_matches_torch_on_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.dequantize(codes, oracle.BF16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


# ---------------------------------------------------------------- brute force

def _brute_force(qd, kd, vd, scale):
    """Materialised causal attention via log-sum-exp over the full masked S x S
    score matrix, with math.fsum; written independently of the oracle."""
    B, S, Hq, _ = qd.shape
    Hkv, Dv = kd.shape[2], vd.shape[3]
    rep = Hq // Hkv
    out = np.zeros((B, S, Hq, Dv))
    for b in range(B):
        for h in range(Hq):
            g = h // rep
            scores = [[-math.inf] * S for _ in range(S)]
            for i in range(S):
                for j in range(S):
                    if j <= i:
                        scores[i][j] = scale * math.fsum(qd[b, i, h, d] * kd[b, j, g, d] for d in range(qd.shape[3]))
            for i in range(S):
                top = max(scores[i])
                lse = top + math.log(math.fsum(math.exp(s - top) for s in scores[i] if s != -math.inf))
                for d in range(Dv):
                    out[b, i, h, d] = math.fsum(math.exp(scores[i][j] - lse) * vd[b, j, g, d] for j in range(i + 1))
    return out


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("S,Hq,Hkv,D", [(1, 1, 1, 4), (7, 2, 1, 8), (13, 2, 2, 5), (16, 4, 2, 8)])
def test_oracle_matches_brute_force(dtype, S, Hq, Hkv, D):
    inp = synth.make_inputs(B=2, S=S, Hq=Hq, Hkv=Hkv, Dqk=D, Dv=D + 1, dtype=dtype, seed=S * 7 + Hq)
    qd, kd, vd = (t.numpy() for t in _decoded(inp))
    ref = _brute_force(qd, kd, vd, inp.scale)
    got = _oracle(inp)
    assert np.max(np.abs(got - ref)) <= 1e-13 * max(1.0, np.max(np.abs(ref)))


# ---------------------------------------------------------------- library routine

@pytest.mark.parametrize("dtype,B,S,Hq,Hkv,Dqk,Dv", [
    ("bf16", 1, 200, 4, 4, 128, 128),
    ("fp8", 2, 130, 4, 2, 128, 128),
    ("fp8", 1, 97, 2, 1, 192, 128),
    ("bf16", 1, 64, 3, 1, 64, 32),
])
def test_oracle_matches_torch_sdpa_float64(dtype, B, S, Hq, Hkv, Dqk, Dv):
    inp = synth.make_inputs(B=B, S=S, Hq=Hq, Hkv=Hkv, Dqk=Dqk, Dv=Dv, dtype=dtype, seed=11 + S)
    qd, kd, vd = _decoded(inp)
    rep = Hq // Hkv
    q = qd.permute(0, 2, 1, 3)
    k = kd.repeat_interleave(rep, dim=2).permute(0, 2, 1, 3)
    v = vd.repeat_interleave(rep, dim=2).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=inp.scale)
    ref = ref.permute(0, 2, 1, 3).numpy()
    got = _oracle(inp)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_oracle_matches_sdpa_on_peaked_structure():
    inp = synth.make_inputs(B=1, S=160, Hq=4, Hkv=1, Dqk=128, Dv=128, dtype="fp8", seed=2, structure="peaked")
    qd, kd, vd = _decoded(inp)
    q = qd.permute(0, 2, 1, 3)
    k = kd.repeat_interleave(4, dim=2).permute(0, 2, 1, 3)
    v = vd.repeat_interleave(4, dim=2).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=inp.scale)
    got = _oracle(inp)
    assert np.max(np.abs(got - ref.permute(0, 2, 1, 3).numpy())) <= 1e-11


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_row_zero_is_v0(dtype):
    inp = synth.make_inputs(B=2, S=40, Hq=4, Hkv=2, Dqk=128, Dv=128, dtype=dtype, seed=3)
    got = _oracle(inp)
    _, _, vd = _decoded(inp)
    for h in range(4):
        assert np.array_equal(got[:, 0, h, :], vd[:, 0, h // 2, :].numpy())


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_equal_scores_give_prefix_mean(dtype):
    """scale = 0 makes every visible score equal: row i is the mean of V[0..i]."""
    inp = synth.make_inputs(B=1, S=75, Hq=2, Hkv=1, Dqk=128, Dv=128, dtype=dtype, seed=4, scale=0.0)
    got = _oracle(inp)
    _, _, vd = _decoded(inp)
    v = vd[0, :, 0, :].numpy()
    prefix_mean = np.cumsum(v, axis=0) / np.arange(1, 76)[:, None]
    for h in range(2):
        assert np.max(np.abs(got[0, :, h, :] - prefix_mean)) <= 1e-13


def test_zero_queries_give_prefix_mean():
    inp = synth.make_inputs(B=1, S=33, Hq=1, Hkv=1, Dqk=128, Dv=64, dtype="bf16", seed=5)
    inp.q.zero_()
    got = _oracle(inp)
    v = _decoded(inp)[2][0, :, 0, :].numpy()
    assert np.max(np.abs(got[0, :, 0, :] - np.cumsum(v, axis=0) / np.arange(1, 34)[:, None])) <= 1e-13


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_probability_rows_sum_to_one_and_are_causal(dtype):
    inp = synth.make_inputs(B=1, S=24, Hq=2, Hkv=1, Dqk=16, Dv=16, dtype=dtype, seed=6)
    dt = oracle.BF16 if dtype == "bf16" else oracle.FP8_E4M3
    dq, dk, _ = inp.descale
    P = oracle.probs(synth.raw_codes(inp.q), synth.raw_codes(inp.k), dt, inp.scale, 0, 1, dq, dk)
    assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= 1e-14
    lower = np.tril(np.ones_like(P, dtype=bool))
    assert np.all(P[~lower] == 0.0) and np.all(P[lower] > 0.0)


def _brute_force_probs(qd, kd, b, h, g, scale):
    """One head's causal softmax matrix, materialised with math.fsum and a
    log-sum-exp per row (independent of the oracle's code): qd, kd already
    carry their dequantisation factors; key head g."""
    S, D = qd.shape[1], qd.shape[3]
    P = np.zeros((S, S))
    for i in range(S):
        s = [scale * math.fsum(qd[b, i, h, d] * kd[b, j, g, d] for d in range(D)) for j in range(i + 1)]
        top = max(s)
        lse = top + math.log(math.fsum(math.exp(x - top) for x in s))
        for j in range(i + 1):
            P[i, j] = math.exp(s[j] - lse)
    return P


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_probs_match_brute_force_and_reproduce_the_output(dtype):
    """oracle.probs on GQA inputs (4 query heads over 2 KV heads, head 3 reads
    KV head 1), a second batch entry, a softmax scale other than 1/sqrt(D) and
    per-tensor factors dq, dk far from 1: equal to a brute-force softmax within
    1e-14, and P @ V * dv equal to oracle.attention's rows within 1e-13. The
    brute force with the KV head, the scale or a descale changed lands far
    from it, so a slip of any of them in oracle.probs would fail."""
    B, S, Hq, Hkv, D = 2, 11, 4, 2, 8
    inp = synth.make_inputs(B=B, S=S, Hq=Hq, Hkv=Hkv, Dqk=D, Dv=D + 3, dtype=dtype, seed=91, scale=0.83)
    if dtype == "bf16":
        dq, dk, dv = 1.0, 1.0, 1.0
    else:
        dq, dk, dv = 0.011, 0.0063, 1.7  # dequantised values of order one, factors far from 1
        inp = synth.AttnInputs(inp.q, inp.k, inp.v, "fp8", inp.scale, (dq, dk, dv))
    dt = oracle.BF16 if dtype == "bf16" else oracle.FP8_E4M3
    qd, kd, vd = (t.numpy() for t in _decoded(inp))
    b, h, g = 1, 3, 1
    P = oracle.probs(synth.raw_codes(inp.q), synth.raw_codes(inp.k), dt, inp.scale, b, h, dq, dk)
    ref = _brute_force_probs(qd, kd, b, h, g, inp.scale)
    assert np.max(np.abs(P - ref)) <= 1e-14
    # the weights are the ones the oracle's output applies
    rows = np.array([[b, h, i] for i in range(S)])
    out = _oracle(inp, rows=rows)
    assert np.max(np.abs(P @ vd[b, :, g, :] - out)) <= 1e-13
    # discrimination: each plausible slip moves P by far more than the tolerance
    for wrong in (_brute_force_probs(qd, kd, b, h, 0, inp.scale),          # KV head h instead of h / (Hq / Hkv)
                  _brute_force_probs(qd, kd, b, h, g, inp.scale * 1.25),   # another scale
                  _brute_force_probs(qd, kd / (dk if dtype == "fp8" else 2.0), b, h, g, inp.scale)):  # dk dropped
        assert np.max(np.abs(P - wrong)) > 1e-3


def test_score_shift_invariance():
    """Adding one vector u to every key shifts each row's scores by a constant
    (scale * q_i . u), which softmax ignores. Integer-valued BF16 inputs keep
    K + u exact."""
    g = torch.Generator().manual_seed(7)
    B, S, H, D = 1, 50, 2, 16
    q = torch.randint(-3, 4, (B, S, H, D), generator=g).to(torch.bfloat16)
    k = torch.randint(-3, 4, (B, S, H, D), generator=g).to(torch.bfloat16)
    v = torch.randn((B, S, H, D), generator=g).to(torch.bfloat16)
    u = torch.randint(-2, 3, (D,), generator=g).to(torch.bfloat16)
    a = synth.AttnInputs(q, k, v, "bf16", 0.1, (1.0, 1.0, 1.0))
    b = synth.AttnInputs(q, (k.float() + u.float()).to(torch.bfloat16), v, "bf16", 0.1, (1.0, 1.0, 1.0))
    assert np.max(np.abs(_oracle(a) - _oracle(b))) <= 1e-12


def test_gqa_equals_mha_with_repeated_kv():
    inp = synth.make_inputs(B=2, S=70, Hq=6, Hkv=2, Dqk=32, Dv=48, dtype="fp8", seed=8)
    rep = synth.AttnInputs(inp.q, inp.k.repeat_interleave(3, dim=2), inp.v.repeat_interleave(3, dim=2), "fp8",
                           inp.scale, inp.descale)
    assert np.array_equal(_oracle(inp), _oracle(rep))


def test_v_column_permutation_permutes_output():
    inp = synth.make_inputs(B=1, S=45, Hq=2, Hkv=2, Dqk=32, Dv=40, dtype="bf16", seed=9)
    perm = torch.randperm(40, generator=torch.Generator().manual_seed(1))
    per = synth.AttnInputs(inp.q, inp.k, inp.v[..., perm].contiguous(), "bf16", inp.scale, inp.descale)
    assert np.array_equal(_oracle(inp)[..., perm.numpy()], _oracle(per))


def test_descale_folding_and_output_linearity():
    inp = synth.make_inputs(B=1, S=60, Hq=2, Hkv=1, Dqk=64, Dv=64, dtype="fp8", seed=10)
    q, k, v = (synth.raw_codes(t) for t in (inp.q, inp.k, inp.v))
    a = oracle.attention(q, k, v, oracle.FP8_E4M3, 0.2, dq=2.0, dk=0.5, dv=1.0)
    b = oracle.attention(q, k, v, oracle.FP8_E4M3, 0.2, dq=1.0, dk=1.0, dv=1.0)
    c = oracle.attention(q, k, v, oracle.FP8_E4M3, 0.2, dq=1.0, dk=1.0, dv=0.25)
    assert np.max(np.abs(a - b)) <= 1e-14
    assert np.array_equal(c, b * 0.25)


def test_row_subset_matches_full():
    inp = synth.make_inputs(B=2, S=90, Hq=4, Hkv=2, Dqk=128, Dv=128, dtype="fp8", seed=12)
    full = _oracle(inp)
    rows = np.array([[0, 0, 0], [1, 3, 89], [0, 2, 45], [1, 1, 1], [1, 0, 64]])
    sub = _oracle(inp, rows=rows)
    for n, (b, h, i) in enumerate(rows):
        assert np.array_equal(sub[n], full[b, i, h])


def test_oracle_rejects_bad_arguments():
    inp = synth.make_inputs(B=1, S=8, Hq=3, Hkv=3, Dqk=8, Dv=8, dtype="bf16", seed=0)
    q, k, v = (synth.raw_codes(t) for t in (inp.q, inp.k, inp.v))
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, oracle.BF16, 1.0, rows=np.array([[0, 3, 0]]))  # head out of range
    with pytest.raises(ValueError):
        oracle.attention(q, k[:, :, :2], v[:, :, :2], oracle.BF16, 1.0)  # Hq % Hkv != 0
    with pytest.raises(TypeError):
        oracle.attention(q.astype(np.uint8), k, v, oracle.BF16, 1.0)


# ---------------------------------------------------------------- log-sum-exp (per-row LSE output)

def _oracle_lse(inp, rows=None, nthreads=2):
    dt = oracle.BF16 if inp.dtype == "bf16" else oracle.FP8_E4M3
    dq, dk, dv = inp.descale
    return oracle.attention(synth.raw_codes(inp.q), synth.raw_codes(inp.k), synth.raw_codes(inp.v), dt,
                            inp.scale, dq, dk, dv, rows=rows, nthreads=nthreads, return_lse=True)


def _brute_force_lse(qd, kd, scale):
    """ln sum_{j<=i} exp(scale <q_i, k_j>) per (b, h, i), materialised with
    math.fsum and written independently of the oracle."""
    B, S, Hq, D = qd.shape
    rep = Hq // kd.shape[2]
    lse = np.zeros((B, Hq, S))
    for b in range(B):
        for h in range(Hq):
            for i in range(S):
                z = [scale * math.fsum(qd[b, i, h, d] * kd[b, j, h // rep, d] for d in range(D)) for j in range(i + 1)]
                top = max(z)
                lse[b, h, i] = top + math.log(math.fsum(math.exp(x - top) for x in z))
    return lse


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("S,Hq,Hkv,D", [(1, 1, 1, 4), (9, 2, 1, 8), (16, 4, 2, 8)])
def test_lse_matches_brute_force(dtype, S, Hq, Hkv, D):
    inp = synth.make_inputs(B=2, S=S, Hq=Hq, Hkv=Hkv, Dqk=D, Dv=D, dtype=dtype, seed=S * 11 + Hq)
    qd, kd, _ = (t.numpy() for t in _decoded(inp))
    out, lse = _oracle_lse(inp)
    assert lse.shape == (2, Hq, S)
    assert np.max(np.abs(lse - _brute_force_lse(qd, kd, inp.scale))) <= 1e-12
    assert np.array_equal(out, _oracle(inp))  # the output does not change with the extra result


def test_lse_closed_forms():
    """Equal scores (Q = 0): every visible key has weight 1, so lse_i = ln(i+1).
    Row 0 sees only key 0: lse_0 = scale <q_0, k_0>."""
    inp = synth.make_inputs(B=1, S=40, Hq=2, Hkv=1, Dqk=64, Dv=64, dtype="bf16", seed=12)
    q0 = inp.q.clone()
    inp.q.zero_()
    _, lse = _oracle_lse(inp)
    assert np.max(np.abs(lse[0] - np.log(np.arange(1, 41))[None, :])) <= 1e-13
    inp.q.copy_(q0)
    _, lse = _oracle_lse(inp)
    qd, kd, _ = (t.numpy() for t in _decoded(inp))
    for h in range(2):
        z00 = inp.scale * math.fsum(qd[0, 0, h, d] * kd[0, 0, 0, d] for d in range(64))
        assert abs(lse[0, h, 0] - z00) <= 1e-13 * max(1.0, abs(z00))


def test_lse_shifts_with_the_scores():
    """Adding u to every key adds scale <q_i, u> to every score of row i, and
    so to its log-sum-exp (integer-valued BF16 inputs keep K + u exact)."""
    g = torch.Generator().manual_seed(13)
    B, S, H, D = 1, 30, 2, 16
    q = torch.randint(-3, 4, (B, S, H, D), generator=g).to(torch.bfloat16)
    k = torch.randint(-3, 4, (B, S, H, D), generator=g).to(torch.bfloat16)
    v = torch.randn((B, S, H, D), generator=g).to(torch.bfloat16)
    u = torch.randint(-2, 3, (D,), generator=g).to(torch.bfloat16)
    a = synth.AttnInputs(q, k, v, "bf16", 0.1, (1.0, 1.0, 1.0))
    b = synth.AttnInputs(q, (k.float() + u.float()).to(torch.bfloat16), v, "bf16", 0.1, (1.0, 1.0, 1.0))
    shift = 0.1 * (q.double() @ u.double())  # [B, S, H]
    _, la = _oracle_lse(a)
    _, lb = _oracle_lse(b)
    assert np.max(np.abs(lb - la - shift.permute(0, 2, 1).numpy())) <= 1e-12


def test_lse_row_subset_matches_full():
    inp = synth.make_inputs(B=2, S=37, Hq=4, Hkv=2, Dqk=16, Dv=16, dtype="fp8", seed=14)
    _, full = _oracle_lse(inp)
    rows = np.array([(1, 3, 36), (0, 0, 0), (1, 1, 17), (0, 2, 5)], dtype=np.int64)
    _, sub = _oracle_lse(inp, rows=rows)
    assert np.array_equal(sub, np.array([full[b, h, i] for b, h, i in rows]))


# ---------------------------------------------------------------- queries after a key prefix (Sq < Sk)

def _prefix_inputs(dtype, B, Sq, Sk, Hq, Hkv, D, seed):
    """Queries of the last Sq positions over Sk keys: the key side of a full
    Sk-long input and the last Sq rows of its queries."""
    full = synth.make_inputs(B=B, S=Sk, Hq=Hq, Hkv=Hkv, Dqk=D, Dv=D + 2, dtype=dtype, seed=seed)
    q = full.q[:, Sk - Sq:].contiguous()
    return full, synth.AttnInputs(q, full.k, full.v, full.dtype, full.scale, full.descale)


def _brute_force_prefix(qd, kd, vd, scale):
    """Materialised attention of Sq queries over Sk keys, query i seeing keys
    j <= i + Sk - Sq, with math.fsum; returns (out, lse)."""
    B, Sq, Hq, D = qd.shape
    Sk, Hkv, Dv = kd.shape[1], kd.shape[2], vd.shape[3]
    rep, off = Hq // Hkv, Sk - Sq
    out, lse = np.zeros((B, Sq, Hq, Dv)), np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            for i in range(Sq):
                z = [scale * math.fsum(qd[b, i, h, d] * kd[b, j, h // rep, d] for d in range(D)) for j in range(i + off + 1)]
                top = max(z)
                ls = top + math.log(math.fsum(math.exp(x - top) for x in z))
                lse[b, h, i] = ls
                for d in range(Dv):
                    out[b, i, h, d] = math.fsum(math.exp(z[j] - ls) * vd[b, j, h // rep, d] for j in range(len(z)))
    return out, lse


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("Sq,Sk,Hq,Hkv", [(1, 9, 2, 1), (5, 12, 2, 2), (7, 7, 4, 2), (3, 20, 4, 1)])
def test_prefix_matches_brute_force(dtype, Sq, Sk, Hq, Hkv):
    _, inp = _prefix_inputs(dtype, 2, Sq, Sk, Hq, Hkv, 6, seed=Sq * 13 + Sk)
    qd, kd, vd = (t.numpy() for t in _decoded(inp))
    ref_o, ref_l = _brute_force_prefix(qd, kd, vd, inp.scale)
    got_o, got_l = _oracle_lse(inp)
    assert np.max(np.abs(got_o - ref_o)) <= 1e-13 * max(1.0, np.max(np.abs(ref_o)))
    assert np.max(np.abs(got_l - ref_l)) <= 1e-12


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_prefix_matches_sdpa_with_bottom_right_mask(dtype):
    _, inp = _prefix_inputs(dtype, 1, 40, 100, 4, 2, 32, seed=77)
    qd, kd, vd = _decoded(inp)
    mask = torch.ones(40, 100, dtype=torch.bool).tril(diagonal=60)  # key j visible to query i iff j <= i + 60
    rep = 2
    ref = torch.nn.functional.scaled_dot_product_attention(
        qd.permute(0, 2, 1, 3), kd.repeat_interleave(rep, dim=2).permute(0, 2, 1, 3),
        vd.repeat_interleave(rep, dim=2).permute(0, 2, 1, 3), attn_mask=mask, scale=inp.scale).permute(0, 2, 1, 3)
    assert np.max(np.abs(_oracle(inp) - ref.numpy())) <= 1e-12


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_prefix_equals_the_suffix_of_full_attention(dtype):
    """Queries after a key prefix give the last rows of full causal attention
    over the whole sequence (output and log-sum-exp)."""
    full, inp = _prefix_inputs(dtype, 2, 45, 130, 4, 2, 16, seed=78)
    fo, fl = _oracle_lse(full)
    po, pl = _oracle_lse(inp)
    assert np.array_equal(po, fo[:, 130 - 45:])
    assert np.array_equal(pl, fl[:, :, 130 - 45:])


def test_prefix_rejects_fewer_keys_than_queries():
    full = synth.make_inputs(B=1, S=8, Hq=1, Hkv=1, Dqk=8, Dv=8, dtype="bf16", seed=1)
    with pytest.raises(ValueError):
        oracle.attention(synth.raw_codes(full.q), synth.raw_codes(full.k[:, :5].contiguous()),
                         synth.raw_codes(full.v[:, :5].contiguous()), oracle.BF16, 0.1)
