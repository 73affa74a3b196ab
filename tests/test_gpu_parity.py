"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle.

Bars (element by element, on the same seeded inputs):
  BF16: relative RMS error <= 1e-2 and max abs error <= 3e-2;
  FP8:  relative RMS error <= 4e-2 and max abs error <= 0.1 * max|V * dv|.
Small shapes are compared over the whole output; the full benchmark shapes
(in the launch configuration the benchmark times) on sampled rows that the
oracle computes one by one.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import leanp
from fp8_bf16_causal_amd import synth

pytestmark = pytest.mark.gpu

BF16_TOL = (1e-2, 3e-2)
FP8_TOL = (4e-2, 0.1)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_bf16_causal_amd._lib as L
    L.load()  # fails loudly if the HIP library is missing
    torch.cuda.set_device(0)


def run_gpu(inp, out=None, stream=None):
    import fp8_bf16_causal_amd as fbc
    dq, dk, dv = inp.descale
    dev = torch.device("cuda", 0)
    q, k, v = (t if t.is_cuda else t.to(dev) for t in (inp.q, inp.k, inp.v))
    if stream is not None:
        with torch.cuda.stream(stream):
            o = fbc.flash_attn_func(q, k, v, inp.scale, causal=True, descale_q=dq, descale_k=dk, descale_v=dv, out=out)
        stream.synchronize()
    else:
        o = fbc.flash_attn_func(q, k, v, inp.scale, causal=True, descale_q=dq, descale_k=dk, descale_v=dv, out=out)
        torch.cuda.synchronize()
    return o


def oracle_out(inp, rows=None):
    dq, dk, dv = inp.descale
    dt = oracle.BF16 if inp.dtype == "bf16" else oracle.FP8_E4M3
    return oracle.attention(synth.raw_codes(inp.q), synth.raw_codes(inp.k), synth.raw_codes(inp.v), dt, inp.scale,
                            dq, dk, dv, rows=rows)


def vmax(inp):
    dt = oracle.BF16 if inp.dtype == "bf16" else oracle.FP8_E4M3
    return float(np.max(np.abs(oracle.dequantize(synth.raw_codes(inp.v), dt, inp.descale[2]))))


def check(inp, got, ref, label):
    got = got.astype(np.float64)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    err = got - ref
    rel_rms = math.sqrt(float(np.sum(err ** 2)) / max(float(np.sum(ref ** 2)), 1e-300))
    maxabs = float(np.max(np.abs(err)))
    if inp.dtype == "bf16":
        lim_rr, lim_ma = BF16_TOL
    else:
        lim_rr, lim_ma = FP8_TOL[0], FP8_TOL[1] * vmax(inp)
    _say(f"{label}: rel_rms={rel_rms:.3e} (<= {lim_rr:g}) maxabs={maxabs:.3e} (<= {lim_ma:.3g})")
    assert rel_rms <= lim_rr and maxabs <= lim_ma, label
    return rel_rms, maxabs


def full_check(inp, label):
    _say(f"case {label} shape={inp.shape} dtype={inp.dtype}")
    out = run_gpu(inp).float().cpu().numpy()
    return check(inp, out, oracle_out(inp), label)


# ------------------------------------------------------------------ small, whole tensor

def test_bf16_small_config_whole_tensor():
    full_check(synth.make_config("bf16_mha_s512"), "bf16_mha_s512")


@pytest.mark.parametrize("structure", ["gaussian", "peaked"])
def test_fp8_small_whole_tensor(structure):
    inp = synth.make_inputs(B=1, S=640, Hq=4, Hkv=2, Dqk=128, Dv=128, dtype="fp8", seed=31, structure=structure)
    full_check(inp, f"fp8 S640 {structure}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("S", [1, 2, 7, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300, 1000])
def test_edge_lengths(dtype, S):
    inp = synth.make_inputs(B=2, S=S, Hq=4, Hkv=2, Dqk=128, Dv=128, dtype=dtype, seed=100 + S)
    full_check(inp, f"{dtype} B2 Hq4 Hkv2 S{S}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (8, 1), (8, 8), (6, 3)])
def test_head_layouts(dtype, Hq, Hkv):
    inp = synth.make_inputs(B=1, S=333, Hq=Hq, Hkv=Hkv, Dqk=128, Dv=128, dtype=dtype, seed=Hq * 10 + Hkv)
    full_check(inp, f"{dtype} Hq{Hq} Hkv{Hkv}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("S", [100, 517])
def test_head_dim_192(dtype, S):
    inp = synth.make_inputs(B=1, S=S, Hq=4, Hkv=4, Dqk=192, Dv=128, dtype=dtype, seed=5 + S)
    full_check(inp, f"{dtype} Dqk192 S{S}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("Dqk", [128, 192])
def test_batched_gqa_ragged(dtype, Dqk):
    """Several batch entries, GQA 6/2 and a length that is not a multiple of
    the 256-row query block or the 128-key tile, at both head dims."""
    inp = synth.make_inputs(B=3, S=389, Hq=6, Hkv=2, Dqk=Dqk, Dv=128, dtype=dtype, seed=31 + Dqk)
    full_check(inp, f"{dtype} B3 Hq6 Hkv2 S389 Dqk{Dqk}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("scale", [0.02, 0.3])
def test_non_default_scale(dtype, scale):
    """The softmax scale is folded into the base-2 score scale: a small one
    (nearly flat rows) and a large one (peaked rows, more rescales)."""
    inp = synth.make_inputs(B=1, S=700, Hq=4, Hkv=2, Dqk=128, Dv=128, dtype=dtype, seed=41, scale=scale)
    full_check(inp, f"{dtype} scale={scale}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_xcd_grouped_mapping(dtype):
    """B * Hkv divisible by 8 takes the XCD-grouped workgroup order."""
    inp = synth.make_inputs(B=2, S=700, Hq=8, Hkv=4, Dqk=128, Dv=128, dtype=dtype, seed=77)
    full_check(inp, f"{dtype} B2 Hq8 Hkv4 (xcd-grouped)")


# ------------------------------------------------------------------ closed forms on the GPU

@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_zero_scale_gives_prefix_mean(dtype):
    inp = synth.make_inputs(B=1, S=400, Hq=2, Hkv=1, Dqk=128, Dv=128, dtype=dtype, seed=9, scale=0.0)
    full_check(inp, f"{dtype} scale=0")


def test_fp8_v_ones_gives_exact_ones():
    """Dividing by the sum of the rounded probabilities: with V = 1 the
    weights sum to one and the output is exactly 1.0 in BF16."""
    inp = synth.make_inputs(B=1, S=1500, Hq=4, Hkv=2, Dqk=128, Dv=128, dtype="fp8", seed=12)
    inp.v = torch.full_like(inp.v.view(torch.uint8), 0x38).view(torch.float8_e4m3fn)
    inp.descale = (inp.descale[0], inp.descale[1], 1.0)
    out = run_gpu(inp).float().cpu().numpy()
    assert np.all(out == 1.0)


@pytest.mark.parametrize("Dqk,structure", [(128, "gaussian"), (128, "peaked"), (192, "gaussian")])
def test_bf16_v_ones_gives_exact_ones(Dqk, structure):
    """The BF16 row sums come from a matrix instruction of a 0/1 lane
    selector against the P operand: with V = 1 they must equal, query by
    query, the weights the P V product applies, so every output is exactly
    1.0 (a selector that mixed the lanes of two queries would not)."""
    inp = synth.make_inputs(B=1, S=1300, Hq=4, Hkv=2, Dqk=Dqk, Dv=128, dtype="bf16", seed=13, structure=structure)
    inp.v = torch.ones_like(inp.v)
    _say(f"case bf16 V=1 Dqk={Dqk} {structure}")
    out = run_gpu(inp).float().cpu().numpy()
    assert np.all(out == 1.0)


def test_fp8_matches_leanp_model_closely():
    """Diagnostic: the kernel follows the FP8-softmax model step by step
    (same tile of 128 keys, same 64-key blocks, same constant, same lazy
    reference max of 8 binades), so it sits much closer to the model than to
    the exact attention."""
    inp = synth.make_inputs(B=1, S=700, Hq=2, Hkv=1, Dqk=128, Dv=128, dtype="fp8", seed=41)
    out = run_gpu(inp).float().cpu().numpy().astype(np.float64)
    dq, dk, dv = inp.descale
    qd = oracle.dequantize(synth.raw_codes(inp.q), oracle.FP8_E4M3, dq)
    kd = oracle.dequantize(synth.raw_codes(inp.k), oracle.FP8_E4M3, dk)
    vd = oracle.dequantize(synth.raw_codes(inp.v), oracle.FP8_E4M3, 1.0)
    rows = [(0, h, i) for h in range(2) for i in list(range(0, 700, 7)) + [699]]
    model = leanp.leanp_attention(qd, kd, vd, inp.scale, dv, rows=rows, lazy_log2=8.0)
    exact = oracle_out(inp, rows=np.array(rows))
    g = np.stack([out[0, i, h] for (_, h, i) in rows])
    to_model = np.sqrt(np.sum((g - model) ** 2) / np.sum(model ** 2))
    to_exact = np.sqrt(np.sum((g - exact) ** 2) / np.sum(exact ** 2))
    _say(f"fp8 vs Lean P model rel_rms={to_model:.3e}; vs exact {to_exact:.3e}")
    assert to_model <= 5e-3 and to_model < 0.5 * to_exact


@pytest.mark.parametrize("structure,S,seed", [("gaussian", 700, 41), ("peaked", 1500, 43)])
def test_fp8_lazy_max_against_the_eager_model(structure, S, seed):
    """The kernel moves its reference max lazily (only on rises of more than 8
    binades); the plain reading of the pages moves it to every tile's max,
    which encodes each row's largest probability exactly (a power of two).
    Against exact attention the kernel's error stays within 1.6x of that
    eager model's (measured: 1.03x Gaussian, 1.46x peaked, where the row max
    dominates the output), and both stay far inside the FP8 bar."""
    inp = synth.make_inputs(B=1, S=S, Hq=2, Hkv=1, Dqk=128, Dv=128, dtype="fp8", seed=seed, structure=structure)
    out = run_gpu(inp).float().cpu().numpy().astype(np.float64)
    dq, dk, dv = inp.descale
    qd = oracle.dequantize(synth.raw_codes(inp.q), oracle.FP8_E4M3, dq)
    kd = oracle.dequantize(synth.raw_codes(inp.k), oracle.FP8_E4M3, dk)
    vd = oracle.dequantize(synth.raw_codes(inp.v), oracle.FP8_E4M3, 1.0)
    rows = [(0, h, i) for h in range(2) for i in list(range(0, S, 7)) + [S - 1]]
    eager = leanp.leanp_attention(qd, kd, vd, inp.scale, dv, rows=rows)
    exact = oracle_out(inp, rows=np.array(rows))
    g = np.stack([out[0, i, h] for (_, h, i) in rows])
    k_err, e_err = _rel(g, exact), _rel(eager, exact)
    _say(f"{structure}: kernel vs exact {k_err:.3e}, eager model vs exact {e_err:.3e}, "
         f"kernel vs eager model {_rel(g, eager):.3e}")
    assert k_err <= 1.6 * e_err and k_err <= 4e-2


# ------------------------------------------------------------------ FP8 softmax ablations

def _model_rows(inp, rows, block_scale=True, **kw):
    """The FP8-softmax model with the kernel's reference-max policy: lazy (8
    binades) with block exponents, moving on every rise without them."""
    dq, dk, dv = inp.descale
    qd = oracle.dequantize(synth.raw_codes(inp.q), oracle.FP8_E4M3, dq)
    kd = oracle.dequantize(synth.raw_codes(inp.k), oracle.FP8_E4M3, dk)
    vd = oracle.dequantize(synth.raw_codes(inp.v), oracle.FP8_E4M3, 1.0)
    return leanp.leanp_attention(qd, kd, vd, inp.scale, dv, rows=rows, lazy_log2=8.0 if block_scale else 0.0,
                                 block_scale=block_scale, **kw)


def _rel(a, b):
    return float(np.sqrt(np.sum((a - b) ** 2) / np.sum(b ** 2)))


@pytest.mark.parametrize("exact_p,block_scale", [(True, True), (False, False), (True, False)])
def test_fp8_ablations_follow_the_model(exact_p, block_scale):
    """Each ablation follows the FP8-softmax model run with the same options,
    much closer than it is to the exact attention."""
    import fp8_bf16_causal_amd as fbc
    inp = synth.make_inputs(B=1, S=700, Hq=2, Hkv=1, Dqk=128, Dv=128, dtype="fp8", seed=41)
    dq, dk, dv = inp.descale
    dev = torch.device("cuda", 0)
    out = fbc.flash_attn_func(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.scale, causal=True,
                              descale_q=dq, descale_k=dk,
                              descale_v=dv, exact_p=exact_p, block_scale=block_scale)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy().astype(np.float64)
    rows = [(0, h, i) for h in range(2) for i in list(range(0, 700, 7)) + [699]]
    model = _model_rows(inp, rows, exact_p=exact_p, block_scale=block_scale)
    exact = oracle_out(inp, rows=np.array(rows))
    g = np.stack([out[0, i, h] for (_, h, i) in rows])
    to_model, to_exact = _rel(g, model), _rel(g, exact)
    _say(f"exact_p={exact_p} block_scale={block_scale}: vs model {to_model:.3e}; vs exact {to_exact:.3e}")
    assert to_model <= 5e-3 and to_model < 0.5 * to_exact


def test_fp8_exact_p_meets_the_bar_and_beats_lean_p():
    inp = synth.make_inputs(B=1, S=1024, Hq=4, Hkv=2, Dqk=128, Dv=128, dtype="fp8", seed=55)
    import fp8_bf16_causal_amd as fbc
    dq, dk, dv = inp.descale
    dev = torch.device("cuda", 0)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    ref = oracle_out(inp)
    errs = {}
    for ex in (False, True):
        o = fbc.flash_attn_func(q, k, v, inp.scale, causal=True, descale_q=dq, descale_k=dk, descale_v=dv, exact_p=ex)
        torch.cuda.synchronize()
        got = o.float().cpu().numpy()
        errs[ex] = check(inp, got, ref, f"fp8 exact_p={ex}")[0]
    assert errs[True] < errs[False]


def test_fp8_block_scaling_matters_on_peaked_inputs():
    """Without the per-block exponent, blocks far below the row max lose
    their small probabilities to e4m3 underflow: on peaked inputs the RMS error
    doubles and the worst element error triples (the FP8-softmax model gives
    2.0x and 3.3x on this input), the reason for the third technique."""
    import fp8_bf16_causal_amd as fbc
    S, Hq, Hkv = 4096, 8, 2
    inp = synth.make_inputs(B=1, S=S, Hq=Hq, Hkv=Hkv, Dqk=128, Dv=128, dtype="fp8", seed=2, structure="peaked")
    dq, dk, dv = inp.descale
    dev = torch.device("cuda", 0)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    rng = np.random.default_rng(5)
    rows = np.array([(0, int(rng.integers(Hq)), int(rng.integers(S // 2, S))) for _ in range(96)], dtype=np.int64)
    ref = oracle_out(inp, rows=rows)
    lim = vmax(inp)
    rr, ma = {}, {}
    for bs in (True, False):
        o = fbc.flash_attn_func(q, k, v, inp.scale, causal=True,
                                descale_q=dq, descale_k=dk, descale_v=dv, block_scale=bs)
        torch.cuda.synchronize()
        got = np.stack([o[b, i, h].float().cpu().numpy() for (b, h, i) in rows]).astype(np.float64)
        rr[bs], ma[bs] = _rel(got, ref), float(np.max(np.abs(got - ref))) / lim
    _say(f"peaked S={S}: rel_rms {rr[True]:.3e} (block scaling) vs {rr[False]:.3e} (none); "
         f"maxabs/max|V| {ma[True]:.3e} vs {ma[False]:.3e}")
    assert rr[True] <= FP8_TOL[0] and rr[False] > 1.4 * rr[True] and ma[False] > 2.0 * ma[True]


# ------------------------------------------------------------------ safety and determinism

@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_every_output_element_written_and_guards_intact(dtype):
    inp = synth.make_inputs(B=2, S=259, Hq=4, Hkv=2, Dqk=128, Dv=128, dtype=dtype, seed=3)
    n = 2 * 259 * 4 * 128
    guard = 4096
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
    buf[:guard] = 7.0
    buf[-guard:] = -7.0
    out = buf[guard:guard + n].view(2, 259, 4, 128)
    run_gpu(inp, out=out)
    assert not torch.isnan(out).any()
    assert torch.all(buf[:guard] == 7.0) and torch.all(buf[-guard:] == -7.0)


@pytest.mark.parametrize("dtype,S,H", [("bf16", 512, 2), ("fp8", 2048, 8)])
def test_bitwise_deterministic_over_100_launches(dtype, S, H):
    inp = synth.make_inputs(B=1, S=S, Hq=H, Hkv=H // 2, Dqk=128, Dv=128, dtype=dtype, seed=8, device="cuda")
    first = run_gpu(inp).clone()
    outs = [run_gpu(inp) for _ in range(99)]
    for o in outs:
        assert torch.equal(o.view(torch.int16), first.view(torch.int16))


@pytest.mark.parametrize("name", ["fp8_mha_s32k", "bf16_mha_s32k", "fp8_mla_s32k"])
def test_bitwise_deterministic_full_size(name):
    """100 launches of a full benchmark shape (into one output buffer, as the
    benchmark runs them) give bitwise the same output each time."""
    import fp8_bf16_causal_amd as fbc
    inp = synth.make_config(name, device="cuda")
    p = inp.shape
    dq, dk, dv = inp.descale
    out = torch.empty((p["B"], p["S"], p["Hq"], p["Dv"]), dtype=torch.bfloat16, device="cuda")
    _say(f"case determinism {name} x100")
    fbc.flash_attn_func(inp.q, inp.k, inp.v, inp.scale, causal=True, descale_q=dq, descale_k=dk, descale_v=dv, out=out)
    first = out.clone()
    for _ in range(99):
        fbc.flash_attn_func(inp.q, inp.k, inp.v, inp.scale, causal=True,
                            descale_q=dq, descale_k=dk, descale_v=dv, out=out)
        assert torch.equal(out.view(torch.int16), first.view(torch.int16))
    torch.cuda.synchronize()


def test_runs_on_a_side_stream():
    inp = synth.make_inputs(B=1, S=300, Hq=2, Hkv=2, Dqk=128, Dv=128, dtype="fp8", seed=4)
    s = torch.cuda.Stream()
    out = run_gpu(inp, stream=s).float().cpu().numpy()
    check(inp, out, oracle_out(inp), "fp8 side stream")


def test_concurrent_calls_from_host_threads_on_separate_streams():
    """The library keeps no state between calls (the device check is cached
    in an atomic): eight host threads, each with its own stream and its own
    inputs (both dtypes, several shapes), call it at the same time, twenty
    times each; every result equals the same call made alone, bit for bit."""
    import threading

    import fp8_bf16_causal_amd as fbc
    cases = []
    for t in range(8):
        dtype = "fp8" if t % 2 else "bf16"
        inp = synth.make_inputs(B=1 + t % 2, S=200 + 97 * t, Hq=4, Hkv=2 if t % 3 else 4, Dqk=192 if t == 5 else 128,
                                Dv=128, dtype=dtype, seed=100 + t, device="cuda")
        alone = run_gpu(inp).clone()
        cases.append((inp, alone))
    errors = []

    def work(i):
        inp, alone = cases[i]
        dq, dk, dv = inp.descale
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            outs = [fbc.flash_attn_func(inp.q, inp.k, inp.v, inp.scale, causal=True,
                                        descale_q=dq, descale_k=dk, descale_v=dv)
                    for _ in range(20)]
        s.synchronize()
        for o in outs:
            if not torch.equal(o.view(torch.int16), alone.view(torch.int16)):
                errors.append(i)
                break

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    _say(f"concurrent host threads: {len(cases)} x 20 calls, mismatching cases {errors}")
    assert not errors


# ------------------------------------------------------------------ full benchmark shapes, sampled rows

def sample_rows(B, S, Hq, n_random, seed):
    rng = np.random.default_rng(seed)
    rows = [(0, 0, i) for i in range(64)]
    rows += [(B - 1, Hq - 1, i) for i in range(S - 64, S)]
    for i in (127, 128, 255, 256, 257, S // 2, S // 2 + 1):
        rows.append((0, int(rng.integers(Hq)), i))
    rows += [(int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(S))) for _ in range(n_random)]
    return np.array(rows, dtype=np.int64)


@pytest.mark.parametrize("name", ["fp8_gqa_s16k_peaked", "fp8_mha_s32k", "bf16_mha_s32k", "fp8_mla_s32k"])
def test_full_size_config_sampled_rows(name):
    inp = synth.make_config(name, device="cuda")
    p = inp.shape
    _say(f"case {name} {p}")
    out = run_gpu(inp)
    rows = sample_rows(p["B"], p["S"], p["Hq"], 192, seed=len(name))
    got = np.stack([out[b, i, h].float().cpu().numpy() for (b, h, i) in rows])
    ref = oracle_out(inp, rows=rows)
    check(inp, got, ref, f"{name} sampled {len(rows)} rows")
    assert not torch.isnan(out).any()
