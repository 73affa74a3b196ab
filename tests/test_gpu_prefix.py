"""GPU tests of queries after a key prefix (attn_fwd_prefix, through the C ABI):
Sq queries, the last Sq positions of Sk >= Sq keys, query i seeing keys
j <= i + Sk - Sq. Compared element by element with the fp64 oracle at the
path's bars (BF16: relative RMS <= 1e-2, max |err| <= 3e-2; FP8: relative
RMS <= 4e-2, max |err| <= 0.1 max|V dv|), and the log-sum-exp at the bounds
derived for attn_fwd_lse (tests/test_gpu_lse.py: BF16 4e-3; FP8 0.095 plus the
per-row bound of the matrix instruction's score truncation)."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from fp8_bf16_causal_amd import synth
from test_gpu_lse import lse_tol

pytestmark = pytest.mark.gpu

TOL = {"bf16": (1e-2, 3e-2), "fp8": (4e-2, 0.1)}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_bf16_causal_amd._lib as L
    L.load()
    torch.cuda.set_device(0)


def _prefix_inputs(dtype, B, Sq, Sk, Hq, Hkv, Dqk, seed, structure="gaussian"):
    full = synth.make_inputs(B=B, S=Sk, Hq=Hq, Hkv=Hkv, Dqk=Dqk, Dv=128, dtype=dtype, seed=seed, structure=structure)
    q = full.q[:, Sk - Sq:].contiguous()
    return synth.AttnInputs(q, full.k, full.v, full.dtype, full.scale, full.descale)


def _gpu(inp):
    import fp8_bf16_causal_amd as fbc
    dq, dk, dv = inp.descale
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    out, lse = fbc.flash_attn_func(q, k, v, inp.scale, causal=True,
                                   descale_q=dq, descale_k=dk, descale_v=dv, return_lse=True)
    torch.cuda.synchronize()
    return out, lse


def _oracle(inp, rows=None):
    dq, dk, dv = inp.descale
    dt = oracle.BF16 if inp.dtype == "bf16" else oracle.FP8_E4M3
    return oracle.attention(synth.raw_codes(inp.q), synth.raw_codes(inp.k), synth.raw_codes(inp.v), dt, inp.scale,
                            dq, dk, dv, rows=rows, return_lse=True)


def _vmax(inp):
    dt = oracle.BF16 if inp.dtype == "bf16" else oracle.FP8_E4M3
    return float(np.max(np.abs(oracle.dequantize(synth.raw_codes(inp.v), dt, inp.descale[2]))))


def _check(inp, got, ref, got_lse, ref_lse, label, rows=None):
    """Output at the parity bars; lse per row at lse_tol (rows: the sampled
    (b, h, i) the lse values belong to, else the whole [B, Hq, Sq])."""
    got = got.astype(np.float64)
    assert np.all(np.isfinite(got)), label
    err = got - ref
    rr = math.sqrt(float(np.sum(err ** 2)) / float(np.sum(ref ** 2)))
    ma = float(np.max(np.abs(err)))
    lim_rr, lim_ma = TOL[inp.dtype]
    if inp.dtype == "fp8":
        lim_ma *= _vmax(inp)
    tol = lse_tol(inp)
    if rows is not None:
        tol = np.array([tol[b, h, i] for b, h, i in rows])
    le = np.abs(np.asarray(got_lse, dtype=np.float64) - ref_lse)
    worst = int(np.argmax(le - tol))
    _say(f"{label}: rel_rms={rr:.3e} maxabs={ma:.3e} lse max err={le.max():.3e} "
         f"(tightest row {le.flat[worst]:.3e} <= {tol.flat[worst]:.3e})")
    assert rr <= lim_rr and ma <= lim_ma, label
    assert np.all(le <= tol), label


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,Dqk", [
    (1, 1, 1000, 2, 1, 128),      # one query over a long prefix
    (2, 65, 300, 4, 2, 128),      # ragged query block and key tile
    (1, 256, 640, 8, 8, 128),     # whole query block, prefix a multiple of the tile
    (1, 300, 301, 4, 1, 128),     # prefix of one key
    (1, 517, 1500, 4, 4, 192),    # MLA head dims
])
def test_prefix_whole_tensor(dtype, B, Sq, Sk, Hq, Hkv, Dqk):
    inp = _prefix_inputs(dtype, B, Sq, Sk, Hq, Hkv, Dqk, seed=Sq + Sk)
    _say(f"case prefix {dtype} B={B} Sq={Sq} Sk={Sk} Hq={Hq} Hkv={Hkv} Dqk={Dqk}")
    out, lse = _gpu(inp)
    ref, ref_lse = _oracle(inp)
    _check(inp, out.float().cpu().numpy(), ref, lse.cpu().numpy(), ref_lse, f"{dtype} Sq={Sq} Sk={Sk}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_prefix_with_equal_lengths_is_the_plain_call(dtype):
    """Sq = Sk through attn_fwd_prefix gives bitwise the output of attn_fwd_ex."""
    import fp8_bf16_causal_amd as fbc
    inp = synth.make_inputs(B=1, S=700, Hq=4, Hkv=2, Dqk=128, Dv=128, dtype=dtype, seed=5)
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    dq, dk, dv = inp.descale
    a = fbc.flash_attn_func(q, k, v, inp.scale, causal=True, descale_q=dq, descale_k=dk, descale_v=dv)
    b = torch.empty_like(a)
    rc = fbc.attn_fwd_prefix(q.data_ptr(), k.data_ptr(), v.data_ptr(), b.data_ptr(), None, 1, 4, 2, 700, 700, 128,
                             128, 1, inp.scale, fbc.ATTN_BF16 if dtype == "bf16" else fbc.ATTN_FP8_E4M3,
                             (dq, dk, dv), torch.cuda.current_stream().cuda_stream, 0)
    torch.cuda.synchronize()
    assert rc == fbc.ATTN_OK
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_prefix_fp8_peaked():
    inp = _prefix_inputs("fp8", 1, 384, 2048, 4, 1, 128, seed=44, structure="peaked")
    _say("case prefix fp8 peaked Sq=384 Sk=2048")
    out, lse = _gpu(inp)
    ref, ref_lse = _oracle(inp)
    _check(inp, out.float().cpu().numpy(), ref, lse.cpu().numpy(), ref_lse, "fp8 peaked prefix")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_prefix_long_context_chunk_sampled_rows(dtype):
    """The last 4,096 queries of a 32K sequence (the shape of one chunk of a
    context-parallel split), on sampled rows."""
    inp = _prefix_inputs(dtype, 1, 4096, 32768, 8, 8, 128, seed=9)
    _say(f"case prefix {dtype} Sq=4096 Sk=32768 H=8")
    out, lse = _gpu(inp)
    rng = np.random.default_rng(1)
    rows = np.array([(0, 0, i) for i in range(32)] + [(0, 7, 4095 - i) for i in range(32)] +
                    [(0, int(rng.integers(8)), int(rng.integers(4096))) for _ in range(64)], dtype=np.int64)
    ref, ref_lse = _oracle(inp, rows=rows)
    got = np.stack([out[b, i, h].float().cpu().numpy() for b, h, i in rows])
    l = lse.cpu().numpy()
    _check(inp, got, ref, np.array([l[b, h, i] for b, h, i in rows]), ref_lse, f"{dtype} chunk sampled rows",
           rows=rows)


@pytest.mark.parametrize("case", range(24))
def test_random_prefix_shapes(case):
    """Seeded random configurations of the prefix case: Sq in 1..1024 queries
    after Sk - Sq in 0..1500 earlier keys, batch 1-2, KV heads 1-4, GQA ratio
    1-4, head dims 128 or 192 / 128, dtype and input structure drawn together;
    output and lse over the whole tensors at the bars above."""
    r = np.random.default_rng(12000 + case)
    hkv = int(r.integers(1, 5))
    sq = int(r.integers(1, 1025))
    c = dict(dtype=str(r.choice(["bf16", "fp8"])), B=int(r.integers(1, 3)), Sq=sq, Sk=sq + int(r.integers(0, 1501)),
             Hq=hkv * int(r.integers(1, 5)), Hkv=hkv, Dqk=int(r.choice([128, 192])),
             structure=str(r.choice(["gaussian", "peaked"])))
    inp = _prefix_inputs(c["dtype"], c["B"], c["Sq"], c["Sk"], c["Hq"], c["Hkv"], c["Dqk"], seed=13000 + case,
                         structure=c["structure"])
    _say(f"random prefix case {case}: {c}")
    out, lse = _gpu(inp)
    ref, ref_lse = _oracle(inp)
    _check(inp, out.float().cpu().numpy(), ref, lse.cpu().numpy(), ref_lse, f"random prefix case {case}")
