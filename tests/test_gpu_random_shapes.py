"""GPU parity on seeded random shapes: batch, head layout (GQA ratio), length,
head dims, dtype, input structure and softmax scale drawn together, each case
compared over its whole output with the fp64 oracle at the parity bars
(BF16: relative RMS <= 1e-2, max abs <= 3e-2; FP8: relative RMS <= 4e-2,
max abs <= 0.1 max|V dv|), and its per-row log-sum-exp at the bounds derived
in tests/test_gpu_lse.py. The draws are fixed by the case index, so a
failure names a reproducible configuration."""
import numpy as np
import pytest
import torch

import oracle
from fp8_bf16_causal_amd import synth
from test_gpu_lse import lse_tol
from test_gpu_parity import _say, check

pytestmark = pytest.mark.gpu

N_CASES = 48


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_bf16_causal_amd._lib as L
    L.load()
    torch.cuda.set_device(0)


def draw(case):
    r = np.random.default_rng(9000 + case)
    hkv = int(r.integers(1, 5))
    return dict(B=int(r.integers(1, 4)), Hkv=hkv, Hq=hkv * int(r.integers(1, 5)), S=int(r.integers(1, 2049)),
                Dqk=int(r.choice([128, 192])), dtype=str(r.choice(["bf16", "fp8"])),
                structure=str(r.choice(["gaussian", "peaked"])), scale=float(10.0 ** r.uniform(-2.0, -0.3)))


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_shape(case):
    import fp8_bf16_causal_amd as fbc
    c = draw(case)
    inp = synth.make_inputs(B=c["B"], S=c["S"], Hq=c["Hq"], Hkv=c["Hkv"], Dqk=c["Dqk"], Dv=128, dtype=c["dtype"],
                            seed=7000 + case, structure=c["structure"], scale=c["scale"])
    label = f"random case {case}: {c}"
    _say(label)
    dq, dk, dv = inp.descale
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    out, lse = fbc.flash_attn_func(q, k, v, inp.scale, causal=True, descale_q=dq, descale_k=dk, descale_v=dv,
                                   return_lse=True)
    torch.cuda.synchronize()
    dt = oracle.BF16 if inp.dtype == "bf16" else oracle.FP8_E4M3
    ref, ref_lse = oracle.attention(synth.raw_codes(inp.q), synth.raw_codes(inp.k), synth.raw_codes(inp.v), dt,
                                    inp.scale, dq, dk, dv, return_lse=True)
    check(inp, out.float().cpu().numpy(), ref, label)
    le = np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse)
    tol = lse_tol(inp)
    worst = int(np.argmax(le - tol))
    _say(f"{label}: lse max err={le.max():.3e} (tightest row {le.flat[worst]:.3e} <= {tol.flat[worst]:.3e})")
    assert np.all(le <= tol), label
