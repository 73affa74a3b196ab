"""GPU: the plain entry point attn_fwd(q, k, v, out, B, Hq, Hkv, S, Dqk, Dv,
causal, scale, dtype) itself, with valid arguments (no descales, the default
stream), against the fp64 oracle at the parity bars, and bit for bit against
attn_fwd_ex(..., descale_qkv=NULL, stream=NULL, flags=0), which it must
equal. FP8 inputs are N(0, 1) values cast to e4m3fn directly, so the unit
dequantisation factors attn_fwd implies are the right ones."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from fp8_bf16_causal_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_bf16_causal_amd._lib as L
    L.load()
    torch.cuda.set_device(0)


def _inputs(dtype, B, S, Hq, Hkv, Dqk, Dv, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, S, Hq, Dqk), generator=g)
    k = torch.randn((B, S, Hkv, Dqk), generator=g)
    v = torch.randn((B, S, Hkv, Dv), generator=g)
    t = torch.bfloat16 if dtype == "bf16" else torch.float8_e4m3fn
    return [x.to(t) for x in (q, k, v)]


@pytest.mark.parametrize("dtype,B,S,Hq,Hkv,Dqk", [
    ("bf16", 2, 333, 4, 2, 128),
    ("fp8", 2, 333, 4, 2, 128),
    ("fp8", 1, 517, 4, 4, 192),
    ("bf16", 1, 300, 2, 1, 192),
])
def test_attn_fwd_matches_oracle_and_attn_fwd_ex(dtype, B, S, Hq, Hkv, Dqk):
    import fp8_bf16_causal_amd as fbc

    Dv = 128
    print(f"case attn_fwd {dtype} B{B} S{S} Hq{Hq} Hkv{Hkv} Dqk{Dqk}", flush=True)
    sys.stdout.flush()
    q, k, v = _inputs(dtype, B, S, Hq, Hkv, Dqk, Dv, seed=S + Dqk)
    dev = torch.device("cuda", 0)
    qg, kg, vg = (x.to(dev) for x in (q, k, v))
    out = torch.full((B, S, Hq, Dv), float("nan"), dtype=torch.bfloat16, device=dev)
    out_ex = torch.full_like(out, float("nan"))
    scale = 1.0 / math.sqrt(Dqk)
    dt = fbc.ATTN_BF16 if dtype == "bf16" else fbc.ATTN_FP8_E4M3
    torch.cuda.synchronize()
    rc = fbc.attn_fwd(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), out.data_ptr(), B, Hq, Hkv, S, Dqk, Dv, 1, scale,
                      dt)
    assert rc == fbc.ATTN_OK, fbc.attn_strerror(rc)
    rc = fbc.attn_fwd_ex(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), out_ex.data_ptr(), B, Hq, Hkv, S, Dqk, Dv, 1,
                         scale, dt, None, None, 0)
    assert rc == fbc.ATTN_OK, fbc.attn_strerror(rc)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_ex.view(torch.int16))
    got = out.float().cpu().numpy().astype(np.float64)
    odt = oracle.BF16 if dtype == "bf16" else oracle.FP8_E4M3
    ref = oracle.attention(synth.raw_codes(q), synth.raw_codes(k), synth.raw_codes(v), odt, scale)
    assert np.all(np.isfinite(got))
    err = got - ref
    rel_rms = math.sqrt(float(np.sum(err ** 2)) / float(np.sum(ref ** 2)))
    maxabs = float(np.max(np.abs(err)))
    if dtype == "bf16":
        lim_rr, lim_ma = 1e-2, 3e-2
    else:
        lim_rr, lim_ma = 4e-2, 0.1 * float(np.max(np.abs(oracle.dequantize(synth.raw_codes(v), odt))))
    print(f"attn_fwd {dtype}: rel_rms={rel_rms:.3e} (<= {lim_rr:g}) maxabs={maxabs:.3e} (<= {lim_ma:.3g})", flush=True)
    assert rel_rms <= lim_rr and maxabs <= lim_ma
