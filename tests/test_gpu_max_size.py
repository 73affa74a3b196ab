"""GPU: the largest tensors the boundary accepts.

One batch entry of q, k, v or out must stay below 4 GiB: the kernels address
a batch entry with 32-bit byte offsets, and the host checks
Sk * max(Hq, Hkv) * max(Dqk, Dv) * 2 bytes against 2^32. With 255 heads of
65,536 rows at head dim 128 that is 4,278,190,080 bytes, 16 MiB below the
limit (BF16 tensors of exactly that size; FP8 tensors of half of it), so the
last head's last rows sit at offsets within 16 MiB of 2^32. Sampled rows of
the first and last heads are compared with the fp64 oracle at the parity
bars; 256 heads (exactly 2^32 bytes) are refused on the host. A second case
has two batch entries of 2 GiB each (BF16, 128 heads), so the second entry
starts past 2^31 and its last rows end near 2^32 bytes into each tensor.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from fp8_bf16_causal_amd import synth

pytestmark = pytest.mark.gpu

S, H, D = 65536, 255, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_bf16_causal_amd._lib as L
    L.load()
    torch.cuda.set_device(0)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _tensor(g, dtype, B=1, heads=H):
    """[B, S, heads, D] N(0, 1) values in dtype, made 4,096 rows at a time."""
    t = torch.empty((B, S, heads, D), dtype=dtype, device="cuda")
    for b in range(B):
        for r in range(0, S, 4096):
            x = torch.randn((4096, heads, D), generator=g, device="cuda", dtype=torch.float32)
            t[b, r:r + 4096] = x.to(dtype)
    return t


def test_refuses_a_batch_entry_of_four_gib():
    import fp8_bf16_causal_amd as fbc
    p = 1 << 12  # a 16-byte-aligned address; nothing is launched for a refused call
    rc = fbc.attn_fwd_ex(p, p, p, p, 1, 256, 256, S, D, D, 1, 0.088, fbc.ATTN_BF16, None, None, 0)
    assert rc == fbc.ATTN_ERR_INVALID


@pytest.mark.parametrize("dtype,B,heads", [("bf16", 1, H), ("fp8", 1, H), ("bf16", 2, 128)])
def test_largest_accepted_tensors(dtype, B, heads):
    import fp8_bf16_causal_amd as fbc
    _say(f"case max size {dtype} B={B} S={S} H={heads} D={D}")
    torch.cuda.empty_cache()
    g = torch.Generator(device="cuda").manual_seed(11 + B + (dtype == "fp8"))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float8_e4m3fn
    q, k, v = (_tensor(g, tdt, B, heads) for _ in range(3))
    out = torch.empty((B, S, heads, D), dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(D)
    dt = fbc.ATTN_BF16 if dtype == "bf16" else fbc.ATTN_FP8_E4M3
    torch.cuda.synchronize()
    rc = fbc.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, heads, heads, S, D, D, 1, scale,
                         dt, None, None, 0)
    assert rc == fbc.ATTN_OK, fbc.attn_strerror(rc)
    torch.cuda.synchronize()
    bl = B - 1  # the last batch entry
    hs = [0, heads - 1]
    rows_i = [0, 1, 127, 128, 4095, 32768, S - 129, S - 2, S - 1]
    sub = [t[bl:bl + 1, :, hs].contiguous() for t in (q, k, v)]
    rows = np.array([(0, j, i) for j in range(len(hs)) for i in rows_i], dtype=np.int64)
    odt = oracle.BF16 if dtype == "bf16" else oracle.FP8_E4M3
    ref = oracle.attention(synth.raw_codes(sub[0]), synth.raw_codes(sub[1]), synth.raw_codes(sub[2]), odt, scale,
                           rows=rows)
    got = np.stack([out[bl, i, hs[j]].float().cpu().numpy() for (_, j, i) in rows]).astype(np.float64)
    vmax = float(np.max(np.abs(oracle.dequantize(synth.raw_codes(sub[2]), odt, 1.0))))
    del q, k, v, out, sub
    torch.cuda.empty_cache()
    assert np.all(np.isfinite(got))
    err = got - ref
    rel_rms = math.sqrt(float(np.sum(err ** 2)) / float(np.sum(ref ** 2)))
    maxabs = float(np.max(np.abs(err)))
    if dtype == "bf16":
        lim_rr, lim_ma = 1e-2, 3e-2
    else:
        lim_rr, lim_ma = 4e-2, 0.1 * vmax  # max |V| over the sampled heads
    _say(f"max size {dtype}: rel_rms={rel_rms:.3e} (<= {lim_rr:g}) maxabs={maxabs:.3e} (<= {lim_ma:.3g})")
    assert rel_rms <= lim_rr and maxabs <= lim_ma
