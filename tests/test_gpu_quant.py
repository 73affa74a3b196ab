"""GPU tests of the FP8 quantize prologue (attn_quantize_e4m3, through the C
ABI): codes bit-exact against the oracle (every code is an fp32 decision both
sides take in the same order), scale and amax equal, and the rotation's effect
on the attention result."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import quant
from fp8_bf16_causal_amd import synth

pytestmark = pytest.mark.gpu


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


def run_quant(x, hadamard):
    import fp8_bf16_causal_amd as fbc
    y, sc = fbc.quantize_e4m3(x.cuda(), hadamard=hadamard)
    torch.cuda.synchronize()
    return y.view(torch.uint8).cpu().numpy(), sc.cpu().numpy()


def bits(x):
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("hadamard", [False, True])
@pytest.mark.parametrize("rows,dim", [(1, 64), (7, 128), (1000, 128), (333, 192), (65, 256), (4099, 128)])
def test_codes_bit_exact(rows, dim, hadamard):
    g = torch.Generator().manual_seed(rows * 7 + dim)
    x = torch.randn((rows, dim), generator=g) * 3
    x[:, :: max(1, dim // 5)] *= 8.0  # a few outlier channels
    x[0, 0] = -0.0
    if rows > 1:
        x[rows - 1] = -0.0  # a whole row of -0: its rotation keeps one -0 per block
    x = x.to(torch.bfloat16)
    _say(f"quantize rows={rows} dim={dim} hadamard={hadamard}")
    codes, sc = run_quant(x, hadamard)
    ref, s, amax = quant.quantize_e4m3(bits(x), hadamard)
    assert sc[1] == amax and sc[0] == s
    mism = int(np.sum(codes.reshape(ref.shape) != ref))
    assert mism == 0, f"{mism} codes differ"


@pytest.mark.parametrize("hadamard", [False, True])
@pytest.mark.parametrize("exp2", [-100, -40, 20])
def test_codes_bit_exact_at_extreme_scales(hadamard, exp2):
    """Values spread over many binades, times 2^exp2 (exact in BF16): with
    2^-100 the scale falls below 2^-69 and the kernel takes its plain-division
    path, with 2^-40 and 2^20 its reciprocal-and-correction path. The spread
    leaves many quotients tiny, so subnormal e4m3 codes are exercised."""
    g = torch.Generator().manual_seed(31 - exp2)
    x = torch.randn((2000, 128), generator=g) * torch.exp2(torch.randn((2000, 1), generator=g) * 6)
    x = (x * 2.0 ** exp2).to(torch.bfloat16)
    _say(f"quantize extreme scale 2^{exp2} hadamard={hadamard}")
    codes, sc = run_quant(x, hadamard)
    ref, s, amax = quant.quantize_e4m3(bits(x), hadamard)
    assert sc[1] == amax and sc[0] == s
    mism = int(np.sum(codes.reshape(ref.shape) != ref))
    assert mism == 0, f"{mism} codes differ"
    assert (ref & 0x7F).min() == 0 and np.sum((ref & 0x7F) < 8) > 1000  # many subnormal codes exercised


@pytest.mark.parametrize("case", range(24))
def test_codes_bit_exact_random(case):
    """Seeded random tensors: rows 1..5000, dim 64/128/192/256, with or without
    the rotation, magnitudes 2^e with e drawn in [-60, 40] and a per-row spread
    of up to 2^+-8, an occasional outlier column and signed zeros: codes bit
    for bit, s and amax equal."""
    r = np.random.default_rng(500 + case)
    rows, dim = int(r.integers(1, 5001)), int(r.choice([64, 128, 192, 256]))
    had, e = bool(r.integers(0, 2)), int(r.integers(-60, 41))
    g = torch.Generator().manual_seed(600 + case)
    x = torch.randn((rows, dim), generator=g) * torch.exp2(torch.randn((rows, 1), generator=g) * 3)
    if r.integers(0, 2):
        x[:, int(r.integers(0, dim))] *= 16.0
    x[int(r.integers(0, rows)), :: 7] = -0.0
    x = (x * 2.0 ** e).to(torch.bfloat16)
    _say(f"quantize random case {case}: rows={rows} dim={dim} hadamard={had} 2^{e}")
    codes, sc = run_quant(x, had)
    ref, s, amax = quant.quantize_e4m3(bits(x), had)
    assert sc[1] == amax and sc[0] == s
    mism = int(np.sum(codes.reshape(ref.shape) != ref))
    assert mism == 0, f"{mism} codes differ"


def test_zero_tensor():
    codes, sc = run_quant(torch.zeros((9, 128), dtype=torch.bfloat16), True)
    assert sc[0] == 1.0 and sc[1] == 0.0 and not codes.any()


@pytest.mark.parametrize("hadamard", [False, True])
def test_full_size_q_tensor(hadamard):
    """A query tensor of the 32K benchmark shape (32768 x 32 heads x 128)."""
    g = torch.Generator().manual_seed(3)
    x = torch.randn((32768, 32, 128), generator=g).to(torch.bfloat16)
    _say(f"quantize full-size Q hadamard={hadamard}")
    codes, sc = run_quant(x, hadamard)
    ref, s, amax = quant.quantize_e4m3(bits(x).reshape(-1, 128), hadamard)
    assert sc[1] == amax and sc[0] == s
    assert np.array_equal(codes.reshape(ref.shape), ref)


def test_rotation_lowers_fp8_attention_error_on_peaked_inputs():
    """Quantise BF16 Q, K, V on the GPU (Q and K rotated or not), run the FP8
    attention, and compare with exact attention of the BF16 inputs: the
    rotation spreads the outlier channels and lowers the error."""
    import fp8_bf16_causal_amd as fbc
    S, H, D = 2048, 4, 128
    inp = synth.make_inputs(B=1, S=S, Hq=H, Hkv=H, Dqk=D, Dv=D, dtype="bf16", seed=2, structure="peaked")
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    rows = np.array([(0, h, i) for h in range(H) for i in range(0, S, 37)] + [(0, 0, S - 1)], dtype=np.int64)
    ref = oracle.attention(synth.raw_codes(inp.q), synth.raw_codes(inp.k), synth.raw_codes(inp.v), oracle.BF16,
                           inp.scale, rows=rows)
    err = {}
    for rot in (False, True):
        cq, sq = fbc.quantize_e4m3(q, hadamard=rot)
        ck, sk = fbc.quantize_e4m3(k, hadamard=rot)
        cv, sv = fbc.quantize_e4m3(v, hadamard=False)
        ds = [float(t[0]) for t in (sq, sk, sv)]
        out = fbc.flash_attn_func(cq, ck, cv, inp.scale, causal=True, descale_q=ds[0], descale_k=ds[1], descale_v=ds[2])
        torch.cuda.synchronize()
        got = np.stack([out[b, i, h].float().cpu().numpy() for (b, h, i) in rows]).astype(np.float64)
        err[rot] = math.sqrt(float(np.sum((got - ref) ** 2)) / float(np.sum(ref ** 2)))
    _say(f"FP8 attention vs exact BF16 attention: rel_rms {err[False]:.3e} plain, {err[True]:.3e} rotated")
    # the pages: the rotation roughly halves the input-quantisation error (here the
    # sink and outlier channels make the per-tensor scale coarse without it)
    assert err[True] < 0.5 * err[False]


@pytest.mark.parametrize("hadamard", [False, True])
def test_more_than_two_to_the_31_elements(hadamard):
    """2^31 + 2^20 elements in 128-element rows, so element indices pass 2^31:
    noise in [-1/16, 1/16] and one spike of 100 in a row past 2^31. The
    spike's block holds the tensor's amax with and without the rotation (any
    other rotated value is below 0.71, the spike's block's above 8.1), so the
    oracle run on that row together with sampled rows (the first, around 2^31,
    the last) decides the same scale, and every sampled code must agree."""
    import fp8_bf16_causal_amd as fbc
    dim = 128
    n = (1 << 31) + (1 << 20)
    rows = n // dim
    _say(f"quantize {n} elements hadamard={hadamard}")
    x = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(77)
    chunk = 1 << 26
    for o in range(0, n, chunk):
        m = min(chunk, n - o)
        x[o:o + m] = ((torch.rand(m, generator=g, device="cuda") - 0.5) * 0.125).to(torch.bfloat16)
    r31 = (1 << 31) // dim
    spike_row = r31 + 1234
    x[spike_row * dim + 37] = 100.0
    y = torch.empty(n, dtype=torch.uint8, device="cuda")
    sc = torch.empty(2, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rc = fbc.attn_quantize_e4m3(x.data_ptr(), y.data_ptr(), sc.data_ptr(), rows, dim, int(hadamard), stream)
    assert rc == fbc.ATTN_OK, fbc.attn_strerror(rc)
    torch.cuda.synchronize()
    sample = [0, 1, r31 - 1, r31, r31 + 1, spike_row, rows - 2, rows - 1]
    xs = torch.stack([x[r * dim:(r + 1) * dim] for r in sample]).cpu()
    got = torch.stack([y[r * dim:(r + 1) * dim] for r in sample]).cpu().numpy()
    scv = sc.cpu().numpy()
    del x, y
    torch.cuda.empty_cache()
    ref, s, amax = quant.quantize_e4m3(bits(xs), hadamard)
    assert scv[1] == amax and scv[0] == s
    mism = int(np.sum(got != ref))
    assert mism == 0, f"{mism} codes differ"
