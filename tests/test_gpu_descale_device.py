"""GPU: FP8 prefill from BF16 tensors with no host round trip. Q and K are
quantised with the Hadamard rotation and V without, by attn_quantize_e4m3,
into one device buffer {dq, amax_q, dk, amax_k, dv, amax_v}; the attention
reads its dequantisation factors from that buffer (ATTN_FLAG_DESCALE_DEVICE).
The output must equal, bit for bit, the same call with the factors read back
and passed from the host, and meet the FP8 bar against the oracle; and the
whole chain (three quantize calls and the attention) captured in a HIP graph
must follow new input values on every replay, scales included."""
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


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bf16_inputs(seed, B=1, S=1000, Hq=4, Hkv=2, D=128):
    inp = synth.make_inputs(B=B, S=S, Hq=Hq, Hkv=Hkv, Dqk=D, Dv=D, dtype="bf16", seed=seed, structure="peaked",
                            device="cuda")
    return inp.q, inp.k, inp.v, inp.scale


def _chain(q, k, v, scale, buf):
    """Quantise (rotating Q and K) into buf, then attention with device factors."""
    import fp8_bf16_causal_amd as fbc
    q8, _ = fbc.quantize_e4m3(q, hadamard=True, scale_out=buf[0:2])
    k8, _ = fbc.quantize_e4m3(k, hadamard=True, scale_out=buf[2:4])
    v8, _ = fbc.quantize_e4m3(v, hadamard=False, scale_out=buf[4:6])
    out = fbc.flash_attn_func(q8, k8, v8, scale, causal=True, descale_device=buf)
    return q8, k8, v8, out


def test_device_factors_equal_host_factors_and_meet_the_bar():
    import fp8_bf16_causal_amd as fbc
    q, k, v, scale = _bf16_inputs(61)
    buf = torch.empty(6, dtype=torch.float32, device="cuda")
    q8, k8, v8, out_dev = _chain(q, k, v, scale, buf)
    torch.cuda.synchronize()
    dq, _, dk, _, dv, _ = [float(x) for x in buf.cpu()]
    out_host = fbc.flash_attn_func(q8, k8, v8, scale, causal=True, descale_q=dq, descale_k=dk, descale_v=dv)
    torch.cuda.synchronize()
    assert torch.equal(out_dev.view(torch.int16), out_host.view(torch.int16))
    ref = oracle.attention(synth.raw_codes(q8), synth.raw_codes(k8), synth.raw_codes(v8), oracle.FP8_E4M3, scale,
                           dq, dk, dv)
    got = out_dev.float().cpu().numpy().astype(np.float64)
    err = got - ref
    rel = math.sqrt(float(np.sum(err ** 2)) / float(np.sum(ref ** 2)))
    vmax = float(np.max(np.abs(oracle.dequantize(synth.raw_codes(v8), oracle.FP8_E4M3, dv))))
    _say(f"device factors dq={dq:.4g} dk={dk:.4g} dv={dv:.4g}: rel_rms={rel:.3e} maxabs={np.max(np.abs(err)):.3e}")
    assert rel <= 4e-2 and float(np.max(np.abs(err))) <= 0.1 * vmax


def test_chain_in_a_graph_follows_new_inputs():
    q, k, v, scale = _bf16_inputs(62)
    sq, sk, sv = (t.clone() for t in (q, k, v))  # static inputs of the graph
    buf = torch.empty(6, dtype=torch.float32, device="cuda")
    _chain(sq, sk, sv, scale, buf)  # warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _, _, _, gout = _chain(sq, sk, sv, scale, buf)
    torch.cuda.synchronize()
    for r in range(3):
        nq, nk, nv, _ = _bf16_inputs(70 + r)
        amp = 0.25 * (r + 1)  # new magnitudes: the factors must change too
        sq.copy_(nq * amp)
        sk.copy_(nk)
        sv.copy_(nv * (4.0 - r))
        gout.fill_(float("nan"))
        buf.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = gout.clone()
        got_buf = buf.clone()
        ebuf = torch.empty(6, dtype=torch.float32, device="cuda")
        _, _, _, eout = _chain(sq, sk, sv, scale, ebuf)
        torch.cuda.synchronize()
        same = torch.equal(got.view(torch.int16), eout.view(torch.int16)) and torch.equal(got_buf, ebuf)
        _say(f"replay {r}: factors {[round(float(x), 5) for x in got_buf.cpu()[0::2]]} identical to eager {same}")
        assert same


@pytest.mark.parametrize("flags", [0, 1, 2, 3])
def test_device_factors_through_lse_and_prefix_entry_points(flags):
    """attn_fwd_lse and attn_fwd_prefix with ATTN_FLAG_DESCALE_DEVICE (alone
    and with each ablation flag): out and lse bit-identical to the calls with
    the same factors passed from the host. The six floats sit at a 4-byte
    offset inside a larger buffer (only 4-byte alignment is required)."""
    import fp8_bf16_causal_amd._lib as L
    q, k, v, scale = _bf16_inputs(63, S=700)
    big = torch.full((16,), -1.0, dtype=torch.float32, device="cuda")
    buf = big[1:7]
    q8, k8, v8, _ = _chain(q, k, v, scale, buf)
    torch.cuda.synchronize()
    host = [float(x) for x in buf.cpu()[0::2]]
    B, S, Hq, D = q8.shape
    Hkv = k8.shape[2]
    dev_flags = flags | L.ATTN_FLAG_DESCALE_DEVICE
    for Sq in (S, 300):
        qq = q8[:, S - Sq:].contiguous()
        res = []
        for fl, ds in ((dev_flags, buf.data_ptr()), (flags, host)):
            out = torch.full((B, Sq, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
            lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device="cuda")
            if Sq == S:
                rc = L.attn_fwd_lse(qq.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq,
                                    Hkv, S, D, D, 1, scale, L.ATTN_FP8_E4M3, ds, None, fl)
            else:
                rc = L.attn_fwd_prefix(qq.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(), lse.data_ptr(), B,
                                       Hq, Hkv, Sq, S, D, D, 1, scale, L.ATTN_FP8_E4M3, ds, None, fl)
            assert rc == 0, L.attn_strerror(rc)
            res.append((out, lse))
        torch.cuda.synchronize()
        (od, ld), (oh, lh) = res
        same = torch.equal(od.view(torch.int16), oh.view(torch.int16)) and torch.equal(ld, lh)
        _say(f"flags={flags} Sq={Sq} Sk={S}: device factors identical to host factors {same}")
        assert same
        assert not torch.isnan(ld).any()


def test_flash_attention_keyword_aliases_give_the_same_result():
    """flash_attn_func's flash-attention spellings (q_descale/k_descale/
    v_descale as one-element device tensors, window_size=(-1, 0) with causal,
    deterministic=True, positional softmax_scale and causal) give the same
    bits as the library's own keywords."""
    import fp8_bf16_causal_amd as fbc
    q, k, v, scale = _bf16_inputs(64, S=500)
    q8, sq = fbc.quantize_e4m3(q, hadamard=True)
    k8, sk = fbc.quantize_e4m3(k, hadamard=True)
    v8, sv = fbc.quantize_e4m3(v)
    torch.cuda.synchronize()
    dq, dk, dv = float(sq[0]), float(sk[0]), float(sv[0])
    a = fbc.flash_attn_func(q8, k8, v8, scale, causal=True, descale_q=dq, descale_k=dk, descale_v=dv)
    b = fbc.flash_attn_func(q8, k8, v8, scale, True, q_descale=sq[0:1], k_descale=sk[0:1], v_descale=sv[0:1],
                            window_size=(-1, 0), deterministic=True)
    torch.cuda.synchronize()
    same = torch.equal(a.view(torch.int16), b.view(torch.int16))
    _say(f"flash-attention keyword spellings identical {same}")
    assert same


@pytest.mark.parametrize("hadamard", [True, False])
def test_one_call_fp8_prefill_from_bf16(hadamard):
    """flash_attn_fp8_func: the same bits as the chain of three quantize calls
    and the attention on device factors, with and without the rotation (and
    with return_lse, the same lse as the chain's)."""
    import fp8_bf16_causal_amd as fbc
    q, k, v, scale = _bf16_inputs(65, S=600)
    buf = torch.empty(6, dtype=torch.float32, device="cuda")
    q8, _ = fbc.quantize_e4m3(q, hadamard=hadamard, scale_out=buf[0:2])
    k8, _ = fbc.quantize_e4m3(k, hadamard=hadamard, scale_out=buf[2:4])
    v8, _ = fbc.quantize_e4m3(v, scale_out=buf[4:6])
    ref, ref_lse = fbc.flash_attn_func(q8, k8, v8, scale, causal=True, descale_device=buf, return_lse=True)
    got, got_lse = fbc.flash_attn_fp8_func(q, k, v, scale, hadamard=hadamard, return_lse=True)
    torch.cuda.synchronize()
    same = torch.equal(got.view(torch.int16), ref.view(torch.int16)) and torch.equal(got_lse, ref_lse)
    _say(f"one-call FP8 prefill (hadamard={hadamard}) identical to the chain {same}")
    assert same
