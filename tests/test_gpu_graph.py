"""GPU: the library's calls captured in a HIP graph (torch.cuda.CUDAGraph)
and replayed, as a serving loop that cannot afford per-call launch overhead
would use them. Each call enqueues kernels only (no memset nodes: the
quantize prologue clears its amax word with a kernel), so the graph holds
five kernel nodes: an FP8 and a BF16 attention call and the three kernels of
one quantize call. Every replay, with the program's own eager work and
synchronisations between replays and the outputs overwritten before each,
must reproduce the eager results bit for bit."""
import sys

import pytest
import torch

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


def test_graph_replays_reproduce_eager_results():
    import fp8_bf16_causal_amd as fbc
    f8 = synth.make_inputs(B=1, S=700, Hq=4, Hkv=2, Dqk=128, Dv=128, dtype="fp8", seed=51, device="cuda")
    b16 = synth.make_inputs(B=2, S=333, Hq=2, Hkv=2, Dqk=192, Dv=128, dtype="bf16", seed=52, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(53)
    x = torch.randn((4096, 128), generator=g, device="cuda").to(torch.bfloat16)
    o8 = torch.empty((1, 700, 4, 128), dtype=torch.bfloat16, device="cuda")
    o16 = torch.empty((2, 333, 2, 128), dtype=torch.bfloat16, device="cuda")
    y = torch.empty(x.numel(), dtype=torch.uint8, device="cuda")
    sc = torch.empty(2, dtype=torch.float32, device="cuda")

    def calls():
        st = torch.cuda.current_stream().cuda_stream
        dq, dk, dv = f8.descale
        rc = fbc.attn_fwd_ex(f8.q.data_ptr(), f8.k.data_ptr(), f8.v.data_ptr(), o8.data_ptr(), 1, 4, 2, 700, 128, 128,
                             1, f8.scale, fbc.ATTN_FP8_E4M3, (dq, dk, dv), st, 0)
        assert rc == fbc.ATTN_OK, fbc.attn_strerror(rc)
        rc = fbc.attn_fwd_ex(b16.q.data_ptr(), b16.k.data_ptr(), b16.v.data_ptr(), o16.data_ptr(), 2, 2, 2, 333, 192,
                             128, 1, b16.scale, fbc.ATTN_BF16, None, st, 0)
        assert rc == fbc.ATTN_OK, fbc.attn_strerror(rc)
        rc = fbc.attn_quantize_e4m3(x.data_ptr(), y.data_ptr(), sc.data_ptr(), 4096, 128, 1, st)
        assert rc == fbc.ATTN_OK, fbc.attn_strerror(rc)

    calls()  # eager
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o8, o16, y, sc)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()  # warm-up on the capture stream's kind of stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()

    other = synth.make_inputs(B=1, S=500, Hq=2, Hkv=1, Dqk=128, Dv=128, dtype="fp8", seed=54, device="cuda")
    for r in range(4):
        # the program's own eager work between replays: a library call on other
        # inputs and a torch product, then the outputs overwritten
        fbc.flash_attn_func(other.q, other.k, other.v, other.scale, causal=True, descale_q=other.descale[0],
                            descale_k=other.descale[1], descale_v=other.descale[2])
        torch.mm(x[:1024].float(), x[:1024].float().t())
        for t in (o8, o16):
            t.fill_(float("nan"))
        y.fill_(0xAB)
        sc.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = [torch.equal(a.view(torch.uint8), b.view(torch.uint8)) for a, b in zip((o8, o16, y, sc), ref)]
        _say(f"replay {r}: fp8 {same[0]} bf16 {same[1]} quantize codes {same[2]} scale {same[3]}")
        assert all(same)
