"""GPU characterisation of the FP8 matrix instruction's dot product, read
through the public API (scores -> softmax weights -> output with V one-hot).

On gfx950 the FP8 matrix instruction (v_mfma_scale_f32_32x32x64_f8f6f4) adds
the products of each group of 8 consecutive k indices (k = 8m .. 8m+7) after
truncating every product toward zero to a multiple of 2^(E - 13), E being the
group's largest exponent sum e_a + e_b of its operands; the group sums then
add exactly. (Measured with an in-bounds probe of the instruction: next to
448 x 448, products of 1 are lost within its group and kept in the next one;
15 becomes 8, 30 becomes 24, -1 becomes 0.) The BF16 instruction shows no
such loss. The FP8 scores, the FP8 row sums and the FP8 P V products inherit
this rounding; the bounds of the log-sum-exp tests include it.

Each case: query 1 sees keys 0 and 1, whose dot products with it share one
large product (448 x 448) and differ by small ones; the softmax scale maps
8 code units of score to one binade, so the weights of keys 0 and 1 are in
the ratio 2^(d/8), d the score difference the instruction computes."""
import math

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_bf16_causal_amd._lib as L
    L.load()
    torch.cuda.set_device(0)


def _ratio(small_at, dtype):
    """small_at: {k: value} products added to key 0's dot product (query
    element value x key element 1.0) beside the shared 448 x 448 at k = 0."""
    import fp8_bf16_causal_amd as fbc
    D = 128
    q = torch.zeros(1, 2, 1, D)
    k = torch.zeros(1, 2, 1, D)
    v = torch.zeros(1, 2, 1, D)
    q[0, :, 0, 0] = 448.0
    k[0, :, 0, 0] = 448.0
    for kk, val in small_at.items():
        q[0, :, 0, kk] = val
        k[0, 0, 0, kk] = 1.0
    v[0, 0, 0, 0] = 1.0
    v[0, 1, 0, 1] = 1.0
    scale = 1.0 / (8.0 * math.log2(math.e))  # 8 code units -> one binade
    t = [x.to(dtype).cuda() for x in (q, k, v)]
    o = fbc.flash_attn_func(*t, softmax_scale=scale, causal=True)
    torch.cuda.synchronize()
    o = o.float().cpu()[0, 1, 0]
    return float(o[0] / o[1])


# (products of key 0 beyond the shared one, score difference the FP8
# instruction computes under the truncation model, exact difference)
CASES = [
    ({k: 1.0 for k in range(1, 8)}, 0, 7),          # seven 1's in the large product's group: all lost
    ({k: 1.0 for k in range(8, 16)}, 8, 8),         # eight 1's in the next group: exact
    ({1: 15.0}, 8, 15),                              # 15 truncated to the group grid of 8
    ({1: 8.0, 9: 8.0}, 16, 16),                      # multiples of the grid: exact
    ({1: 4.0, 8: 4.0}, 4, 8),                        # 4 lost in the group of 448^2, kept in the next
]


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_fp8_products_truncated_per_group_of_eight(idx):
    small_at, d_fp8, d_exact = CASES[idx]
    r8 = _ratio(small_at, torch.float8_e4m3fn)
    r16 = _ratio(small_at, torch.bfloat16)
    print(f"case {idx}: FP8 weight ratio {r8:.4f} (model 2^({d_fp8}/8) = {2 ** (d_fp8 / 8):.4f}), "
          f"BF16 {r16:.4f} (exact 2^({d_exact}/8) = {2 ** (d_exact / 8):.4f})", flush=True)
    # FP8: Lean P codes of weights whose ratio is a power of two are exact, so
    # the ratio is the model's to BF16 output rounding; otherwise within the
    # encoding's 7.5% per weight
    tol8 = 0.01 if d_fp8 % 8 == 0 else 0.16
    assert abs(r8 / 2 ** (d_fp8 / 8) - 1.0) <= tol8
    # BF16: the exact difference (weights rounded to BF16 and output to BF16)
    assert abs(r16 / 2 ** (d_exact / 8) - 1.0) <= 0.01
