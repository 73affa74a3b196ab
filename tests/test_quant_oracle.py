"""Pins of the quantize-prologue oracle against things it does not compute
itself: the textbook Hadamard matrix (scipy), the algebra of the normalised
transform, torch's float8_e4m3fn cast, and hand-derived codes."""
import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import quant


def _bf16_bits(a):
    return torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("n", [64, 128])
def test_fwht_matches_the_textbook_hadamard_matrix(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal((7, 3 * n)).astype(np.float32)
    H = scipy.linalg.hadamard(n).astype(np.float64) / np.sqrt(n)
    ref = np.concatenate([x[:, j * n:(j + 1) * n].astype(np.float64) @ H.T for j in range(3)], axis=1)
    got = quant.fwht_f32(x, n).astype(np.float64)
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))


def test_fwht_is_orthogonal_and_an_involution():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    y = quant.fwht_f32(x, 128)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-5)
    np.testing.assert_allclose(quant.fwht_f32(y, 128), x, atol=1e-5)
    # (Q H)(K H)^T = Q K^T: the rotation leaves the scores unchanged
    k = rng.standard_normal((16, 128)).astype(np.float32)
    np.testing.assert_allclose(y @ quant.fwht_f32(k, 128).T, x @ k.T, atol=1e-4)


def test_fwht_of_a_unit_vector_is_a_constant_row():
    e = np.zeros((1, 64), dtype=np.float32)
    e[0, 0] = 1.0
    np.testing.assert_array_equal(quant.fwht_f32(e, 64), np.full((1, 64), 0.125, dtype=np.float32))


def test_codes_match_torchs_float8_cast():
    rng = np.random.default_rng(5)
    q = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-1, 1, 20000) * 2.0 ** -6,
                        np.arange(-448, 448.5, 0.25)]).astype(np.float32)
    ref = torch.tensor(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(quant.e4m3_codes(q), ref)


def test_hand_derived_codes_without_rotation():
    # amax = 448 -> s = 1; 448 = 1.75 * 2^8 (exponent field 15, mantissa 6), -224 = -1.75 * 2^7,
    # 1 = 2^0 (exponent field 7), 0.5 = 2^-1, 2^-9 the smallest subnormal, 0 stays 0
    x = _bf16_bits([448.0, -224.0, 1.0, 0.5, 2.0 ** -9, 0.0] + [0.0] * 58)
    codes, s, amax = quant.quantize_e4m3(x.reshape(1, 64), hadamard=False)
    assert s == np.float32(1.0) and amax == np.float32(448.0)
    assert list(codes[0, :6]) == [0x7E, 0xF6, 0x38, 0x30, 0x01, 0x00]


def test_zero_tensor_gets_unit_scale():
    codes, s, amax = quant.quantize_e4m3(np.zeros((3, 128), dtype=np.uint16), hadamard=True)
    assert s == np.float32(1.0) and amax == np.float32(0.0) and not codes.any()


@pytest.mark.parametrize("hadamard", [False, True])
def test_dequantised_values_within_half_a_code_step(hadamard):
    rng = np.random.default_rng(11)
    x = _bf16_bits(rng.standard_normal((40, 192)) * 3)
    codes, s, amax = quant.quantize_e4m3(x, hadamard)
    y = quant.bf16_to_f32(x)
    if hadamard:
        y = quant.fwht_f32(y, 64)
    deq = torch.tensor(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64) * float(s)
    err = np.abs(deq - y)
    # e4m3: 3 mantissa bits -> half a step is 2^-4 relative for normals, 2^-10 * s absolute for subnormals
    assert np.all(err <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10 * float(s)) * (1 + 1e-6))
    assert np.max(codes & 0x7F) == 0x7E  # the largest magnitude maps to 448


def test_rotation_spreads_outlier_channels():
    """With a few large channels (the peaked inputs), rotating first lowers the
    quantisation error of the scores: the reason for the rotation."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal((256, 128))
    k = rng.standard_normal((256, 128))
    q[:, [3, 50, 77, 101]] *= 8.0
    k[:, [3, 50, 77, 101]] *= 8.0
    exact = q @ k.T

    def scores(h):
        cq, sq, _ = quant.quantize_e4m3(_bf16_bits(q), h)
        ck, sk, _ = quant.quantize_e4m3(_bf16_bits(k), h)
        dq = torch.tensor(cq).view(torch.float8_e4m3fn).double().numpy() * float(sq)
        dk = torch.tensor(ck).view(torch.float8_e4m3fn).double().numpy() * float(sk)
        return dq @ dk.T

    e_plain = np.linalg.norm(scores(False) - exact)
    e_rot = np.linalg.norm(scores(True) - exact)
    assert e_rot < 0.75 * e_plain
