"""The seeded input recipe against what the pages report of real inputs.

The peaked structure stands in for the captured model layer the pages
measure on; the one statistic the pages give for that layer is the share of
(row, 64-key block) pairs whose largest probability lies more than 8 binades
below the row maximum (the blocks per-block scaling exists for). The
Gaussian benchmark inputs have almost none.
"""
import math

import numpy as np
import pytest

import oracle
from fp8_bf16_causal_amd import synth


def far_block_share(name, n_rows, seed=0):
    inp = synth.make_config(name)
    p = inp.shape
    dq, dk, _ = inp.descale
    q = oracle.dequantize(synth.raw_codes(inp.q), oracle.FP8_E4M3, dq)
    k = oracle.dequantize(synth.raw_codes(inp.k), oracle.FP8_E4M3, dk)
    G = p["Hq"] // p["Hkv"]
    rng = np.random.default_rng(seed)
    far = tot = 0
    for _ in range(n_rows):
        h, i = int(rng.integers(p["Hq"])), int(rng.integers(256, p["S"]))
        t = (k[0, :i + 1, h // G, :] @ q[0, i, h, :]) * inp.scale * math.log2(math.e)
        t -= t.max()
        nb = (i + 1 + 63) // 64
        bm = np.maximum.reduceat(t, np.arange(0, 64 * nb, 64))
        far += int(np.sum(bm < -8.0))
        tot += nb
    return far / tot


def test_peaked_inputs_reproduce_the_pages_far_block_share(golden):
    share = far_block_share("fp8_gqa_s16k_peaked", 96)
    target = golden["far_block_share_real_layer"]["value"]
    print(f"peaked far-block share {share:.3f} (pages, real layer: {target})")
    assert abs(share - target) < 0.04


def test_gaussian_inputs_have_almost_no_far_blocks():
    assert far_block_share("fp8_mha_s32k", 24) < 0.01
