"""Seeded synthetic inputs for causal prefill attention.

This module only draws and encodes inputs; it holds none of the attention
arithmetic. Both sides of every parity check (the HIP library and the CPU
oracle) receive the tensors it returns.

Recipe (the pages benchmark on Gaussian inputs and on attention inputs
captured from Mistral-7B, Qwen3-8B and DeepSeek-V2-Lite; the captures are not
available, so seeded inputs of the same shapes stand in for both):

* ``torch.Generator(device).manual_seed(seed)``; Q, K, V are drawn in that
  order with ``torch.randn`` as float32 in (batch, seq, heads, dim) layout.
* ``structure="peaked"`` (stand-in for a captured Mistral-7B layer): 4 channels
  picked by a seeded ``randperm`` of the head dim are multiplied by 8 in both Q
  and K (every head), and a fifth such channel carries an attention sink:
  Q[..., c] = 1 and K[:, 0, :, c] = 6 * sqrt(Dqk), which adds 6 (in units of
  scaled logits at the default scale) to every query's score with key 0.
* BF16 inputs: ``.to(torch.bfloat16)`` (round to nearest even).
* FP8 inputs: one factor per tensor, s = amax / 448 (s = 1 when amax = 0); the
  codes are ``(x / s).clamp(-448, 448).to(torch.float8_e4m3fn)`` (round to
  nearest even) and s is the tensor's dequantisation factor.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

E4M3_MAX = 448.0


@dataclass
class AttnInputs:
    q: torch.Tensor  # [B, S, Hq, Dqk], bfloat16 or float8_e4m3fn
    k: torch.Tensor  # [B, S, Hkv, Dqk]
    v: torch.Tensor  # [B, S, Hkv, Dv]
    dtype: str  # "bf16" or "fp8"
    scale: float  # softmax scale
    descale: tuple  # (dq, dk, dv) per-tensor dequantisation factors (1 for BF16)

    @property
    def shape(self):
        B, S, Hq, Dqk = self.q.shape
        return dict(B=B, S=S, Hq=Hq, Hkv=self.k.shape[2], Dqk=Dqk, Dv=self.v.shape[3])


# The workloads: (name -> parameters). The first is the small case used for
# whole-tensor parity; the others are the benchmark shapes.
CONFIGS = {
    "bf16_mha_s512": dict(dtype="bf16", B=1, Hq=2, Hkv=2, S=512, Dqk=128, Dv=128, structure="gaussian", seed=1),
    "fp8_gqa_s16k_peaked": dict(dtype="fp8", B=1, Hq=32, Hkv=8, S=16384, Dqk=128, Dv=128, structure="peaked",
                                seed=2),
    "fp8_mha_s32k": dict(dtype="fp8", B=1, Hq=32, Hkv=32, S=32768, Dqk=128, Dv=128, structure="gaussian", seed=3),
    "bf16_mha_s32k": dict(dtype="bf16", B=1, Hq=32, Hkv=32, S=32768, Dqk=128, Dv=128, structure="gaussian",
                          seed=4),
    "fp8_mla_s32k": dict(dtype="fp8", B=1, Hq=16, Hkv=16, S=32768, Dqk=192, Dv=128, structure="gaussian", seed=5),
}


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor e4m3fn quantisation: returns (codes, dequantisation factor)."""
    amax = float(x.abs().max()) if x.numel() else 0.0
    s = amax / E4M3_MAX if amax > 0 else 1.0
    codes = (x / s).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return codes, s


def make_inputs(B: int, S: int, Hq: int, Hkv: int, Dqk: int, Dv: int, dtype: str = "bf16", seed: int = 0,
                structure: str = "gaussian", scale: float | None = None, device="cpu") -> AttnInputs:
    if dtype not in ("bf16", "fp8"):
        raise ValueError(dtype)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    q = torch.randn((B, S, Hq, Dqk), generator=g, device=device, dtype=torch.float32)
    k = torch.randn((B, S, Hkv, Dqk), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((B, S, Hkv, Dv), generator=g, device=device, dtype=torch.float32)
    if structure == "peaked":
        ch = torch.randperm(Dqk, generator=torch.Generator().manual_seed(seed))[:5].tolist()
        for c in ch[:4]:
            q[..., c] *= 8.0
            k[..., c] *= 8.0
        cs = ch[4]
        q[..., cs] = 1.0
        k[:, 0, :, cs] = 6.0 * math.sqrt(Dqk)
    elif structure != "gaussian":
        raise ValueError(structure)
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    if dtype == "bf16":
        return AttnInputs(q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16), "bf16", scale,
                          (1.0, 1.0, 1.0))
    (qc, dq), (kc, dk), (vc, dv) = quantize_e4m3(q), quantize_e4m3(k), quantize_e4m3(v)
    return AttnInputs(qc, kc, vc, "fp8", scale, (dq, dk, dv))


def make_config(name: str, device="cpu", **override) -> AttnInputs:
    p = dict(CONFIGS[name])
    p.update(override)
    return make_inputs(**p, device=device)


def raw_codes(t: torch.Tensor):
    """The element codes of a bfloat16 / float8_e4m3fn tensor as a host numpy
    array (uint16 / uint8), the form the oracle reads."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view("uint16")
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    raise TypeError(t.dtype)
