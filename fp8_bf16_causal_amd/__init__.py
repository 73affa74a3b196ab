"""MI355X (gfx950) causal prefill attention forward, FP8 e4m3 and BF16 inputs, BF16 output."""
from . import synth  # noqa: F401
