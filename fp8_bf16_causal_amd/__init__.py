"""MI355X (gfx950) causal prefill attention forward: FP8 e4m3 or BF16 inputs,
BF16 output, through the C-ABI library libfp8_bf16_causal.so.

``attn_fwd`` / ``attn_fwd_ex`` / ``attn_fwd_lse`` / ``attn_fwd_prefix`` /
``attn_quantize_e4m3`` / ``attn_strerror`` are the C entry points (device
addresses as ints); ``flash_attn_func`` and ``quantize_e4m3`` take torch
tensors. PyTorch only provides device memory and the stream.
"""
from __future__ import annotations

import math

from . import synth  # noqa: F401
from ._lib import (ATTN_BF16, ATTN_ERR_INVALID, ATTN_ERR_LAUNCH, ATTN_ERR_UNSUPPORTED, ATTN_FLAG_DESCALE_DEVICE,
                   ATTN_FLAG_EXACT_P, ATTN_FLAG_NO_BLOCKSCALE, ATTN_FP8_E4M3, ATTN_OK, attn_fwd, attn_fwd_ex,
                   attn_fwd_lse, attn_fwd_prefix, attn_quantize_e4m3, attn_strerror)

__all__ = ["attn_fwd", "attn_fwd_ex", "attn_fwd_lse", "attn_fwd_prefix", "attn_quantize_e4m3", "attn_strerror",
           "flash_attn_func", "quantize_e4m3", "ATTN_BF16", "ATTN_FP8_E4M3", "ATTN_OK", "ATTN_ERR_INVALID",
           "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_LAUNCH", "ATTN_FLAG_EXACT_P", "ATTN_FLAG_NO_BLOCKSCALE",
           "ATTN_FLAG_DESCALE_DEVICE", "flash_attn_fp8_func"]


def _raise(code: int):
    msg = attn_strerror(code)
    if code == ATTN_ERR_INVALID:
        raise ValueError(msg)
    if code == ATTN_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise RuntimeError(msg)


def _factor(x, name):
    """A per-tensor dequantisation factor: a number, or a one-element tensor
    (flash-attention's per-(batch, head) descale tensors are accepted only when
    they hold a single value)."""
    if x is None or isinstance(x, (int, float)):
        return x
    if hasattr(x, "numel"):
        if x.numel() != 1:
            raise ValueError(f"{name}: one factor per tensor (a number or a one-element tensor)")
        return float(x.reshape(-1)[0])
    return float(x)


def flash_attn_func(q, k, v, softmax_scale=None, causal=True, *, q_descale=None, k_descale=None, v_descale=None,
                    window_size=(-1, -1), softcap=0.0, alibi_slopes=None, deterministic=False, dropout_p=0.0,
                    descale_q=None, descale_k=None, descale_v=None, out=None, exact_p=False, block_scale=True,
                    return_lse=False, descale_device=None):
    """Causal prefill attention on torch tensors in (batch, seq, heads, dim)
    layout: bfloat16, or float8_e4m3fn with optional per-tensor dequantisation
    factors (ValueError for a factor other than 1 with bfloat16). Returns a
    new (or the given) bfloat16 tensor [B, S, Hq, Dv], enqueued on the
    current stream; with return_lse=True, also a float32
    tensor [B, Hq, S] of each row's log-sum-exp (attn_fwd_lse). k and v may be
    longer than q (Sk > Sq): the queries are then the last Sq positions and
    query i sees keys j <= i + Sk - Sq (attn_fwd_prefix). exact_p=True /
    block_scale=False select the FP8 softmax ablations (ATTN_FLAG_EXACT_P /
    ATTN_FLAG_NO_BLOCKSCALE). descale_device: instead of descale_q/k/v, a
    contiguous float32 tensor on q's device holding {dq, amax_q, dk, amax_k,
    dv, amax_v} (three quantize_e4m3 calls with scale_out=buf[0:2], buf[2:4],
    buf[4:6]), read by the kernels: no host round trip
    (ATTN_FLAG_DESCALE_DEVICE).

    The positional order (q, k, v, softmax_scale, causal) and the keywords
    q_descale / k_descale / v_descale, window_size, softcap, alibi_slopes,
    deterministic and dropout_p follow flash-attention's FP8-capable
    flash_attn_func. What the kernels do not implement raises
    NotImplementedError rather than returning something else: causal=False,
    a sliding window, a softcap, ALiBi slopes and dropout. causal defaults to
    True here, the only mode the method has (flash-attention's default is
    False: calls written for it that rely on that default must pass causal).
    q_descale etc. are aliases of descale_q etc. (one factor per tensor). The
    kernels are deterministic whatever `deterministic` says."""
    if dropout_p != 0.0:
        raise NotImplementedError("dropout is not supported (inference prefill forward only)")
    if softcap != 0.0 or alibi_slopes is not None:
        raise NotImplementedError("softcap and ALiBi slopes are not supported")
    if tuple(window_size) not in ((-1, -1), (-1, 0)) or (tuple(window_size) == (-1, 0) and not causal):
        raise NotImplementedError("sliding-window attention is not supported (window_size must be (-1, -1))")
    if not causal:
        raise NotImplementedError("only causal attention is implemented (pass causal=True)")
    for a, b, name in ((q_descale, descale_q, "q"), (k_descale, descale_k, "k"), (v_descale, descale_v, "v")):
        if a is not None and b is not None:
            raise ValueError(f"give {name}_descale or descale_{name}, not both")
    descale_q = _factor(descale_q if q_descale is None else q_descale, "q_descale")
    descale_k = _factor(descale_k if k_descale is None else k_descale, "k_descale")
    descale_v = _factor(descale_v if v_descale is None else v_descale, "v_descale")
    import torch

    if q.dtype == torch.bfloat16:
        dtype = ATTN_BF16
    elif q.dtype == torch.float8_e4m3fn:
        dtype = ATTN_FP8_E4M3
    else:
        raise TypeError(f"q must be bfloat16 or float8_e4m3fn, got {q.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must have the same dtype")
    if dtype == ATTN_BF16 and any(x is not None and float(x) != 1.0 for x in (descale_q, descale_k, descale_v)):
        # bfloat16 values are their own: a factor other than 1 would be silently ignored
        raise ValueError("descale_q/k/v apply to float8_e4m3fn inputs only (bfloat16 inputs take none, or 1.0)")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [batch, seq, heads, dim]")
    if not (q.is_cuda and k.is_cuda and v.is_cuda and q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, S, Hq, Dqk = q.shape
    Sk = k.shape[1]
    if k.shape[0] != B or Sk < S or v.shape[:3] != k.shape[:3] or k.shape[3] != Dqk:
        raise ValueError("shape mismatch between q, k and v")
    Hkv, Dv = k.shape[2], v.shape[3]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(Dqk)
    if out is None:
        out = torch.empty((B, S, Hq, Dv), dtype=torch.bfloat16, device=q.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (B, S, Hq, Dv) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 [B, S, Hq, Dv] tensor")
    ds = None
    if dtype == ATTN_FP8_E4M3 and any(x is not None for x in (descale_q, descale_k, descale_v)):
        ds = tuple(1.0 if x is None else float(x) for x in (descale_q, descale_k, descale_v))
    flags = (ATTN_FLAG_EXACT_P if exact_p else 0) | (0 if block_scale else ATTN_FLAG_NO_BLOCKSCALE)
    if descale_device is not None:
        if dtype != ATTN_FP8_E4M3 or ds is not None:
            raise ValueError("descale_device goes with float8_e4m3fn inputs and no descale_q/k/v")
        if (descale_device.dtype != torch.float32 or descale_device.device != q.device
                or not descale_device.is_contiguous() or descale_device.numel() < 5):
            raise ValueError("descale_device must be a contiguous float32 tensor on q's device holding at least "
                             "{dq, amax_q, dk, amax_k, dv} (the kernels read elements 0, 2 and 4)")
        ds = descale_device.data_ptr()
        flags |= ATTN_FLAG_DESCALE_DEVICE
    stream = torch.cuda.current_stream(q.device).cuda_stream
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device) if return_lse else None
    with torch.cuda.device(q.device):
        if Sk != S:
            rc = attn_fwd_prefix(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr() if return_lse else None, B, Hq, Hkv, S, Sk, Dqk, Dv, 1 if causal else 0,
                                 float(softmax_scale), dtype, ds, stream, flags)
        elif return_lse:
            rc = attn_fwd_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv,
                              S, Dqk, Dv, 1 if causal else 0, float(softmax_scale), dtype, ds, stream, flags)
        else:
            rc = attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, S, Dqk, Dv,
                             1 if causal else 0, float(softmax_scale), dtype, ds, stream, flags)
    if rc != ATTN_OK:
        _raise(rc)
    return (out, lse) if return_lse else out


def quantize_e4m3(x, hadamard=False, scale_out=None):
    """Per-tensor e4m3fn quantisation of a bfloat16 tensor [..., dim] on the
    GPU (dim 64, 128, 192 or 256), optionally rotating each row by a Hadamard
    transform first (for Q and K). Returns (codes as float8_e4m3fn, a device
    float32 tensor [s, amax]); attn_fwd takes the codes with descale s.
    scale_out: optional contiguous float32 device tensor of 2 values to write
    [s, amax] into (e.g. a slice of flash_attn_func's descale_device buffer).
    Enqueued on the current stream."""
    import torch

    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous() or x.dim() < 1:
        raise ValueError("x must be a contiguous bfloat16 GPU tensor")
    dim = x.shape[-1]
    rows = x.numel() // dim if dim else 0
    y = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device)
    if scale_out is None:
        scale = torch.empty(2, dtype=torch.float32, device=x.device)
    else:
        if (scale_out.dtype != torch.float32 or scale_out.device != x.device or not scale_out.is_contiguous()
                or scale_out.numel() != 2):
            raise ValueError("scale_out must be a contiguous float32 tensor of 2 values on x's device")
        scale = scale_out
    stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device):
        rc = attn_quantize_e4m3(x.data_ptr(), y.data_ptr(), scale.data_ptr(), rows, dim, 1 if hadamard else 0, stream)
    if rc != ATTN_OK:
        _raise(rc)
    return y, scale


def flash_attn_fp8_func(q, k, v, softmax_scale=None, causal=True, hadamard=True, out=None, return_lse=False,
                        exact_p=False, block_scale=True):
    """FP8 prefill from bfloat16 tensors in one call: Q and K quantised to
    e4m3fn with the Hadamard rotation (hadamard=True, the default; one
    orthogonal rotation on both leaves Q K^T unchanged) and V without, each
    with its own per-tensor factor, then the FP8 attention reading those
    factors on the device (ATTN_FLAG_DESCALE_DEVICE): four launches on the
    current stream, no host synchronisation. Returns what flash_attn_func
    returns. The codes and factors are temporaries of this call; use
    quantize_e4m3 and flash_attn_func(descale_device=...) to keep them."""
    import torch

    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("flash_attn_fp8_func takes bfloat16 q, k and v")
    buf = torch.empty(6, dtype=torch.float32, device=q.device)
    q8, _ = quantize_e4m3(q, hadamard=hadamard, scale_out=buf[0:2])
    k8, _ = quantize_e4m3(k, hadamard=hadamard, scale_out=buf[2:4])
    v8, _ = quantize_e4m3(v, hadamard=False, scale_out=buf[4:6])
    return flash_attn_func(q8, k8, v8, softmax_scale, causal, out=out, return_lse=return_lse, exact_p=exact_p,
                           block_scale=block_scale, descale_device=buf)
