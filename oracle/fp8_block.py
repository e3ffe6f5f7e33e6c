"""The per-rank block with FP8 operands, forward and backward, float64.

Test infrastructure (see the package header). The inputs are the
dequantised FP8 tensors the device consumes: x, W1, W2 from E4M3 codes and
dy from E5M2 codes, each decode(code) * scale_inv. The block is then the
plain one (column-parallel fc1, bias + GELU or the gated SwiGLU, row-parallel
fc2, its data and weight gradients -- Megatron-LM code tour, "The
Tensor-Parallel Primitives" and "The Transformer Stack"; FP8 through
Transformer Engine, concept note "Megatron-LM / Megatron-Core", "Key math /
How it works"), with the two tensors that the block itself produces and
feeds to a later product quantised on the way, at the scale the call is
given (delayed scaling, see oracle.fp8):

* the activation a (gelu(h), or silu(gate) * up for the gated block), to
  E4M3, before fc2 and the fc2 weight gradient;
* the gradient dH (dA * gelu'(h), or both halves [dA * up * silu'(gate) |
  dA * silu(gate)]), to E5M2 with one scale for the whole tensor, before the
  fc1 data and weight gradients and the bias gradient.

The gated block's h is [gate | up] along the features, as in oracle.block.

Everything else is float64 on those values: h = x W1^T + b1 is kept
exact and the activation, forward and backward, is taken of it (the plain
block's reading, with no storage rounding). The device stores h in bfloat16
and applies the activation to that stored value; the GPU tests bound the
effect of that rounding on each code they check rather than copying it here.
The value handed to the quantiser is fl32(fl32(v) * scale), which is the
scaling recipe's own definition (see oracle.fp8).

``round_bf16`` (float32 to bfloat16, round to nearest even) is a format
utility for the tests' validity windows; no result of the block uses it.
"""
from __future__ import annotations

import numpy as np

from .activations import gelu_tanh, gelu_tanh_grad, silu, silu_grad
from .fp8 import dequantize, quantize


def _inv(scale) -> np.float32:
    return np.float32(np.float32(1.0) / np.float32(scale))


def round_bf16(v) -> np.ndarray:
    """bfloat16 value of fl32(v), round to nearest even, as float64: the top
    16 bits of the float32 pattern after adding half of the dropped range
    (0x7fff, plus 1 when the kept part is odd). Finite inputs only."""
    b = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def _act(h, act: str):
    if act == "gelu":
        return gelu_tanh(h)
    if act == "swiglu":
        fs = h.shape[1] // 2
        return silu(h[:, :fs]) * h[:, fs:]
    raise ValueError(f"unknown activation {act!r}")


def rank_forward_fp8(x, W1, b1, W2, a_scale, act: str = "gelu") -> dict:
    """h = x W1^T + b1; a = gelu(h), or silu(gate) * up with h = [gate | up];
    a quantised to E4M3 at a_scale (codes, and a_q = decode(code) / a_scale);
    y = a_q W2^T. amax = max |a|. All float64 except the quantiser's float32
    product. "h_exact" is the same array as "h" (the name the tests bound
    the device's stored h against)."""
    h = x @ W1.T + (0.0 if b1 is None else b1)
    a = _act(h, act)
    codes = quantize(a, "e4m3", a_scale)
    a_q = dequantize(codes, "e4m3", _inv(a_scale))
    y = a_q @ W2.T
    amax = float(np.max(np.abs(a))) if a.size else 0.0
    return {"h_exact": h, "h": h, "a": a, "a_codes": codes, "a_q": a_q, "y": y,
            "amax": amax}


def rank_dgrad_fp8(dy, W1, W2, h, dH_scale, act: str = "gelu") -> dict:
    """dA = dy W2; dH = dA * gelu'(h), or [dA * up * silu'(gate) |
    dA * silu(gate)] (h as given: the forward's exact h); dH quantised to
    E5M2 at dH_scale (codes, and dH_q); dx = dH_q W1. amax = max |dH|."""
    dA = dy @ W2
    if act == "gelu":
        dH = dA * gelu_tanh_grad(h)
    elif act == "swiglu":
        fs = h.shape[1] // 2
        gate, up = h[:, :fs], h[:, fs:]
        dH = np.concatenate([dA * up * silu_grad(gate), dA * silu(gate)], axis=1)
    else:
        raise ValueError(f"unknown activation {act!r}")
    codes = quantize(dH, "e5m2", dH_scale)
    dH_q = dequantize(codes, "e5m2", _inv(dH_scale))
    dx = dH_q @ W1
    amax = float(np.max(np.abs(dH))) if dH.size else 0.0
    return {"dA": dA, "dH": dH, "dH_codes": codes, "dH_q": dH_q, "dx": dx, "amax": amax}


def rank_wgrad_fp8(dy, x, a_q, dH_q, dW1_in=None, db1_in=None, dW2_in=None) -> dict:
    """dW2 = dy^T a_q; dW1 = dH_q^T x; db1 = column sums of dH_q; each added
    to the given prior value when one is given (accumulation)."""
    dW2 = dy.T @ a_q
    dW1 = dH_q.T @ x
    db1 = dH_q.sum(axis=0)
    if dW2_in is not None:
        dW2 = np.asarray(dW2_in, dtype=np.float64) + dW2
    if dW1_in is not None:
        dW1 = np.asarray(dW1_in, dtype=np.float64) + dW1
    if db1_in is not None:
        db1 = np.asarray(db1_in, dtype=np.float64) + db1
    return {"dW1": dW1, "db1": db1, "dW2": dW2}
