"""The per-rank column->row MLP block, forward and backward, float64.

Test infrastructure (see the package header). Notation: T tokens, H hidden,
F unsharded intermediate size, tp the tensor-parallel degree, Fs = F/tp, and
G = 2 for the gated block (gate and up halves), 1 otherwise. Weights follow
the [out, in] convention: W1 [G*F, H] unsharded, [G*Fs, H] per rank;
W2 [H, F] unsharded, [H, Fs] per rank.

Pages followed:

* Column-parallel fc1 splits its weight along the output dimension, so each
  rank computes a slice of the output features from the full input; the
  row-parallel fc2 splits along its input dimension and returns a partial sum
  that is all-reduced afterwards; chaining the two needs one all-reduce per
  block -- Megatron-LM code tour (pyshine.com), "The Tensor-Parallel
  Primitives"; concept note "Megatron-LM / Megatron-Core", "Key math / How it
  works" (the f/g conjugate operators).
* The block is fc1, a fused GELU, fc2; gated variants multiply an activated
  gate by a second projection -- code tour, "The Transformer Stack".
* Weight-gradient accumulation is a separate step from the data gradient --
  code tour, "The Tensor-Parallel Primitives".

Readings where the pages are silent: the bias is added to fc1's output
before the activation and the saved pre-activation h includes it; fc2's bias
is outside the per-rank partial sum (it is added once after the all-reduce);
for the gated block the first Fs columns of fc1's per-rank output are the
gate (activated with SiLU) and the second Fs columns the up projection, each
rank holding the matching gate and up blocks.
"""
from __future__ import annotations

import numpy as np

from .activations import gelu_tanh, gelu_tanh_grad, silu, silu_grad


def to_f64(t):
    """A torch tensor or array-like as a float64 NumPy array (exact widening)."""
    if t is None:
        return None
    if hasattr(t, "detach"):
        import torch
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def _check_act(act: str) -> int:
    if act == "gelu":
        return 1
    if act == "swiglu":
        return 2
    raise ValueError(f"unknown activation {act!r}")


def shard_rank(W1, b1, W2, tp: int, r: int, act: str):
    """Rank r's shard of unsharded weights, contiguous blocks.

    fc1 (column-parallel): output features [r*Fs, (r+1)*Fs); for the gated
    block the gate rows [r*Fs, (r+1)*Fs) and the up rows F + [r*Fs, (r+1)*Fs)
    are stacked gate first. fc2 (row-parallel): input features
    [r*Fs, (r+1)*Fs), i.e. a block of W2's columns.
    """
    g = _check_act(act)
    F = W2.shape[1]
    if F % tp != 0:
        raise ValueError("intermediate size must divide evenly by the TP degree")
    if W1.shape[0] != g * F:
        raise ValueError("W1 rows must be G*F")
    fs = F // tp
    idx = np.arange(r * fs, (r + 1) * fs)
    return select_features(W1, b1, W2, idx, act)


def select_features(W1, b1, W2, idx, act: str):
    """Restrict the block to the intermediate features ``idx`` (indices into
    [0, F) where F = W2.shape[1]). This is the column->row split applied to
    an arbitrary feature subset: fc1 rows (gate and up rows for the gated
    block), the matching bias entries and fc2 columns."""
    g = _check_act(act)
    idx = np.asarray(idx)
    F = W2.shape[1]
    if g == 2:
        rows = np.concatenate([idx, F + idx])
    else:
        rows = idx
    W1s = W1[rows]
    b1s = None if b1 is None else b1[rows]
    W2s = W2[:, idx]
    return W1s, b1s, W2s


def rank_forward(x, W1, b1, W2, act: str):
    """Forward of one rank: h = x W1^T (+ b1); a = act(h); y_partial = a W2^T.

    Returns dict with ``h`` (saved pre-activation, [T, G*Fs]), ``a`` ([T, Fs])
    and ``y`` (this rank's partial sum, [T, H])."""
    g = _check_act(act)
    x = to_f64(x)
    W1 = to_f64(W1)
    W2 = to_f64(W2)
    h = x @ W1.T
    if b1 is not None:
        h = h + to_f64(b1)[None, :]
    if g == 1:
        a = gelu_tanh(h)
    else:
        fs = W1.shape[0] // 2
        gate, up = h[:, :fs], h[:, fs:]
        a = silu(gate) * up
    y = a @ W2.T
    return {"h": h, "a": a, "y": y}


def rank_dgrad(dy, W1, W2, h, act: str):
    """Data gradient of one rank, given the replicated output gradient dy
    (g's backward is the identity).

    dA = dy W2; dH = dA * act'(h) (gated: [dA*u*silu'(g) | dA*silu(g)]);
    dx_partial = dH W1 (f's backward all-reduces it across ranks)."""
    g = _check_act(act)
    dy = to_f64(dy)
    W1 = to_f64(W1)
    W2 = to_f64(W2)
    h = to_f64(h)
    dA = dy @ W2
    if g == 1:
        dH = dA * gelu_tanh_grad(h)
    else:
        fs = W1.shape[0] // 2
        gate, up = h[:, :fs], h[:, fs:]
        dH = np.concatenate([dA * up * silu_grad(gate), dA * silu(gate)], axis=1)
    dx = dH @ W1
    return {"dA": dA, "dH": dH, "dx": dx}


def rank_wgrad(dy, x, a, dH, has_bias: bool, dW1_in=None, db1_in=None, dW2_in=None):
    """Weight gradients of one rank: dW2 = dy^T a, dW1 = dH^T x,
    db1 = sum over tokens of dH. With prior buffers given (accumulate mode)
    each result is ``prior + value``."""
    dy = to_f64(dy)
    x = to_f64(x)
    a = to_f64(a)
    dH = to_f64(dH)
    dW2 = dy.T @ a
    dW1 = dH.T @ x
    db1 = dH.sum(axis=0) if has_bias else None
    if dW2_in is not None:
        dW2 = to_f64(dW2_in) + dW2
    if dW1_in is not None:
        dW1 = to_f64(dW1_in) + dW1
    if db1 is not None and db1_in is not None:
        db1 = to_f64(db1_in) + db1
    return {"dW1": dW1, "db1": db1, "dW2": dW2}


def unsharded_forward(x, W1, b1, W2, act: str):
    """The whole block on one device (tp = 1): y = act(x W1^T + b1) W2^T."""
    return rank_forward(x, W1, b1, W2, act)


def unsharded_backward(x, W1, b1, W2, dy, act: str):
    """All gradients of the unsharded block for output gradient dy."""
    fwd = rank_forward(x, W1, b1, W2, act)
    dg = rank_dgrad(dy, W1, W2, fwd["h"], act)
    wg = rank_wgrad(dy, x, fwd["a"], dg["dH"], b1 is not None)
    return {"dx": dg["dx"], "dW1": wg["dW1"], "db1": wg["db1"], "dW2": wg["dW2"],
            "dH": dg["dH"], "h": fwd["h"], "a": fwd["a"], "y": fwd["y"]}


def block_loss(x, W1, b1, W2, dy, act: str) -> float:
    """Scalar L = sum(dy * y) whose gradients are the block's backward for dy."""
    y = rank_forward(x, W1, b1, W2, act)["y"]
    return float(np.sum(to_f64(dy) * y))
