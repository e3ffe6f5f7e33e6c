"""Expert MLPs of a mixture-of-experts layer over ragged token groups (one
rank's local experts), forward and backward, float64.

Test infrastructure (see the package header). Pages followed:

* Megatron-LM supports mixture-of-experts layers, which grow the parameter
  count while the compute per token stays fixed -- onegen.ai overview, "Key
  Features"; concept note "Megatron-LM / Megatron-Core", "Key math / How it
  works" (expert parallelism: all-to-all dispatch and combine, with the
  expert model-parallel and expert tensor-parallel sizes set separately).
* Each expert is the block of the MLP (column-parallel fc1, bias + GELU or
  SwiGLU, row-parallel fc2), so an expert's share on a rank is the per-rank
  block of ``oracle.block`` with its own weights.

Readings where the pages are silent:

* The dispatch (routing, the all-to-all, the permutation of tokens by
  expert) and the combine (un-permutation, weighting by the router's
  probabilities) are outside the expert computation: its input is the
  token rows already grouped by local expert, x_perm [T, H] with expert e
  owning rows [off_e, off_e + counts[e]), off_e = counts[0] + ... +
  counts[e-1], and its output rows y_perm follow the same grouping.
* Expert e's weights are W1[e] [G*Fs, H], b1[e] [G*Fs], W2[e] [H, Fs] (the
  per-rank shard of an expert under expert tensor parallelism). Weight
  gradients are per expert: dW1[e] sums over expert e's rows only.
"""
from __future__ import annotations

import numpy as np

from .block import rank_dgrad, rank_forward, rank_wgrad


def offsets(counts):
    """Start row of each expert's group (exclusive prefix sum of counts)."""
    c = np.asarray(counts, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(c)[:-1]]) if c.size else c


def _groups(counts):
    off = offsets(counts)
    return [(int(e), int(o), int(o + c)) for e, (o, c) in enumerate(zip(off, counts))]


def grouped_forward(x, counts, W1, b1, W2, act: str) -> dict:
    """Each expert's rows through its own block: h, a, y stacked in row order."""
    T = x.shape[0]
    G = 2 if act == "swiglu" else 1
    Fs = W2.shape[2]
    out = {"h": np.zeros((T, G * Fs)), "a": np.zeros((T, Fs)), "y": np.zeros((T, x.shape[1]))}
    for e, r0, r1 in _groups(counts):
        f = rank_forward(x[r0:r1], W1[e], None if b1 is None else b1[e], W2[e], act)
        for k in out:
            out[k][r0:r1] = f[k]
    return out


def grouped_dgrad(dy, counts, W1, W2, h, act: str) -> dict:
    """dH and dx_partial of each expert's rows."""
    T, H = dy.shape
    out = {"dH": np.zeros_like(h), "dx": np.zeros((T, H))}
    for e, r0, r1 in _groups(counts):
        g = rank_dgrad(dy[r0:r1], W1[e], W2[e], h[r0:r1], act)
        out["dH"][r0:r1] = g["dH"]
        out["dx"][r0:r1] = g["dx"]
    return out


def grouped_wgrad(dy, x, a, dH, counts, has_bias: bool, dW1_in=None, db1_in=None,
                  dW2_in=None) -> dict:
    """Per-expert dW1[e], db1[e], dW2[e] over the expert's rows only (added to
    the given prior values when given)."""
    E = len(counts)
    H, GFs, Fs = x.shape[1], dH.shape[1], a.shape[1]
    out = {"dW1": np.zeros((E, GFs, H)), "db1": np.zeros((E, GFs)) if has_bias else None,
           "dW2": np.zeros((E, H, Fs))}
    for e, r0, r1 in _groups(counts):
        w = rank_wgrad(dy[r0:r1], x[r0:r1], a[r0:r1], dH[r0:r1], has_bias,
                       None if dW1_in is None else dW1_in[e],
                       None if db1_in is None else db1_in[e],
                       None if dW2_in is None else dW2_in[e])
        out["dW1"][e] = w["dW1"]
        out["dW2"][e] = w["dW2"]
        if has_bias:
            out["db1"][e] = w["db1"]
    return out
