"""The per-rank attention projections (packed QKV column-parallel, output
row-parallel), forward and backward, float64.

Test infrastructure (see the package header). Pages followed:

* SelfAttention builds one packed QKV projection that is column-parallel and
  an output projection that is row-parallel, through the same parallel
  linear layers as the MLP; the core attention math is delegated to fused
  backends -- Megatron-LM code tour (pyshine.com), "The Transformer Stack"
  and its key-symbol list (SelfAttention).
* Tensor parallelism splits multi-head attention by heads, and the hidden
  size and the number of attention heads must both divide by the TP degree;
  column into row needs one all-reduce per attention block -- concept note
  "Megatron-LM / Megatron-Core", "Key math / How it works"; code tour, "The
  Tensor-Parallel Primitives".

Notation: T tokens, H hidden, hn the head size, nq query heads and nkv
key/value heads (nkv = nq without grouped queries; query head j uses
key/value head j // (nq / nkv)), tp the TP degree, nq_r = nq / tp and
nkv_r = nkv / tp per rank. Unsharded weights use the [out, in] convention:
Wq [nq*hn, H], Wk and Wv [nkv*hn, H], Wo [H, nq*hn].

Readings where the pages are silent:

* Rank r holds query heads [r*nq_r, (r+1)*nq_r) and key/value heads
  [r*nkv_r, (r+1)*nkv_r) (contiguous blocks, as for the MLP), which keeps
  every query head on the rank of its key/value head.
* The per-rank packed weight stacks the rank's rows as [Wq rows; Wk rows;
  Wv rows] (likewise the bias), so the projection's output row for a token is
  [q heads | k heads | v heads]: q, k and v are column ranges of one
  [T, (nq_r + 2 nkv_r) hn] tensor, each [T, heads, hn] with the head size
  contiguous. Megatron orders the packed rows by query group instead; that
  is a fixed permutation of rows, applied once to a checkpoint's weights.
* The QKV projection has a bias (Megatron's default linear layers); the
  output projection's bias is added once after the all-reduce, outside the
  per-rank partial sum, as for fc2.
* The core attention (not part of the per-rank projections; here only to
  state the block the projections belong to) is causal softmax attention
  with scale 1/sqrt(hn), tokens ordered batch-major (t = b*S + s).
"""
from __future__ import annotations

import numpy as np


def _check(nq: int, nkv: int, tp: int):
    if nq % nkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    if nq % tp or nkv % tp:
        raise ValueError("heads must divide by the TP degree")


def shard_attn_rank(Wq, Wk, Wv, bq, bk, bv, Wo, nq: int, nkv: int, hn: int, tp: int, r: int):
    """Rank r's (Wqkv [(nq_r + 2 nkv_r) hn, H], bqkv or None, Wo_r [H, nq_r hn])."""
    _check(nq, nkv, tp)
    nq_r, nkv_r = nq // tp, nkv // tp
    qs = slice(r * nq_r * hn, (r + 1) * nq_r * hn)
    ks = slice(r * nkv_r * hn, (r + 1) * nkv_r * hn)
    Wqkv = np.concatenate([Wq[qs], Wk[ks], Wv[ks]], axis=0)
    bqkv = None if bq is None else np.concatenate([bq[qs], bk[ks], bv[ks]])
    return Wqkv, bqkv, Wo[:, qs]


def split_qkv(qkv, nq_r: int, nkv_r: int, hn: int):
    """Column ranges q [T, nq_r hn], k and v [T, nkv_r hn] of the packed output."""
    a, b = nq_r * hn, (nq_r + nkv_r) * hn
    return qkv[:, :a], qkv[:, a:b], qkv[:, b:]


def qkv_forward(x, Wqkv, bqkv=None):
    """qkv = x Wqkv^T (+ bqkv): the column-parallel packed projection."""
    y = x @ Wqkv.T
    return y if bqkv is None else y + bqkv


def out_forward(ctx, Wo_r):
    """y_partial = ctx Wo_r^T: the row-parallel output projection's partial sum."""
    return ctx @ Wo_r.T


def out_dgrad(dy, Wo_r):
    """d ctx = dy Wo_r (dy replicated on every rank)."""
    return dy @ Wo_r


def out_wgrad(dy, ctx, dWo_in=None):
    """dWo_r (+)= dy^T ctx."""
    d = dy.T @ ctx
    return d if dWo_in is None else np.asarray(dWo_in, dtype=np.float64) + d


def qkv_dgrad(dqkv, Wqkv):
    """dx_partial = dqkv Wqkv (summed over ranks by the f backward all-reduce)."""
    return dqkv @ Wqkv


def qkv_wgrad(dqkv, x, dW_in=None, db_in=None, has_bias=True):
    """dWqkv (+)= dqkv^T x; dbqkv (+)= column sums of dqkv."""
    dW = dqkv.T @ x
    if dW_in is not None:
        dW = np.asarray(dW_in, dtype=np.float64) + dW
    db = None
    if has_bias:
        db = dqkv.sum(axis=0)
        if db_in is not None:
            db = np.asarray(db_in, dtype=np.float64) + db
    return dW, db


def core_attention(q, k, v, nq: int, nkv: int, hn: int, batch: int):
    """Causal softmax attention per sequence and query head, scale 1/sqrt(hn);
    q [T, nq hn], k and v [T, nkv hn], T = batch * S tokens batch-major;
    returns ctx [T, nq hn]."""
    T = q.shape[0]
    S = T // batch
    grp = nq // nkv
    ctx = np.zeros((T, nq * hn))
    mask = np.triu(np.ones((S, S), dtype=bool), 1)
    for b in range(batch):
        rows = slice(b * S, (b + 1) * S)
        for j in range(nq):
            c = j // grp
            qj = q[rows, j * hn:(j + 1) * hn]
            kj = k[rows, c * hn:(c + 1) * hn]
            vj = v[rows, c * hn:(c + 1) * hn]
            s = (qj @ kj.T) / np.sqrt(hn)
            s[mask] = -np.inf
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            ctx[rows, j * hn:(j + 1) * hn] = p @ vj
    return ctx
