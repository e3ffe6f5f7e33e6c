"""CPU pins of the attention-projection oracle (oracle.attention).

* The whole attention block sharded by heads over tp ranks -- packed QKV
  projection, core attention per rank, output projection partial sums --
  adds up to the unsharded block (the column->row pairing is exact), with and
  without grouped queries; a shard that pairs query heads with another
  group's key/value heads breaks it (negative control).
* The core attention used to state the block is torch's scaled dot-product
  attention (float64, causal).
* The per-rank gradients of both projections, assembled over the ranks, are
  torch autograd's gradients of the unsharded block, and finite differences
  of the block's loss confirm a sample of them.
"""
import numpy as np
import pytest
import torch

from oracle import attention as oa


def _weights(rng, H, nq, nkv, hn, bias=True):
    Wq = rng.standard_normal((nq * hn, H)) * 0.3
    Wk = rng.standard_normal((nkv * hn, H)) * 0.3
    Wv = rng.standard_normal((nkv * hn, H)) * 0.3
    Wo = rng.standard_normal((H, nq * hn)) * 0.3
    if bias:
        bq, bk, bv = (rng.standard_normal(n) * 0.2 for n in (nq * hn, nkv * hn, nkv * hn))
    else:
        bq = bk = bv = None
    return Wq, Wk, Wv, bq, bk, bv, Wo


def _unsharded(x, Wq, Wk, Wv, bq, bk, bv, Wo, nq, nkv, hn, batch):
    add = lambda y, b: y if b is None else y + b
    q, k, v = add(x @ Wq.T, bq), add(x @ Wk.T, bk), add(x @ Wv.T, bv)
    return oa.core_attention(q, k, v, nq, nkv, hn, batch) @ Wo.T


def _sharded(x, ws, nq, nkv, hn, tp, batch, shard=oa.shard_attn_rank):
    y = 0.0
    for r in range(tp):
        Wqkv, bqkv, Wo_r = shard(*ws, nq, nkv, hn, tp, r)
        q, k, v = oa.split_qkv(oa.qkv_forward(x, Wqkv, bqkv), nq // tp, nkv // tp, hn)
        y = y + oa.out_forward(oa.core_attention(q, k, v, nq // tp, nkv // tp, hn, batch), Wo_r)
    return y


@pytest.mark.parametrize("nq,nkv,tp", [(8, 8, 1), (8, 8, 2), (8, 8, 4), (8, 4, 2), (8, 4, 4),
                                       (8, 2, 2), (6, 3, 3)])
@pytest.mark.parametrize("bias", [True, False])
def test_block_shard_sum_invariant(nq, nkv, tp, bias):
    rng = np.random.default_rng(nq * 100 + nkv * 10 + tp)
    batch, S, H, hn = 2, 5, 24, 4
    x = rng.standard_normal((batch * S, H))
    ws = _weights(rng, H, nq, nkv, hn, bias)
    want = _unsharded(x, *ws, nq, nkv, hn, batch)
    got = _sharded(x, ws, nq, nkv, hn, tp, batch)
    assert np.allclose(got, want, rtol=0, atol=1e-12 * np.max(np.abs(want)))


def test_wrong_group_pairing_breaks_invariant():
    """Rank r taking the key/value heads of rank (r+1) % tp pairs its query
    heads with another group: the sum no longer matches."""
    rng = np.random.default_rng(3)
    nq, nkv, tp, batch, S, H, hn = 8, 4, 2, 1, 6, 16, 4
    x = rng.standard_normal((batch * S, H))
    ws = _weights(rng, H, nq, nkv, hn)

    def bad(Wq, Wk, Wv, bq, bk, bv, Wo, nq, nkv, hn, tp, r):
        Wqkv, bqkv, Wo_r = oa.shard_attn_rank(Wq, Wk, Wv, bq, bk, bv, Wo, nq, nkv, hn, tp, r)
        W2, b2, _ = oa.shard_attn_rank(Wq, Wk, Wv, bq, bk, bv, Wo, nq, nkv, hn, tp, (r + 1) % tp)
        a = nq // tp * hn
        return (np.concatenate([Wqkv[:a], W2[a:]]), np.concatenate([bqkv[:a], b2[a:]]), Wo_r)

    want = _unsharded(x, *ws, nq, nkv, hn, batch)
    assert np.allclose(_sharded(x, ws, nq, nkv, hn, tp, batch), want, atol=1e-12)
    assert not np.allclose(_sharded(x, ws, nq, nkv, hn, tp, batch, shard=bad), want, atol=1e-3)


@pytest.mark.parametrize("nq,nkv", [(4, 4), (4, 2), (6, 1)])
def test_core_attention_is_torch_sdpa(nq, nkv):
    rng = np.random.default_rng(nq + 7 * nkv)
    batch, S, hn = 3, 7, 8
    q = rng.standard_normal((batch * S, nq * hn))
    k = rng.standard_normal((batch * S, nkv * hn))
    v = rng.standard_normal((batch * S, nkv * hn))
    got = oa.core_attention(q, k, v, nq, nkv, hn, batch)
    tq = torch.from_numpy(q).view(batch, S, nq, hn).transpose(1, 2)
    tk = torch.from_numpy(k).view(batch, S, nkv, hn).transpose(1, 2)
    tv = torch.from_numpy(v).view(batch, S, nkv, hn).transpose(1, 2)
    tk = tk.repeat_interleave(nq // nkv, dim=1)
    tv = tv.repeat_interleave(nq // nkv, dim=1)
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    want = want.transpose(1, 2).reshape(batch * S, nq * hn).numpy()
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def _torch_block(x, ws, nq, nkv, hn, batch, dy):
    """Unsharded block in torch float64 with autograd; returns the grads."""
    t = [None if w is None else torch.tensor(w, requires_grad=True) for w in (x,) + tuple(ws)]
    tx, tWq, tWk, tWv, tbq, tbk, tbv, tWo = t
    lin = lambda a, W, b: a @ W.T + (0 if b is None else b)
    T = x.shape[0]
    S = T // batch
    sh = lambda a, n: a.view(batch, S, n, hn).transpose(1, 2)
    q, k, v = sh(lin(tx, tWq, tbq), nq), sh(lin(tx, tWk, tbk), nkv), sh(lin(tx, tWv, tbv), nkv)
    k = k.repeat_interleave(nq // nkv, dim=1)
    v = v.repeat_interleave(nq // nkv, dim=1)
    ctx = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    ctx = ctx.transpose(1, 2).reshape(T, nq * hn)
    y = ctx @ tWo.T
    (y * torch.from_numpy(dy)).sum().backward()
    return {n: (None if a is None else a.grad.numpy())
            for n, a in zip(("x", "Wq", "Wk", "Wv", "bq", "bk", "bv", "Wo"), t)}


def _oracle_grads(x, ws, nq, nkv, hn, tp, batch, dy):
    """Per-rank projection gradients from the oracle, assembled over ranks.
    The core attention's own backward (outside the projections) comes from
    torch autograd on each rank's q, k, v."""
    H = x.shape[1]
    nq_r, nkv_r = nq // tp, nkv // tp
    dx = np.zeros_like(x)
    dWq, dWk, dWv = np.zeros((nq * hn, H)), np.zeros((nkv * hn, H)), np.zeros((nkv * hn, H))
    dbq, dbk, dbv = np.zeros(nq * hn), np.zeros(nkv * hn), np.zeros(nkv * hn)
    dWo = np.zeros((H, nq * hn))
    T, S = x.shape[0], x.shape[0] // batch
    for r in range(tp):
        Wqkv, bqkv, Wo_r = oa.shard_attn_rank(*ws, nq, nkv, hn, tp, r)
        qkv = oa.qkv_forward(x, Wqkv, bqkv)
        q, k, v = oa.split_qkv(qkv, nq_r, nkv_r, hn)
        ctx = oa.core_attention(q, k, v, nq_r, nkv_r, hn, batch)
        dctx = oa.out_dgrad(dy, Wo_r)
        dWo_r = oa.out_wgrad(dy, ctx)
        # core attention backward by autograd on this rank's heads
        tqkv = torch.tensor(qkv, requires_grad=True)
        tq, tk, tv = oa.split_qkv(tqkv, nq_r, nkv_r, hn)
        sh = lambda a, n: a.reshape(batch, S, n, hn).transpose(1, 2)
        kk = sh(tk, nkv_r).repeat_interleave(nq_r // nkv_r, dim=1)
        vv = sh(tv, nkv_r).repeat_interleave(nq_r // nkv_r, dim=1)
        c = torch.nn.functional.scaled_dot_product_attention(sh(tq, nq_r), kk, vv, is_causal=True)
        c = c.transpose(1, 2).reshape(T, nq_r * hn)
        (c * torch.from_numpy(dctx)).sum().backward()
        dqkv = tqkv.grad.numpy()
        dx += oa.qkv_dgrad(dqkv, Wqkv)
        dW, db = oa.qkv_wgrad(dqkv, x, has_bias=bqkv is not None)
        a, b = nq_r * hn, (nq_r + nkv_r) * hn
        qs = slice(r * a, (r + 1) * a)
        ks = slice(r * nkv_r * hn, (r + 1) * nkv_r * hn)
        dWq[qs], dWk[ks], dWv[ks] = dW[:a], dW[a:b], dW[b:]
        if db is not None:
            dbq[qs], dbk[ks], dbv[ks] = db[:a], db[a:b], db[b:]
        dWo[:, qs] = dWo_r
    return {"x": dx, "Wq": dWq, "Wk": dWk, "Wv": dWv, "bq": dbq, "bk": dbk, "bv": dbv, "Wo": dWo}


@pytest.mark.parametrize("nq,nkv,tp", [(4, 4, 2), (8, 2, 2), (4, 4, 4), (6, 3, 3)])
def test_projection_gradients_match_autograd_of_the_block(nq, nkv, tp):
    rng = np.random.default_rng(11 * nq + nkv + tp)
    batch, S, H, hn = 2, 4, 12, 4
    x = rng.standard_normal((batch * S, H))
    ws = _weights(rng, H, nq, nkv, hn)
    dy = rng.standard_normal((batch * S, H))
    want = _torch_block(x, ws, nq, nkv, hn, batch, dy)
    got = _oracle_grads(x, ws, nq, nkv, hn, tp, batch, dy)
    for k in want:
        assert np.allclose(got[k], want[k], rtol=1e-10, atol=1e-12), k


def test_finite_differences_of_the_block_loss():
    """L = sum(dy * y) of the sharded block: central differences (eps 1e-6)
    at sampled entries of every input agree with the assembled gradients."""
    rng = np.random.default_rng(21)
    nq, nkv, tp, batch, S, H, hn = 4, 2, 2, 2, 3, 6, 3
    x = rng.standard_normal((batch * S, H))
    ws = list(_weights(rng, H, nq, nkv, hn))
    dy = rng.standard_normal((batch * S, H))
    g = _oracle_grads(x, ws, nq, nkv, hn, tp, batch, dy)
    names = ("Wq", "Wk", "Wv", "bq", "bk", "bv", "Wo")

    def loss(xx, wws):
        return float(np.sum(dy * _sharded(xx, wws, nq, nkv, hn, tp, batch)))

    eps = 1e-6
    for n, arr in [("x", x)] + list(zip(names, ws)):
        flat = arr.reshape(-1)
        for idx in rng.choice(flat.size, size=min(6, flat.size), replace=False):
            old = flat[idx]
            flat[idx] = old + eps
            lp = loss(x, ws)
            flat[idx] = old - eps
            lm = loss(x, ws)
            flat[idx] = old
            fd = (lp - lm) / (2 * eps)
            an = g[n].reshape(-1)[idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (n, idx, fd, an)
