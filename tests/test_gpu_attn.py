"""GPU parity of the attention projections (tpmlp_attn_*) through the C ABI
against the oracle's per-rank projections (oracle.attention) on the same
seeded inputs, max|gpu - oracle| / max|oracle| within 2e-2 (bf16) or 1e-5
(fp32) per output tensor.

* Small and ragged shapes (T, H, heads and head size not multiples of the
  256 x 256 tile), grouped and ungrouped queries, with and without the QKV
  bias, and the accumulate mode of both weight gradients.
* The whole attention block at fp32, sharded over two simulated ranks on the
  GPU (the library's projections around torch's own attention on the
  device), summed over ranks and compared with the unsharded block of the
  oracle: the column->row pairing is exact, forward and backward.
* The full per-rank shapes (the 1024-hidden example model at TP 2 and the
  8192-hidden model at TP 8) on sampled rows, features and columns.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import attention as oa
from _gpu_helpers import TOL, rel_err, require_gpu, say, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("qkv", "y", "dctx", "dWo", "dx", "dWqkv", "dbqkv")


@pytest.fixture(scope="module")
def tp():
    require_gpu()
    import tensor_transformer_mlp_rank_amd as m
    return m


def _gpu_attn(tp, inp, nq, nkv, hn, dtype, has_bias, prior=None):
    T, H = inp["x"].shape
    desc = tp.make_attn_desc(T, H, nq, nkv, hn, dtype=dtype, has_bias=has_bias)
    say(f"  attn dtype={dtype} T={T} H={H} nq={nq} nkv={nkv} hn={hn} bias={has_bias} "
        f"accumulate={prior is not None}")
    dv = to_dev(inp)
    qkv, q, k, v = tp.attn_qkv_fwd(desc, dv["x"], dv["Wqkv"], dv["bqkv"] if has_bias else None)
    y = tp.attn_out_fwd(desc, dv["ctx"], dv["Wo"])
    pr = {} if prior is None else to_dev(prior)
    dctx, dWo = tp.attn_out_bwd(desc, dv["dy"], dv["Wo"], dv["ctx"], dWo=pr.get("dWo"))
    dx, dWqkv, dbqkv = tp.attn_qkv_bwd(desc, dv["dqkv"], dv["Wqkv"], dv["x"],
                                       dWqkv=pr.get("dWqkv"), dbqkv=pr.get("dbqkv"))
    torch.cuda.synchronize()
    out = dict(qkv=qkv, q=q, k=k, v=v, y=y, dctx=dctx, dWo=dWo, dx=dx, dWqkv=dWqkv, dbqkv=dbqkv)
    return {n: (None if t is None else t.cpu()) for n, t in out.items()}


def _oracle_attn(inp, nq, nkv, hn, has_bias, prior=None):
    f = oracle.to_f64
    x, W, Wo, dy, ctx, dqkv = (f(inp[n]) for n in ("x", "Wqkv", "Wo", "dy", "ctx", "dqkv"))
    b = f(inp["bqkv"]) if has_bias else None
    p = {} if prior is None else {n: f(t) for n, t in prior.items()}
    qkv = oa.qkv_forward(x, W, b)
    q, k, v = oa.split_qkv(qkv, nq, nkv, hn)
    dWqkv, dbqkv = oa.qkv_wgrad(dqkv, x, p.get("dWqkv"), p.get("dbqkv"), has_bias=has_bias)
    return dict(qkv=qkv, q=q, k=k, v=v, y=oa.out_forward(ctx, Wo), dctx=oa.out_dgrad(dy, Wo),
                dWo=oa.out_wgrad(dy, ctx, p.get("dWo")), dx=oa.qkv_dgrad(dqkv, W),
                dWqkv=dWqkv, dbqkv=dbqkv)


def _check(got, ref, tol, names=NAMES + ("q", "k", "v")):
    errs = {n: rel_err(got[n], ref[n]) for n in names if ref.get(n) is not None}
    say("    rel errors " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"tolerance {tol} exceeded: {bad}"


@pytest.mark.parametrize("T,H,nq,nkv,hn,bias", [
    (300, 528, 4, 2, 64, True), (37, 48, 2, 1, 16, False), (513, 1040, 6, 3, 32, True),
    (1, 64, 1, 1, 16, True), (4096, 1024, 8, 8, 64, True), (260, 272, 3, 3, 128, False),
    # the widest hidden size the calls accept (2^21), and the widest q|k|v
    # (3 x 699040 = 2^21 - 32 features; K = 699040 for the out-projection)
    (32, 1 << 21, 1, 1, 16, True), (16, 64, 1, 1, 699040, False),
])
def test_attn_small_and_ragged(tp, T, H, nq, nkv, hn, bias):
    w = synth.ATTN_WORKLOADS[6]
    inp = synth.make_attn_inputs(w, tokens=T, hidden=H, q_heads=nq, kv_heads=nkv, head_dim=hn,
                                 seed_base=600 + T)
    got = _gpu_attn(tp, inp, nq, nkv, hn, "bf16", bias)
    _check(got, _oracle_attn(inp, nq, nkv, hn, bias), TOL["bf16"])


@pytest.mark.parametrize("bias", [True, False])
def test_attn_accumulate(tp, bias):
    T, H, nq, nkv, hn = 264, 272, 2, 2, 64
    w = synth.ATTN_WORKLOADS[6]
    inp = synth.make_attn_inputs(w, tokens=T, hidden=H, q_heads=nq, kv_heads=nkv, head_dim=hn,
                                 seed_base=650)
    nqkv, d = (nq + 2 * nkv) * hn, nq * hn
    prior = {"dWqkv": synth.grad_init(6, (nqkv, H), 1), "dWo": synth.grad_init(6, (H, d), 2)}
    if bias:
        prior["dbqkv"] = synth.grad_init(6, (nqkv,), 3)
    got = _gpu_attn(tp, inp, nq, nkv, hn, "bf16", bias, prior=prior)
    _check(got, _oracle_attn(inp, nq, nkv, hn, bias, prior=prior), TOL["bf16"],
           names=("dWo", "dWqkv", "dbqkv"))


def test_attn_zero_tokens(tp):
    """T = 0: the forward and dgrad calls enqueue nothing; wgrad overwrites
    with zeros (accumulate = 0) or leaves the buffers alone (accumulate = 1)."""
    H, nq, nkv, hn = 64, 2, 1, 16
    desc = tp.make_attn_desc(0, H, nq, nkv, hn, dtype="bf16", has_bias=True)
    nqkv, d = (nq + 2 * nkv) * hn, nq * hn
    anyp = torch.zeros(16, dtype=torch.bfloat16, device="cuda")  # valid aligned pointer
    tp.tpmlp_attn_qkv_fwd(desc, anyp, anyp, anyp, anyp)
    tp.tpmlp_attn_out_fwd(desc, anyp, anyp, anyp)
    tp.tpmlp_attn_out_bwd_dgrad(desc, anyp, anyp, anyp)
    tp.tpmlp_attn_qkv_bwd_dgrad(desc, anyp, anyp, anyp)
    dWo = torch.full((H, d), 7.0, device="cuda")
    dW = torch.full((nqkv, H), 7.0, device="cuda")
    db = torch.full((nqkv,), 7.0, device="cuda")
    ws = torch.empty(max(tp.attn_workspace_size(desc), 16), dtype=torch.uint8, device="cuda")
    for acc in (True, False):
        tp.tpmlp_attn_out_bwd_wgrad(desc, anyp, anyp, dWo, acc)
        tp.tpmlp_attn_qkv_bwd_wgrad(desc, anyp, anyp, dW, db, acc, ws)
        torch.cuda.synchronize()
        want = 7.0 if acc else 0.0
        assert torch.all(dWo == want) and torch.all(dW == want) and torch.all(db == want)


# ------------------------------------------------------------------ exactness at fp32
def _sdpa(q, k, v, nq, nkv, hn, batch):
    """torch's causal attention on [T, heads*hn] views (the core attention
    the projections surround; not part of the library)."""
    T = q.shape[0]
    S = T // batch
    sh = lambda a, n: a.reshape(batch, S, n, hn).transpose(1, 2)
    kk = sh(k, nkv).repeat_interleave(nq // nkv, dim=1)
    vv = sh(v, nkv).repeat_interleave(nq // nkv, dim=1)
    c = torch.nn.functional.scaled_dot_product_attention(sh(q, nq), kk, vv, is_causal=True)
    return c.transpose(1, 2).reshape(T, nq * hn)


@pytest.mark.parametrize("nq,nkv", [(4, 4), (4, 2)])
def test_attn_block_fp32_two_ranks_sum_to_unsharded(tp, nq, nkv):
    """fp32, tp = 2: on the GPU each rank's packed projection, torch's
    attention on its heads and its output projection; the ranks' y_partial
    and dx_partial summed, and their weight gradients put back in place,
    equal the oracle's unsharded block and torch autograd of it in float64
    on the CPU within 1e-5."""
    tpd, batch, S, H, hn = 2, 2, 64, 256, 64
    T = batch * S
    rng = np.random.default_rng(nq * 10 + nkv)
    f32 = lambda a: np.asarray(a, np.float32)
    x = f32(rng.standard_normal((T, H)))
    Wq, Wk, Wv = (f32(rng.standard_normal((n * hn, H)) * 0.05) for n in (nq, nkv, nkv))
    bq, bk, bv = (f32(rng.standard_normal(n * hn) * 0.1) for n in (nq, nkv, nkv))
    Wo = f32(rng.standard_normal((H, nq * hn)) * 0.05)
    dy = f32(rng.standard_normal((T, H)))
    ws = (Wq, Wk, Wv, bq, bk, bv, Wo)
    # oracle: unsharded forward; float64 torch autograd of the unsharded block
    f = oracle.to_f64
    y_ref = oa.core_attention(f(x) @ f(Wq).T + bq, f(x) @ f(Wk).T + bk, f(x) @ f(Wv).T + bv,
                              nq, nkv, hn, batch) @ f(Wo).T
    t = [torch.tensor(f(a), requires_grad=True) for a in (x,) + ws]
    lin = lambda a, W, b: a @ W.T + b
    yt = _sdpa(lin(t[0], t[1], t[4]), lin(t[0], t[2], t[5]), lin(t[0], t[3], t[6]),
               nq, nkv, hn, batch) @ t[7].T
    (yt * torch.from_numpy(f(dy))).sum().backward()
    g = {n: a.grad.numpy() for n, a in zip(("x", "Wq", "Wk", "Wv", "bq", "bk", "bv", "Wo"), t)}
    # device: two ranks
    nq_r, nkv_r = nq // tpd, nkv // tpd
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    y = torch.zeros((T, H), device="cuda")
    dx = torch.zeros((T, H), device="cuda")
    dWq, dWk, dWv = np.zeros_like(Wq), np.zeros_like(Wk), np.zeros_like(Wv)
    dbq, dbk, dbv = np.zeros_like(bq), np.zeros_like(bk), np.zeros_like(bv)
    dWo = np.zeros_like(Wo)
    for r in range(tpd):
        # rank r's shard, laid out as the library takes it (heads of rank r,
        # rows stacked q, k, v); the slicing is plain indexing
        qs = slice(r * nq_r * hn, (r + 1) * nq_r * hn)
        ks = slice(r * nkv_r * hn, (r + 1) * nkv_r * hn)
        Wqkv = dev(np.concatenate([Wq[qs], Wk[ks], Wv[ks]]))
        bqkv = dev(np.concatenate([bq[qs], bk[ks], bv[ks]]))
        Wo_r = dev(Wo[:, qs])
        desc = tp.make_attn_desc(T, H, nq_r, nkv_r, hn, dtype="f32", has_bias=True)
        say(f"  fp32 block rank {r}: nq_r={nq_r} nkv_r={nkv_r}")
        qkv, q, k, v = tp.attn_qkv_fwd(desc, dev(x), Wqkv, bqkv)
        qkv_l = qkv.clone().requires_grad_(True)
        a, b = nq_r * hn, (nq_r + nkv_r) * hn
        ctx_l = _sdpa(qkv_l[:, :a], qkv_l[:, a:b], qkv_l[:, b:], nq_r, nkv_r, hn, batch)
        ctx = ctx_l.detach().contiguous()
        y += tp.attn_out_fwd(desc, ctx, Wo_r)
        dctx, dWo_r = tp.attn_out_bwd(desc, dev(dy), Wo_r, ctx)
        ctx_l.backward(dctx)
        dqkv = qkv_l.grad.contiguous()
        dx_r, dW_r, db_r = tp.attn_qkv_bwd(desc, dqkv, Wqkv, dev(x))
        dx += dx_r
        dW_r, db_r = dW_r.cpu().numpy(), db_r.cpu().numpy()
        dWq[qs], dWk[ks], dWv[ks] = dW_r[:a], dW_r[a:b], dW_r[b:]
        dbq[qs], dbk[ks], dbv[ks] = db_r[:a], db_r[a:b], db_r[b:]
        dWo[:, qs] = dWo_r.cpu().numpy()
    torch.cuda.synchronize()
    got = {"y": y.cpu(), "x": dx.cpu(), "Wq": dWq, "Wk": dWk, "Wv": dWv, "bq": dbq, "bk": dbk,
           "bv": dbv, "Wo": dWo}
    ref = dict(g, y=y_ref)
    # the key bias shifts every score of a query by the same amount, which the
    # softmax cancels: its gradient is zero, so both sides hold rounding noise;
    # it is held to the scale of the other bias gradients instead
    bscale = max(np.max(np.abs(ref["bq"])), np.max(np.abs(ref["bv"])))
    assert np.max(np.abs(ref["bk"])) <= 1e-12 * bscale
    e_bk = float(np.max(np.abs(got.pop("bk")))) / bscale
    errs = {n: rel_err(got[n], ref[n]) for n in got}
    errs["bk (abs, to the bias scale)"] = e_bk
    say("    rel errors " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL["f32"] for v in errs.values()), errs


# ------------------------------------------------------------------ full per-rank shapes
ROWS = np.array([0, 1, 255, 256, 2049, 4095])
FEATS = np.array([0, 1, 63, 64, 700, 1023])


@pytest.mark.parametrize("cfg", [6, 7])
def test_attn_full_size_sampled(tp, cfg):
    """The per-rank shapes of the attention workloads in full; the oracle
    checks sampled token rows (qkv, y, dctx, dx), sampled packed features
    (dWqkv rows, dbqkv entries) and sampled dWo columns."""
    w = synth.ATTN_WORKLOADS[cfg]
    say(f"attention config {cfg} {w.name}: generating inputs")
    inp = synth.make_attn_inputs(w)
    nq, nkv, hn = w.q_heads_rank, w.kv_heads_rank, w.head_dim
    got = _gpu_attn(tp, inp, nq, nkv, hn, w.dtype, w.b_std is not None)
    f = oracle.to_f64
    x, W, Wo, dy, ctx, dqkv = (f(inp[n]) for n in ("x", "Wqkv", "Wo", "dy", "ctx", "dqkv"))
    b = f(inp["bqkv"])
    rows = ROWS[ROWS < w.tokens]
    feats = np.concatenate([FEATS, w.nqkv - 1 - FEATS])
    cols = FEATS[FEATS < w.d]
    dWs, dbs = oa.qkv_wgrad(dqkv[:, feats], x)
    ref = {"qkv": oa.qkv_forward(x[rows], W, b), "y": oa.out_forward(ctx[rows], Wo),
           "dctx": oa.out_dgrad(dy[rows], Wo), "dx": oa.qkv_dgrad(dqkv[rows], W),
           "dWqkv": dWs, "dbqkv": dbs, "dWo": oa.out_wgrad(dy, ctx[:, cols])}
    smp = {"qkv": got["qkv"][rows], "y": got["y"][rows], "dctx": got["dctx"][rows],
           "dx": got["dx"][rows], "dWqkv": got["dWqkv"][feats], "dbqkv": got["dbqkv"][feats],
           "dWo": got["dWo"][:, cols]}
    _check(smp, ref, TOL[w.dtype], names=tuple(ref))
