"""HIP graph capture of the library's calls: a whole step (the MLP block's
forward, dgrad and weight gradients with accumulation; the attention
projections; the grouped expert MLPs) is captured once on a side stream and
replayed several times, with eager work and synchronisations between the
replays. The library enqueues kernels only (no memory set or copy nodes, no
allocation; the counters of a split partial last round are cleared by a
kernel), so every replay must reproduce the eager results bit for bit (the
kernels are deterministic: fixed summation orders, no sum through atomics);
the accumulating weight gradients must grow by exactly one step per
replay."""
import pytest
import torch

import synth
from _gpu_helpers import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tp():
    require_gpu()
    import tensor_transformer_mlp_rank_amd as m
    return m


def _capture(fn):
    """Capture fn() on a side stream (warmed up eagerly first)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def _replays(g, snapshot, n=3):
    """Replay n times with eager work between; returns the snapshot after each."""
    got = []
    for i in range(n):
        junk = torch.randn(1 << 20, device="cuda") * i   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got.append(snapshot())
        del junk
    return got


# (2048, 4352, 4336): the weight gradients' 289- and 578-tile grids split their
# partial last round (counters cleared in the graph, halves met through the
# workspace on every replay)
@pytest.mark.parametrize("T,H,Fs", [(1030, 528, 272), (2048, 4352, 4336)])
@pytest.mark.parametrize("act,bias", [("gelu", True), ("swiglu", False)])
def test_mlp_step_in_a_graph(tp, act, bias, T, H, Fs):
    w = synth.WORKLOADS[2 if act == "gelu" else 4]
    inp = synth.make_rank_inputs(w, tokens=T, hidden=H, ffn_shard=Fs, seed_base=31)
    G = 2 if act == "swiglu" else 1
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    desc = tp.make_desc(T, H, Fs, act=act, dtype="bf16", has_bias=bias)
    bf = torch.bfloat16
    buf = {"y": torch.empty((T, H), dtype=bf, device="cuda"),
           "h": torch.empty((T, G * Fs), dtype=bf, device="cuda"),
           "a": torch.empty((T, Fs), dtype=bf, device="cuda"),
           "dH": torch.empty((T, G * Fs), dtype=bf, device="cuda"),
           "dx": torch.empty((T, H), dtype=bf, device="cuda"),
           "dW1": torch.zeros((G * Fs, H), device="cuda"),
           "db1": torch.zeros((G * Fs,), device="cuda") if bias else None,
           "dW2": torch.zeros((H, Fs), device="cuda")}
    n = tp.workspace_size(desc, tp.CALL_WGRAD)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")

    def step():
        s = torch.cuda.current_stream()
        tp.tpmlp_fwd(desc, d["x"], d["W1"], d["b1"] if bias else None, d["W2"], buf["y"],
                     buf["h"], buf["a"], stream=s)
        tp.tpmlp_bwd_dgrad(desc, d["dy"], d["W1"], d["W2"], buf["h"], buf["dH"], buf["dx"],
                           stream=s)
        tp.tpmlp_bwd_wgrad(desc, d["dy"], d["x"], buf["a"], buf["dH"], buf["dW1"], buf["db1"],
                           buf["dW2"], accumulate=True, workspace=ws[:n] if n else None, stream=s)

    # eager reference: one step from zero gradients
    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in buf.items() if v is not None}
    say(f"  graph: MLP {act} bias={bias} T={T} H={H} Fs={Fs}")
    g = _capture(step)  # the capture's warm-up and capture add two more steps of gradient
    for k in ("dW1", "db1", "dW2"):
        if buf[k] is not None:
            buf[k].zero_()
    snaps = _replays(g, lambda: {k: v.clone() for k, v in buf.items() if v is not None})
    for i, snap in enumerate(snaps):
        for k in ("y", "h", "a", "dH", "dx"):
            assert torch.equal(snap[k], eager[k]), (i, k)
        for k in ("dW1", "db1", "dW2"):
            if buf[k] is None:
                continue
            # the same fp32 adds as eager accumulation of i + 1 steps
            acc = torch.zeros_like(eager[k])
            for _ in range(i + 1):
                acc += eager[k]
            assert torch.equal(snap[k], acc), (i, k)


def test_attention_and_moe_in_a_graph(tp):
    # attention projections (split-K products included)
    T, H, nq, nkv, hn = 2048, 1024, 8, 8, 64
    aw = synth.ATTN_WORKLOADS[6]
    ai = {k: (None if v is None else v.cuda()) for k, v in
          synth.make_attn_inputs(aw, tokens=T, hidden=H, q_heads=nq, kv_heads=nkv, head_dim=hn,
                                 seed_base=41).items()}
    ad = tp.make_attn_desc(T, H, nq, nkv, hn, dtype="bf16", has_bias=True)
    N, D = ad.nqkv, ad.d
    bf = torch.bfloat16
    ab = {"qkv": torch.empty((T, N), dtype=bf, device="cuda"),
          "y": torch.empty((T, H), dtype=bf, device="cuda"),
          "dctx": torch.empty((T, D), dtype=bf, device="cuda"),
          "dx": torch.empty((T, H), dtype=bf, device="cuda"),
          "dWo": torch.empty((H, D), device="cuda"), "dW": torch.empty((N, H), device="cuda"),
          "db": torch.empty((N,), device="cuda")}
    aws = torch.empty(tp.attn_workspace_size(ad), dtype=torch.uint8, device="cuda")
    # grouped experts
    mw = synth.MOE_WORKLOADS[9]
    counts = [300, 0, 700, 37, 500]
    mi = {k: (None if v is None else v.cuda()) for k, v in
          synth.make_moe_inputs(mw, counts, hidden=256, ffn_shard=176, experts=5,
                                seed_base=42).items()}
    R = sum(counts)
    md = tp.make_moe_desc(R, 256, 176, 5, act="gelu", dtype="bf16", has_bias=True)
    mb = {"y": torch.empty((R, 256), dtype=bf, device="cuda"),
          "h": torch.empty((R, 176), dtype=bf, device="cuda"),
          "a": torch.empty((R, 176), dtype=bf, device="cuda"),
          "dH": torch.empty((R, 176), dtype=bf, device="cuda"),
          "dx": torch.empty((R, 256), dtype=bf, device="cuda"),
          "dW1": torch.empty((5, 176, 256), device="cuda"), "db1": torch.empty((5, 176), device="cuda"),
          "dW2": torch.empty((5, 256, 176), device="cuda")}
    mws = torch.empty(tp.moe_workspace_size(md), dtype=torch.uint8, device="cuda")

    def step():
        s = torch.cuda.current_stream()
        tp.tpmlp_attn_qkv_fwd(ad, ai["x"], ai["Wqkv"], ai["bqkv"], ab["qkv"], stream=s)
        tp.tpmlp_attn_out_fwd(ad, ai["ctx"], ai["Wo"], ab["y"], stream=s)
        tp.tpmlp_attn_out_bwd_dgrad(ad, ai["dy"], ai["Wo"], ab["dctx"], aws, stream=s)
        tp.tpmlp_attn_out_bwd_wgrad(ad, ai["dy"], ai["ctx"], ab["dWo"], False, aws, stream=s)
        tp.tpmlp_attn_qkv_bwd_dgrad(ad, ai["dqkv"], ai["Wqkv"], ab["dx"], stream=s)
        tp.tpmlp_attn_qkv_bwd_wgrad(ad, ai["dqkv"], ai["x"], ab["dW"], ab["db"], False, aws,
                                    stream=s)
        c = mi["counts"]
        tp.tpmlp_moe_fwd(md, c, mi["x"], mi["W1"], mi["b1"], mi["W2"], mb["y"], mb["h"], mb["a"],
                         stream=s)
        tp.tpmlp_moe_bwd_dgrad(md, c, mi["dy"], mi["W1"], mi["W2"], mb["h"], mb["dH"], mb["dx"],
                               stream=s)
        tp.tpmlp_moe_bwd_wgrad(md, c, mi["dy"], mi["x"], mb["a"], mb["dH"], mb["dW1"], mb["db1"],
                               mb["dW2"], False, mws, stream=s)

    step()
    torch.cuda.synchronize()
    eager = {("a", k): v.clone() for k, v in ab.items()}
    eager.update({("m", k): v.clone() for k, v in mb.items()})
    say("  graph: attention projections + grouped experts")
    g = _capture(step)
    for b in (ab, mb):
        for v in b.values():
            v.fill_(float("nan"))   # a replay must rewrite every output
    snap = lambda: {**{("a", k): v.clone() for k, v in ab.items()},
                    **{("m", k): v.clone() for k, v in mb.items()}}
    for i, got in enumerate(_replays(g, snap)):
        for k, v in eager.items():
            assert torch.equal(got[k], v), (i, k)
