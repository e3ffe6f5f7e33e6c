"""The allocation-free weight gradient, tpmlp_bwd_wgrad_noalloc, through the
C ABI against tpmlp_bwd_wgrad given only the workspace it cannot run without
(the db1 partial sums; neither splits along K): the same kernels in the same
order, so dW1, db1 and dW2 must agree bit for bit. Calls in a row share the
library's fixed scratch: a larger problem, then a smaller one accumulating
into prior gradients (the scratch still holds the larger call's partial
sums), then an FP8 block and a gated block without bias (no partial sums).
The first call is also held to the oracle at the bf16 tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu_helpers import TOL, oracle_block, rel_err, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tp():
    require_gpu()
    import tensor_transformer_mlp_rank_amd as m
    return m


def _min_workspace(T, H, Fs, G, bias):
    if not bias:
        return 0
    tiles_n = (H + 255) // 256
    return ((tiles_n * G * Fs * 4 + 255) // 256) * 256


def _both(tp, desc, dev, a, dH, T, H, Fs, G, bias, accumulate, fp8=None, prior=None):
    """(noalloc outputs, tpmlp_bwd_wgrad outputs), each into fresh buffers
    holding `prior` (or garbage when not accumulating)."""
    def bufs():
        if prior is not None:
            return {k: (None if v is None else v.clone()) for k, v in prior.items()}
        return {"dW1": torch.full((G * Fs, H), 3.0, device="cuda"),
                "db1": torch.full((G * Fs,), 3.0, device="cuda") if bias else None,
                "dW2": torch.full((H, Fs), 3.0, device="cuda")}
    got, ref = bufs(), bufs()
    tp.tpmlp_bwd_wgrad_noalloc(desc, dev["dy"], dev["x"], a, dH, got["dW1"], got["db1"],
                               got["dW2"], accumulate=accumulate, fp8=fp8)
    n = _min_workspace(T, H, Fs, G, bias)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
    tp.tpmlp_bwd_wgrad(desc, dev["dy"], dev["x"], a, dH, ref["dW1"], ref["db1"], ref["dW2"],
                       accumulate=accumulate, fp8=fp8, workspace=ws[:n] if n else None)
    torch.cuda.synchronize()
    return got, ref


def _bf16_case(tp, T, H, Fs, act, seed, accumulate):
    w = synth.WORKLOADS[4 if act == "swiglu" else 2]
    inp = synth.make_rank_inputs(w, tokens=T, hidden=H, ffn_shard=Fs, seed_base=seed)
    bias = act == "gelu"
    G = 2 if act == "swiglu" else 1
    desc = tp.make_desc(T, H, Fs, act=act, dtype="bf16", has_bias=bias)
    dev = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    f = tp.fwd(desc, dev["x"], dev["W1"], dev["b1"] if bias else None, dev["W2"])
    g = tp.bwd_dgrad(desc, dev["dy"], dev["W1"], dev["W2"], f["h"])
    prior = None
    if accumulate:
        prior = {"dW1": synth.grad_init(seed, (G * Fs, H), 1).cuda(),
                 "db1": synth.grad_init(seed, (G * Fs,), 2).cuda() if bias else None,
                 "dW2": synth.grad_init(seed, (H, Fs), 3).cuda()}
    say(f"  noalloc wgrad {act} T={T} H={H} Fs={Fs} accumulate={accumulate}")
    got, ref = _both(tp, desc, dev, f["a"], g["dH"], T, H, Fs, G, bias, accumulate, prior=prior)
    for k in ("dW1", "db1", "dW2"):
        if ref[k] is None:
            continue
        assert torch.equal(got[k], ref[k]), k
        assert rel_err(got[k].cpu(), ref[k].cpu()) <= TOL["bf16"], k
    return inp, got, prior


def test_noalloc_matches_the_workspace_call_on_calls_in_a_row(tp):
    # 1: larger problem (1040 / 256 -> 5 tile columns of db1 partials), against the oracle too
    inp, got, _ = _bf16_case(tp, 1000, 1040, 528, "gelu", seed=71, accumulate=False)
    ref = oracle_block(inp, "gelu", True)
    for k in ("dW1", "db1", "dW2"):
        e = rel_err(got[k].cpu(), ref[k])
        say(f"    {k} against the oracle: {e:.2e}")
        assert e <= TOL["bf16"], k
    # 2: smaller, accumulating into prior gradients
    _bf16_case(tp, 300, 272, 144, "gelu", seed=72, accumulate=True)
    # 3: gated, no bias: no partial sums, the scratch is not needed
    _bf16_case(tp, 200, 256, 96, "swiglu", seed=73, accumulate=False)


def test_noalloc_fp8(tp):
    """E4M3 block: the db1 partial sums of the E5M2 dH codes in the scratch."""
    T, H, Fs = 300, 528, 272
    w = synth.WORKLOADS[5]
    inp = synth.make_rank_inputs(w, tokens=T, hidden=H, ffn_shard=Fs, seed_base=74)
    dev, sinv = {}, {}
    for k, e5 in (("x", False), ("W1", False), ("W2", False), ("dy", True)):
        dev[k], _, sinv[k] = tp.quantize_e4m3(inp[k].float().cuda(), e5m2=e5)
    desc = tp.make_desc(T, H, Fs, act="gelu", dtype="e4m3", has_bias=True)
    ah = tp.DelayedScaling(4, scale=64.0)
    dh = tp.DelayedScaling(4, scale=1024.0)
    f = tp.fwd(desc, dev["x"], dev["W1"], inp["b1"].cuda(), dev["W2"],
               fp8_in_scales=(sinv["x"], sinv["W1"], sinv["W2"]), a_history=ah)
    g = tp.bwd_dgrad(desc, dev["dy"], dev["W1"], dev["W2"], f["h"],
                     fp8=dict(dy_scale_inv=sinv["dy"], w1_scale_inv=sinv["W1"],
                              w2_scale_inv=sinv["W2"], dH_history=dh))
    sc = tp.fp8_scales(x_scale_inv=sinv["x"], a_scale_inv=ah.scale_inv, dy_scale_inv=sinv["dy"],
                       dH_scale_inv=dh.scale_inv)
    say(f"  noalloc wgrad e4m3 T={T} H={H} Fs={Fs}")
    got, ref = _both(tp, desc, dev, f["a"], g["dH"], T, H, Fs, 1, True, False, fp8=sc)
    for k in ("dW1", "db1", "dW2"):
        assert torch.equal(got[k], ref[k]), k
    assert float(torch.max(torch.abs(got["db1"]))) > 0
