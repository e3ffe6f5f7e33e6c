"""GPU parity of the grouped expert MLPs (tpmlp_moe_*) through the C ABI
against the oracle's grouped block (oracle.moe) on the same seeded inputs,
max|gpu - oracle| / max|oracle| within 2e-2 per output tensor (bf16).

* Ragged groups: empty experts, single-row experts, group sizes that are
  not multiples of the 256-row tile, up to 64 experts; GELU with bias,
  GELU without, SwiGLU; the accumulate mode of the weight gradients.
* The documented clamping of the counts: with counts that sum past the
  tensors' rows, or are negative, no row outside [0, tokens) is touched
  (the tensors carry sentinel rows past `tokens`), and the result is the
  oracle's on the clamped counts; rows past the sum of the counts keep
  their contents.
* Zero tokens.
* The two expert workloads at full size on sampled rows and features.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import block as ob
from oracle import moe as om
from _gpu_helpers import TOL, rel_err, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tp():
    require_gpu()
    import tensor_transformer_mlp_rank_amd as m
    return m


def _gpu_moe(tp, inp, counts_dev, tokens, act, has_bias, prior=None, pad=0):
    """fwd, dgrad, wgrad on the device. Token-major tensors get `pad`
    sentinel rows (value 7) past `tokens`; returns CPU tensors with the
    padding still attached."""
    x = inp["x"]
    H = x.shape[1]
    E, GFs, _ = inp["W1"].shape
    Fs = inp["W2"].shape[2]
    desc = tp.make_moe_desc(tokens, H, Fs, E, act=act, dtype="bf16", has_bias=has_bias)
    say(f"  moe act={act} bias={has_bias} E={E} H={H} Fs={Fs} tokens={tokens} pad={pad} "
        f"counts={counts_dev.cpu().tolist()[:12]}")
    dev = lambda t: None if t is None else t.contiguous().cuda()

    def padded(t, cols):
        buf = torch.full((tokens + pad, cols), 7.0, dtype=torch.bfloat16, device="cuda")
        if t is not None:
            buf[:t.shape[0]] = t.cuda()
        return buf

    xd, dyd = padded(x[:tokens], H), padded(inp["dy"][:tokens], H)
    W1, W2 = dev(inp["W1"]), dev(inp["W2"])
    b1 = dev(inp["b1"]) if has_bias else None
    y, h, a = padded(None, H), padded(None, GFs), padded(None, Fs)
    tp.tpmlp_moe_fwd(desc, counts_dev, xd, W1, b1, W2, y, h, a)
    dH, dx = padded(None, GFs), padded(None, H)
    tp.tpmlp_moe_bwd_dgrad(desc, counts_dev, dyd, W1, W2, h, dH, dx)
    acc = None if prior is None else {k: (None if v is None else v.cuda()) for k, v in prior.items()}
    w = tp.moe_bwd_wgrad(desc, counts_dev, dyd, xd, a, dH, accumulate_into=acc)
    torch.cuda.synchronize()
    out = dict(y=y, h=h, a=a, dH=dH, dx=dx, dW1=w["dW1"], db1=w.get("db1"), dW2=w["dW2"])
    return {k: (None if v is None else v.cpu()) for k, v in out.items()}


def _oracle_moe(inp, counts, tokens, act, has_bias, prior=None):
    f = oracle.to_f64
    x, dy = f(inp["x"])[:tokens], f(inp["dy"])[:tokens]
    W1, W2 = f(inp["W1"]), f(inp["W2"])
    b1 = f(inp["b1"]) if has_bias else None
    fw = om.grouped_forward(x, counts, W1, b1, W2, act)
    g = om.grouped_dgrad(dy, counts, W1, W2, fw["h"], act)
    p = {} if prior is None else {k: (None if v is None else f(v)) for k, v in prior.items()}
    w = om.grouped_wgrad(dy, x, fw["a"], g["dH"], counts, has_bias, p.get("dW1"), p.get("db1"),
                         p.get("dW2"))
    return {**fw, **g, **w}


def _check(got, ref, rows, names=("y", "h", "a", "dH", "dx", "dW1", "db1", "dW2")):
    errs = {}
    for n in names:
        if ref.get(n) is None:
            continue
        g = got[n][:rows] if n in ("y", "h", "a", "dH", "dx") else got[n]
        errs[n] = rel_err(g, ref[n])
    say("    rel errors " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL["bf16"]}
    assert not bad, f"tolerance exceeded: {bad}"


CASES = [
    # counts, H, Fs, act, bias
    ([300, 0, 1, 513, 256, 37], 272, 144, "gelu", True),
    ([5, 700, 0, 0, 260], 528, 96, "swiglu", False),
    ([1], 64, 16, "gelu", False),
    (list(range(0, 64 * 7, 7)), 256, 64, "gelu", True),
    ([1024, 768], 512, 512, "swiglu", False),
    # 9 tile columns in each expert's dW1, more than its stages
    ([130, 0, 64, 7], 2304, 80, "gelu", True),
    # the most experts the calls accept (1024), each with 0 to 4 rows
    ([(7 * i) % 5 for i in range(1024)], 64, 16, "gelu", True),
]


@pytest.mark.parametrize("counts,H,Fs,act,bias", CASES)
def test_moe_ragged_groups(tp, counts, H, Fs, act, bias):
    w = synth.MOE_WORKLOADS[9 if act == "gelu" else 8]
    inp = synth.make_moe_inputs(w, counts, hidden=H, ffn_shard=Fs, experts=len(counts),
                                seed_base=800 + len(counts) + H)
    if not bias:
        inp["b1"] = None
    T = int(sum(counts))
    cd = torch.tensor(counts, dtype=torch.int32, device="cuda")
    got = _gpu_moe(tp, inp, cd, T, act, bias, pad=8)
    ref = _oracle_moe(inp, counts, T, act, bias)
    _check(got, ref, T)
    for n in ("y", "h", "a", "dH", "dx"):   # the padding rows are untouched
        assert torch.all(got[n][T:] == 7.0), n


def test_moe_accumulate(tp):
    counts = [200, 0, 333, 64]
    H, Fs = 272, 112
    w = synth.MOE_WORKLOADS[9]
    inp = synth.make_moe_inputs(w, counts, hidden=H, ffn_shard=Fs, experts=4, seed_base=880)
    prior = {"dW1": synth.grad_init(9, (4, Fs, H), 1), "db1": synth.grad_init(9, (4, Fs), 2),
             "dW2": synth.grad_init(9, (4, H, Fs), 3)}
    T = sum(counts)
    got = _gpu_moe(tp, inp, torch.tensor(counts, dtype=torch.int32, device="cuda"), T, "gelu",
                   True, prior=prior)
    ref = _oracle_moe(inp, counts, T, "gelu", True, prior=prior)
    _check(got, ref, T, names=("dW1", "db1", "dW2"))


def _clamped(counts, rows):
    """The documented clamping: negative counts as 0, running total capped."""
    out, tot = [], 0
    for c in counts:
        c = max(int(c), 0)
        n = min(c, rows - tot)
        out.append(n)
        tot += n
    return out


@pytest.mark.parametrize("counts,rows", [
    ([300, -5, 400, 200], 600),     # past the rows: the third group is cut, the fourth empty
    ([100, 50, 0, 20], 400),        # short of the rows: rows 170..399 keep their contents
    ([-1, 2 ** 31 - 1, 7], 333),    # negative and huge counts
])
def test_moe_counts_are_clamped(tp, counts, rows):
    H, Fs, E = 128, 64, len(counts)
    w = synth.MOE_WORKLOADS[9]
    cl = _clamped(counts, rows)
    inp = synth.make_moe_inputs(w, [rows], hidden=H, ffn_shard=Fs, experts=E, seed_base=890)
    cd = torch.tensor(counts, dtype=torch.int32, device="cuda")
    got = _gpu_moe(tp, inp, cd, rows, "gelu", True, pad=16)
    covered = sum(cl)
    ref = _oracle_moe(inp, cl, covered, "gelu", True)
    _check(got, ref, covered)
    for n in ("y", "h", "a", "dH", "dx"):
        assert torch.all(got[n][covered:] == 7.0), n   # uncovered and padding rows untouched


def test_moe_zero_tokens(tp):
    H, Fs, E = 64, 32, 3
    desc = tp.make_moe_desc(0, H, Fs, E, act="gelu", dtype="bf16", has_bias=True)
    cd = torch.zeros(E, dtype=torch.int32, device="cuda")
    anyp = torch.zeros(64, dtype=torch.bfloat16, device="cuda")  # valid aligned pointer
    W1 = torch.zeros((E, Fs, H), dtype=torch.bfloat16, device="cuda")
    W2 = torch.zeros((E, H, Fs), dtype=torch.bfloat16, device="cuda")
    b1 = torch.zeros((E, Fs), dtype=torch.bfloat16, device="cuda")
    tp.tpmlp_moe_fwd(desc, cd, anyp, W1, b1, W2, anyp, anyp, anyp)
    tp.tpmlp_moe_bwd_dgrad(desc, cd, anyp, W1, W2, anyp, anyp, anyp)
    dW1 = torch.full((E, Fs, H), 7.0, device="cuda")
    db1 = torch.full((E, Fs), 7.0, device="cuda")
    dW2 = torch.full((E, H, Fs), 7.0, device="cuda")
    ws = torch.empty(tp.moe_workspace_size(desc), dtype=torch.uint8, device="cuda")
    for acc in (True, False):
        tp.tpmlp_moe_bwd_wgrad(desc, cd, anyp, anyp, anyp, anyp, dW1, db1, dW2, acc, ws)
        torch.cuda.synchronize()
        want = 7.0 if acc else 0.0
        assert torch.all(dW1 == want) and torch.all(db1 == want) and torch.all(dW2 == want)


@pytest.mark.parametrize("cfg", [8, 9])
def test_moe_full_size_sampled(tp, cfg):
    """The expert workloads at full size; the oracle checks sampled rows (y,
    h, a, dH, dx, each through its own expert) and sampled features of
    three experts (rows of dW1, entries of db1, columns of dW2)."""
    w = synth.MOE_WORKLOADS[cfg]
    counts = synth.moe_counts(w)
    say(f"moe config {cfg} {w.name}: counts {counts.tolist()[:16]}")
    inp = synth.make_moe_inputs(w, counts)
    T = int(counts.sum())
    got = _gpu_moe(tp, inp, torch.from_numpy(counts).cuda(), T, w.act, w.has_bias)
    cache = {}

    def f(t):  # float64 copies of the (large) expert weights, made once each
        if isinstance(t, tuple):
            if t not in cache:
                name, e = t
                cache[t] = oracle.to_f64(inp[name][e])
            return cache[t]
        return oracle.to_f64(t)
    off = om.offsets(counts)
    owner = np.repeat(np.arange(w.experts), counts)
    rows = np.array([0, 1, T // 3, T // 2 + 7, T - 2, T - 1])
    ref_rows = {k: [] for k in ("y", "h", "a", "dH", "dx")}
    for r in rows:
        e = owner[r]
        b1 = f(inp["b1"][e]) if w.has_bias else None
        fr = ob.rank_forward(f(inp["x"][r:r + 1]), f(("W1", e)), b1, f(("W2", e)), w.act)
        gr = ob.rank_dgrad(f(inp["dy"][r:r + 1]), f(("W1", e)), f(("W2", e)), fr["h"], w.act)
        for k in ("y", "h", "a"):
            ref_rows[k].append(fr[k][0])
        for k in ("dH", "dx"):
            ref_rows[k].append(gr[k][0])
    ref = {k: np.stack(v) for k, v in ref_rows.items()}
    smp = {k: got[k][rows] for k in ref}
    errs = {k: rel_err(smp[k], ref[k]) for k in ref}
    # weight gradients: three experts, sampled features
    Fs = w.ffn_shard
    feats = np.array([0, 1, 255, 256, Fs - 1])
    w1rows = feats if w.act == "gelu" else np.concatenate([feats, Fs + feats])
    for e in (0, int(np.argmax(counts)), w.experts - 1):
        r0, r1 = int(off[e]), int(off[e] + counts[e])
        x, dy = f(inp["x"][r0:r1]), f(inp["dy"][r0:r1])
        b1 = f(inp["b1"][e]) if w.has_bias else None
        W1s, b1s, W2s = ob.select_features(f(("W1", e)), b1, f(("W2", e)), feats, w.act)
        fc = ob.rank_forward(x, W1s, b1s, W2s, w.act)
        gc = ob.rank_dgrad(dy, W1s, W2s, fc["h"], w.act)
        wc = ob.rank_wgrad(dy, x, fc["a"], gc["dH"], w.has_bias)
        errs[f"dW1[{e}]"] = rel_err(got["dW1"][e][w1rows], wc["dW1"])
        errs[f"dW2[{e}]"] = rel_err(got["dW2"][e][:, feats], wc["dW2"])
        if w.has_bias:
            errs[f"db1[{e}]"] = rel_err(got["db1"][e][feats], wc["db1"])
    say("    rel errors " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL["bf16"]}
    assert not bad, f"tolerance exceeded: {bad}"
