"""Helpers for the GPU parity tests: run the block through the C ABI and
compute the oracle's reference on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth

# max|gpu - oracle| / max|oracle| per output tensor
TOL = {"f32": 1e-5, "bf16": 2e-2, "e4m3": 6e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rel_err(gpu, ref) -> float:
    gpu = oracle.to_f64(gpu)
    ref = oracle.to_f64(ref)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    den = np.max(np.abs(ref))
    num = np.max(np.abs(gpu - ref))
    if den == 0:
        return float(num)
    return float(num / den)


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X (run them with -m gpu on a machine that has one)"


def to_dev(d: dict) -> dict:
    return {k: (None if v is None else v.contiguous().cuda()) for k, v in d.items()}


def gpu_block(tp, inp: dict, act: str, dtype: str, has_bias: bool, calls=("fwd", "dgrad", "wgrad"),
              accumulate_into=None, recompute=False) -> dict:
    """Run the requested calls on one rank's shard; returns CPU tensors.
    ``recompute``: the weight gradients through tpmlp_bwd_wgrad_recompute,
    from the saved h instead of a."""
    x = inp["x"]
    T, H = x.shape
    G = 2 if act == "swiglu" else 1
    Fs = inp["W1"].shape[0] // G
    desc = tp.make_desc(T, H, Fs, act=act, dtype=dtype, has_bias=has_bias)
    dv = to_dev(inp)
    out = {}
    say(f"  gpu_block act={act} dtype={dtype} T={T} H={H} Fs={Fs} calls={calls}")
    f = tp.fwd(desc, dv["x"], dv["W1"], dv["b1"] if has_bias else None, dv["W2"])
    out.update(y=f["y"], h=f["h"], a=f["a"])
    if "dgrad" in calls:
        g = tp.bwd_dgrad(desc, dv["dy"], dv["W1"], dv["W2"], f["h"])
        out.update(dH=g["dH"], dx=g["dx"])
        if "wgrad" in calls:
            acc = None if accumulate_into is None else to_dev(accumulate_into)
            w = tp.bwd_wgrad(desc, dv["dy"], dv["x"], f["h"] if recompute else f["a"], g["dH"],
                             accumulate_into=acc, recompute=recompute)
            out.update(dW1=w["dW1"], db1=w.get("db1"), dW2=w["dW2"])
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu()) for k, v in out.items()}


def oracle_block(inp: dict, act: str, has_bias: bool, prior=None) -> dict:
    b1 = inp["b1"] if has_bias else None
    f = oracle.rank_forward(inp["x"], inp["W1"], b1, inp["W2"], act)
    g = oracle.rank_dgrad(inp["dy"], inp["W1"], inp["W2"], f["h"], act)
    p = prior or {}
    w = oracle.rank_wgrad(inp["dy"], inp["x"], f["a"], g["dH"], has_bias,
                          p.get("dW1"), p.get("db1"), p.get("dW2"))
    return {**f, **g, **w}


def check(gpu: dict, ref: dict, dtype: str, names, tol=None):
    tol = TOL[dtype] if tol is None else tol
    errs = {}
    for n in names:
        if ref.get(n) is None:
            continue
        errs[n] = rel_err(gpu[n], ref[n])
    say("  rel errors:", {k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"tolerance {tol} exceeded: {bad}"
    return errs


def sampled_reference(inp: dict, act: str, has_bias: bool, rows, cols) -> dict:
    """Oracle values at sampled token rows (y, h, a, dH, dx) and sampled
    intermediate features (columns of dW2, rows of dW1, entries of db1), each
    computed from the full inputs through the same definitions."""
    b1 = inp["b1"] if has_bias else None
    x = oracle.to_f64(inp["x"])
    dy = oracle.to_f64(inp["dy"])
    W1 = oracle.to_f64(inp["W1"])
    W2 = oracle.to_f64(inp["W2"])
    b1 = None if b1 is None else oracle.to_f64(b1)
    f = oracle.rank_forward(x[rows], W1, b1, W2, act)
    g = oracle.rank_dgrad(dy[rows], W1, W2, f["h"], act)
    W1s, b1s, W2s = oracle.select_features(W1, b1, W2, cols, act)
    fc = oracle.rank_forward(x, W1s, b1s, W2s, act)
    gc = oracle.rank_dgrad(dy, W1s, W2s, fc["h"], act)
    wc = oracle.rank_wgrad(dy, x, fc["a"], gc["dH"], has_bias)
    return {"y": f["y"], "h": f["h"], "a": f["a"], "dH": g["dH"], "dx": g["dx"],
            "dW2": wc["dW2"], "dW1": wc["dW1"], "db1": wc["db1"]}


def sample_gpu(gpu: dict, act: str, Fs: int, rows, cols) -> dict:
    cols = np.asarray(cols)
    w1rows = cols if act == "gelu" else np.concatenate([cols, Fs + cols])
    out = {k: gpu[k][rows] for k in ("y", "h", "a", "dH", "dx") if gpu.get(k) is not None}
    if gpu.get("dW2") is not None:
        out["dW2"] = gpu["dW2"][:, cols]
        out["dW1"] = gpu["dW1"][w1rows]
        if gpu.get("db1") is not None:
            out["db1"] = gpu["db1"][cols]
    return out
