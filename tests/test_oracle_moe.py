"""CPU pins of the grouped expert-MLP oracle (oracle.moe).

* Torch autograd of an independent formulation -- every token through every
  expert's block, masked by a one-hot expert assignment and summed -- gives
  the same outputs and the same per-expert gradients, for GELU with bias and
  SwiGLU without, with empty, single-row and large groups.
* One expert holding every row is the plain per-rank block.
* Reordering the rows inside each group reorders the outputs the same way
  and leaves the weight gradients unchanged; moving a row to another group
  changes them (negative control).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle import block as ob
from oracle import moe


def _experts(rng, E, H, Fs, act, bias):
    G = 2 if act == "swiglu" else 1
    W1 = rng.standard_normal((E, G * Fs, H)) * 0.3
    W2 = rng.standard_normal((E, H, Fs)) * 0.3
    b1 = rng.standard_normal((E, G * Fs)) * 0.2 if bias else None
    return W1, b1, W2


def _torch_masked(x, counts, W1, b1, W2, dy, act):
    """Every token through every expert, masked by its group; autograd."""
    T = x.shape[0]
    E = len(counts)
    Fs = W2.shape[2]
    owner = np.repeat(np.arange(E), counts)
    mask = torch.from_numpy((owner[:, None] == np.arange(E)[None, :]).astype(np.float64))
    tx = torch.tensor(x, requires_grad=True)
    tW1 = torch.tensor(W1, requires_grad=True)
    tW2 = torch.tensor(W2, requires_grad=True)
    tb1 = None if b1 is None else torch.tensor(b1, requires_grad=True)
    y = torch.zeros(T, x.shape[1], dtype=torch.float64)
    for e in range(E):
        h = tx @ tW1[e].T + (0 if tb1 is None else tb1[e])
        if act == "gelu":
            a = Fn.gelu(h, approximate="tanh")
        else:
            a = Fn.silu(h[:, :Fs]) * h[:, Fs:]
        y = y + mask[:, e:e + 1] * (a @ tW2[e].T)
    (y * torch.from_numpy(dy)).sum().backward()
    return {"y": y.detach().numpy(), "dx": tx.grad.numpy(), "dW1": tW1.grad.numpy(),
            "dW2": tW2.grad.numpy(), "db1": None if tb1 is None else tb1.grad.numpy()}


@pytest.mark.parametrize("act,bias", [("gelu", True), ("swiglu", False), ("gelu", False)])
@pytest.mark.parametrize("counts", [[3, 0, 5, 1], [9], [0, 0, 4], [2, 7, 0, 0, 1, 3]])
def test_grouped_block_matches_masked_dense_autograd(act, bias, counts):
    rng = np.random.default_rng(sum(counts) + len(counts) * 13 + (act == "swiglu"))
    E, H, Fs = len(counts), 6, 5
    T = sum(counts)
    x = rng.standard_normal((T, H))
    dy = rng.standard_normal((T, H))
    W1, b1, W2 = _experts(rng, E, H, Fs, act, bias)
    f = moe.grouped_forward(x, counts, W1, b1, W2, act)
    g = moe.grouped_dgrad(dy, counts, W1, W2, f["h"], act)
    w = moe.grouped_wgrad(dy, x, f["a"], g["dH"], counts, bias)
    ref = _torch_masked(x, counts, W1, b1, W2, dy, act)
    assert np.allclose(f["y"], ref["y"], rtol=0, atol=1e-12)
    assert np.allclose(g["dx"], ref["dx"], rtol=0, atol=1e-12)
    assert np.allclose(w["dW1"], ref["dW1"], rtol=0, atol=1e-12)
    assert np.allclose(w["dW2"], ref["dW2"], rtol=0, atol=1e-12)
    if bias:
        assert np.allclose(w["db1"], ref["db1"], rtol=0, atol=1e-12)
    # an empty group's weight gradients are zero
    for e, c in enumerate(counts):
        if c == 0:
            assert not np.any(w["dW1"][e]) and not np.any(w["dW2"][e])


def test_one_expert_is_the_plain_block():
    rng = np.random.default_rng(4)
    T, H, Fs = 7, 8, 6
    x, dy = rng.standard_normal((T, H)), rng.standard_normal((T, H))
    W1, b1, W2 = _experts(rng, 1, H, Fs, "gelu", True)
    f = moe.grouped_forward(x, [T], W1, b1, W2, "gelu")
    p = ob.rank_forward(x, W1[0], b1[0], W2[0], "gelu")
    assert np.array_equal(f["y"], p["y"]) and np.array_equal(f["h"], p["h"])
    g = moe.grouped_dgrad(dy, [T], W1, W2, f["h"], "gelu")
    q = ob.rank_dgrad(dy, W1[0], W2[0], p["h"], "gelu")
    assert np.array_equal(g["dx"], q["dx"])
    w = moe.grouped_wgrad(dy, x, f["a"], g["dH"], [T], True, dW1_in=np.ones((1, Fs, H)))
    r = ob.rank_wgrad(dy, x, p["a"], q["dH"], True)
    assert np.allclose(w["dW1"][0], r["dW1"] + 1.0, rtol=0, atol=1e-12)


def test_row_order_within_groups_and_group_membership():
    rng = np.random.default_rng(8)
    counts = [4, 3, 5]
    E, H, Fs, T = 3, 5, 4, 12
    x, dy = rng.standard_normal((T, H)), rng.standard_normal((T, H))
    W1, b1, W2 = _experts(rng, E, H, Fs, "gelu", True)

    def run(xx, dyy, cc):
        f = moe.grouped_forward(xx, cc, W1, b1, W2, "gelu")
        g = moe.grouped_dgrad(dyy, cc, W1, W2, f["h"], "gelu")
        return f, g, moe.grouped_wgrad(dyy, xx, f["a"], g["dH"], cc, True)

    f, g, w = run(x, dy, counts)
    perm = np.concatenate([rng.permutation(np.arange(o, o + c))
                           for o, c in zip(moe.offsets(counts), counts)])
    fp, gp, wp = run(x[perm], dy[perm], counts)
    assert np.allclose(fp["y"], f["y"][perm], atol=1e-12)
    assert np.allclose(gp["dx"], g["dx"][perm], atol=1e-12)
    for k in ("dW1", "db1", "dW2"):
        assert np.allclose(wp[k], w[k], atol=1e-12), k
    # one row moved from group 0 to group 1: different outputs for that row
    f2, _, w2 = run(x, dy, [3, 4, 5])
    assert not np.allclose(f2["y"][3], f["y"][3], atol=1e-6)
    assert not np.allclose(w2["dW1"][0], w["dW1"][0], atol=1e-6)
