"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: an independent
library routine (torch's GELU/SiLU and autograd in float64), a closed form,
finite differences, the column->row shard-sum invariant, brute-force loops,
or the OCP E4M3 table. Each is chosen so that a plausible slip in the oracle
(a dropped term, a wrong sign, a transposed operand, a wrong gate/up split,
an off-by-one exponent bias) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn
from scipy.special import ndtr

import oracle
from oracle import block as ob
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRID = np.concatenate([np.linspace(-12, 12, 4001), [0.0, 1e-8, -1e-8, 30.0, -30.0]])


# ---------------------------------------------------------------- activations
def test_gelu_matches_torch_tanh_gelu():
    ref = Fn.gelu(torch.from_numpy(GRID), approximate="tanh").numpy()
    np.testing.assert_allclose(oracle.gelu_tanh(GRID), ref, rtol=0, atol=1e-14)


def test_gelu_grad_matches_torch_autograd():
    z = torch.from_numpy(GRID.copy()).requires_grad_(True)
    Fn.gelu(z, approximate="tanh").sum().backward()
    np.testing.assert_allclose(oracle.gelu_tanh_grad(GRID), z.grad.numpy(), rtol=0, atol=1e-13)


def test_gelu_closed_forms():
    z = GRID
    # tanh is odd, so gelu(z) - gelu(-z) = z exactly and gelu'(z) + gelu'(-z) = 1
    np.testing.assert_allclose(oracle.gelu_tanh(z) - oracle.gelu_tanh(-z), z, atol=1e-14)
    np.testing.assert_allclose(oracle.gelu_tanh_grad(z) + oracle.gelu_tanh_grad(-z), 1.0,
                               atol=1e-14)
    assert oracle.gelu_tanh(0.0) == 0.0
    assert oracle.gelu_tanh_grad(0.0) == 0.5
    assert abs(oracle.gelu_tanh(30.0) - 30.0) < 1e-12
    assert abs(oracle.gelu_tanh(-30.0)) < 1e-12


def test_gelu_is_tanh_variant_not_erf():
    # close to z*Phi(z) (the exact GELU) but measurably different: the tanh form
    diff = np.max(np.abs(oracle.gelu_tanh(GRID) - GRID * ndtr(GRID)))
    assert 1e-4 < diff < 1e-3


def test_gelu_grad_finite_difference():
    z = np.linspace(-8, 8, 801)
    eps = 1e-6
    fd = (oracle.gelu_tanh(z + eps) - oracle.gelu_tanh(z - eps)) / (2 * eps)
    np.testing.assert_allclose(oracle.gelu_tanh_grad(z), fd, atol=1e-8)


def test_silu_matches_torch_and_autograd():
    np.testing.assert_allclose(oracle.silu(GRID), Fn.silu(torch.from_numpy(GRID)).numpy(),
                               rtol=0, atol=1e-14)
    z = torch.from_numpy(GRID.copy()).requires_grad_(True)
    Fn.silu(z).sum().backward()
    np.testing.assert_allclose(oracle.silu_grad(GRID), z.grad.numpy(), rtol=0, atol=1e-13)


def test_silu_closed_forms():
    z = GRID
    np.testing.assert_allclose(oracle.silu(z) - oracle.silu(-z), z, atol=1e-13)
    np.testing.assert_allclose(oracle.silu_grad(z) + oracle.silu_grad(-z), 1.0, atol=1e-13)
    assert oracle.silu(0.0) == 0.0 and oracle.silu_grad(0.0) == 0.5
    fd = (oracle.silu(z + 1e-6) - oracle.silu(z - 1e-6)) / 2e-6
    np.testing.assert_allclose(oracle.silu_grad(z), fd, atol=1e-8)
    # no overflow warnings turn into NaN far out
    assert np.all(np.isfinite(oracle.silu(np.array([-800.0, 800.0]))))


# ---------------------------------------------------------------- block helpers
def _tiny(act, T=7, H=12, F=16, bias=True, seed=11):
    w = synth.WORKLOADS[4 if act == "swiglu" else 1]
    d = synth.make_unsharded_inputs(w, tokens=T, hidden=H, ffn=F, dtype="f32", seed_base=seed,
                                    b1_std=(0.3 if bias else None))
    # larger weights than the workloads so the activations leave their linear range
    d = {k: (None if v is None else oracle.to_f64(v)) for k, v in d.items()}
    d["W1"] = d["W1"] * 40.0
    d["W2"] = d["W2"] * 10.0
    return d


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("tp", [1, 2, 4])
def test_shard_sum_invariant(act, tp):
    """Column->row pairing is exact: summing the per-rank partial outputs
    reproduces the unsharded block; likewise dx, and the weight gradients
    are the unsharded ones cut along the same splits."""
    d = _tiny(act, bias=(act == "gelu"))
    full = ob.unsharded_backward(d["x"], d["W1"], d["b1"], d["W2"], d["dy"], act)
    ys, dxs, dW1s, dW2s, db1s = [], [], [], [], []
    for r in range(tp):
        W1r, b1r, W2r = oracle.shard_rank(d["W1"], d["b1"], d["W2"], tp, r, act)
        f = oracle.rank_forward(d["x"], W1r, b1r, W2r, act)
        g = oracle.rank_dgrad(d["dy"], W1r, W2r, f["h"], act)
        w = oracle.rank_wgrad(d["dy"], d["x"], f["a"], g["dH"], b1r is not None)
        ys.append(f["y"]); dxs.append(g["dx"]); dW1s.append(w["dW1"]); dW2s.append(w["dW2"])
        db1s.append(w["db1"])
    assert _rel(sum(ys), full["y"]) < 1e-12
    assert _rel(sum(dxs), full["dx"]) < 1e-12
    assert _rel(np.concatenate(dW2s, axis=1), full["dW2"]) < 1e-12
    F = d["W2"].shape[1]
    fs = F // tp
    if act == "gelu":
        assert _rel(np.concatenate(dW1s, axis=0), full["dW1"]) < 1e-12
        assert _rel(np.concatenate(db1s), full["db1"]) < 1e-12
    else:
        gate = np.concatenate([w_[:fs] for w_ in dW1s], axis=0)
        up = np.concatenate([w_[fs:] for w_ in dW1s], axis=0)
        assert _rel(np.concatenate([gate, up], axis=0), full["dW1"]) < 1e-12


def test_swiglu_wrong_split_breaks_invariant():
    """Negative control: giving rank r contiguous rows of the stacked
    [gate; up] matrix (so gate and up no longer match) must not reproduce
    the unsharded block."""
    d = _tiny("swiglu", bias=False)
    full = ob.unsharded_forward(d["x"], d["W1"], None, d["W2"], "swiglu")
    tp, F = 2, d["W2"].shape[1]
    fs = F // tp
    ys = []
    for r in range(tp):
        W1r = d["W1"][r * 2 * fs:(r + 1) * 2 * fs]
        W2r = d["W2"][:, r * fs:(r + 1) * fs]
        ys.append(oracle.rank_forward(d["x"], W1r, None, W2r, "swiglu")["y"])
    assert _rel(sum(ys), full["y"]) > 1e-2


def test_bias_is_inside_activation_and_in_h():
    d = _tiny("gelu")
    f = oracle.rank_forward(d["x"], d["W1"], d["b1"], d["W2"], "gelu")
    f0 = oracle.rank_forward(d["x"], d["W1"], None, d["W2"], "gelu")
    np.testing.assert_allclose(f["h"] - f0["h"], np.broadcast_to(d["b1"], f["h"].shape),
                               atol=1e-12)


# ---------------------------------------------------------------- gradients
@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_gradients_finite_difference_every_entry(act):
    """Central differences of L = sum(dy * y) for every entry of x, W1, b1,
    W2 at T=4, H=6, Fs=5, tp=2 (rank 0's shard)."""
    T, H, F, tp = 4, 6, 10, 2
    d = _tiny(act, T=T, H=H, F=F, bias=(act == "gelu"), seed=23)
    W1, b1, W2 = oracle.shard_rank(d["W1"], d["b1"], d["W2"], tp, 0, act)
    x, dy = d["x"], d["dy"]
    f = oracle.rank_forward(x, W1, b1, W2, act)
    g = oracle.rank_dgrad(dy, W1, W2, f["h"], act)
    w = oracle.rank_wgrad(dy, x, f["a"], g["dH"], b1 is not None)
    params = {"x": (x, g["dx"]), "W1": (W1, w["dW1"]), "W2": (W2, w["dW2"])}
    if b1 is not None:
        params["b1"] = (b1, w["db1"])
    eps = 1e-6
    for name, (p, grad) in params.items():
        fd = np.zeros_like(p)
        for i in np.ndindex(p.shape):
            old = p[i]
            p[i] = old + eps
            lp = ob.block_loss(x, W1, b1, W2, dy, act)
            p[i] = old - eps
            lm = ob.block_loss(x, W1, b1, W2, dy, act)
            p[i] = old
            fd[i] = (lp - lm) / (2 * eps)
        assert _rel(grad, fd) < 1e-6, name


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("T,H,F", [(9, 24, 32), (16, 16, 32), (8, 16, 16)])
def test_gradients_match_torch_autograd(act, T, H, F):
    """The whole rank shard differentiated by torch autograd in float64 (an
    independent implementation of the block and its derivative). Square
    shards (H == G*Fs, or T == H) are included so that a transposed operand
    cannot hide behind a shape error."""
    tp = 2
    d = _tiny(act, T=T, H=H, F=F, bias=(act == "gelu"), seed=31)
    W1, b1, W2 = oracle.shard_rank(d["W1"], d["b1"], d["W2"], tp, 1, act)
    tx, tW1, tW2 = (torch.tensor(v, requires_grad=True) for v in (d["x"], W1, W2))
    tb1 = None if b1 is None else torch.tensor(b1, requires_grad=True)
    hh = tx @ tW1.T + (0 if tb1 is None else tb1)
    if act == "gelu":
        aa = Fn.gelu(hh, approximate="tanh")
    else:
        fs = W1.shape[0] // 2
        aa = Fn.silu(hh[:, :fs]) * hh[:, fs:]
    yy = aa @ tW2.T
    (yy * torch.tensor(d["dy"])).sum().backward()
    f = oracle.rank_forward(d["x"], W1, b1, W2, act)
    g = oracle.rank_dgrad(d["dy"], W1, W2, f["h"], act)
    w = oracle.rank_wgrad(d["dy"], d["x"], f["a"], g["dH"], b1 is not None)
    assert _rel(f["y"], yy.detach().numpy()) < 1e-13
    assert _rel(g["dx"], tx.grad.numpy()) < 1e-12
    assert _rel(w["dW1"], tW1.grad.numpy()) < 1e-12
    assert _rel(w["dW2"], tW2.grad.numpy()) < 1e-12
    if b1 is not None:
        assert _rel(w["db1"], tb1.grad.numpy()) < 1e-12


def test_brute_force_loops_match():
    """Scalar loops over the contractions (activations from torch) at a tiny
    size; catches transposed operands and wrong indices."""
    T, H, F = 3, 5, 4
    d = _tiny("gelu", T=T, H=H, F=F, seed=41)
    x, W1, b1, W2, dy = d["x"], d["W1"], d["b1"], d["W2"], d["dy"]
    act = lambda v: float(Fn.gelu(torch.tensor(v, dtype=torch.float64), approximate="tanh"))

    def dact(v):
        t = torch.tensor(v, dtype=torch.float64, requires_grad=True)
        Fn.gelu(t, approximate="tanh").backward()
        return float(t.grad)

    h = [[b1[j] + sum(x[t][k] * W1[j][k] for k in range(H)) for j in range(F)] for t in range(T)]
    a = [[act(h[t][j]) for j in range(F)] for t in range(T)]
    y = [[sum(a[t][j] * W2[i][j] for j in range(F)) for i in range(H)] for t in range(T)]
    dH = [[sum(dy[t][i] * W2[i][j] for i in range(H)) * dact(h[t][j]) for j in range(F)]
          for t in range(T)]
    dx = [[sum(dH[t][j] * W1[j][k] for j in range(F)) for k in range(H)] for t in range(T)]
    dW2 = [[sum(dy[t][i] * a[t][j] for t in range(T)) for j in range(F)] for i in range(H)]
    dW1 = [[sum(dH[t][j] * x[t][k] for t in range(T)) for k in range(H)] for j in range(F)]
    db1 = [sum(dH[t][j] for t in range(T)) for j in range(F)]
    full = ob.unsharded_backward(x, W1, b1, W2, dy, "gelu")
    for name, ref in (("y", y), ("dx", dx), ("dW2", dW2), ("dW1", dW1), ("db1", db1),
                      ("h", h), ("a", a), ("dH", dH)):
        assert _rel(full[name], np.array(ref)) < 1e-13, name


def test_accumulate_adds_prior_buffers():
    d = _tiny("gelu", seed=5)
    f = oracle.rank_forward(d["x"], d["W1"], d["b1"], d["W2"], "gelu")
    g = oracle.rank_dgrad(d["dy"], d["W1"], d["W2"], f["h"], "gelu")
    w0 = oracle.rank_wgrad(d["dy"], d["x"], f["a"], g["dH"], True)
    rng = np.random.default_rng(0)
    p1 = rng.standard_normal(w0["dW1"].shape)
    pb = rng.standard_normal(w0["db1"].shape)
    p2 = rng.standard_normal(w0["dW2"].shape)
    w1 = oracle.rank_wgrad(d["dy"], d["x"], f["a"], g["dH"], True, p1, pb, p2)
    np.testing.assert_allclose(w1["dW1"], p1 + w0["dW1"], atol=1e-14)
    np.testing.assert_allclose(w1["db1"], pb + w0["db1"], atol=1e-14)
    np.testing.assert_allclose(w1["dW2"], p2 + w0["dW2"], atol=1e-14)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_feature_subsets_give_sampled_outputs(act):
    """Restricting the block to a subset of intermediate features gives exactly
    the matching columns of dW2, rows of dW1 and entries of db1 -- the basis
    of the sampled full-size checks."""
    d = _tiny(act, T=10, H=8, F=12, bias=(act == "gelu"), seed=7)
    full = ob.unsharded_backward(d["x"], d["W1"], d["b1"], d["W2"], d["dy"], act)
    idx = np.array([0, 5, 11])
    W1s, b1s, W2s = oracle.select_features(d["W1"], d["b1"], d["W2"], idx, act)
    f = oracle.rank_forward(d["x"], W1s, b1s, W2s, act)
    g = oracle.rank_dgrad(d["dy"], W1s, W2s, f["h"], act)
    w = oracle.rank_wgrad(d["dy"], d["x"], f["a"], g["dH"], b1s is not None)
    F = d["W2"].shape[1]
    rows = idx if act == "gelu" else np.concatenate([idx, F + idx])
    np.testing.assert_allclose(w["dW2"], full["dW2"][:, idx], atol=1e-12)
    np.testing.assert_allclose(w["dW1"], full["dW1"][rows], atol=1e-12)
    if act == "gelu":
        np.testing.assert_allclose(w["db1"], full["db1"][idx], atol=1e-12)


# ---------------------------------------------------------------- E4M3
def _torch_e4m3_codes(v):
    t = torch.from_numpy(np.clip(np.asarray(v, np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_golden_points_from_ocp_table():
    with open(os.path.join(GOLDEN, "e4m3_ocp_points.txt")) as fh:
        rows = [ln.split()[:2] for ln in fh if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 10
    for code_s, val_s in rows:
        code = int(code_s, 16)
        dec = oracle.e4m3_decode(np.array([code], np.uint8))[0]
        if val_s == "nan":
            assert np.isnan(dec)
        else:
            val = float(val_s)
            assert dec == val and math.copysign(1.0, dec) == math.copysign(1.0, val)
            assert oracle.e4m3_encode(np.array([val]))[0] == code


def test_e4m3_decode_table_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # 253 finite distinct magnitudes incl. signed zeros: max is 448
    assert np.nanmax(ours) == 448.0


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(123)
    vals = [rng.standard_normal(200000).astype(np.float32) * s for s in (1e-3, 0.05, 1, 30, 300)]
    # exact codes, midpoints between neighbours (ties) and their float32 neighbours
    grid = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    grid = np.unique(grid[np.isfinite(grid)])
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(np.inf)),
                           np.nextafter(mids, np.float32(-np.inf))])
    big = np.array([448, 449, 463.9, 464, 480, 1e6, -500, -448.5], np.float32)
    v = np.concatenate(vals + [grid.astype(np.float32), mids, near, big])
    assert np.array_equal(oracle.e4m3_encode(v), _torch_e4m3_codes(v))


def test_e4m3_ties_round_to_even_and_saturate():
    # 1 + 1/16 lies halfway between 1.0 (mantissa 0) and 1.125 (mantissa 1): to even
    assert oracle.e4m3_encode(np.array([1.0625]))[0] == 0x38
    # 1.1875 between 1.125 (odd) and 1.25 (even): up
    assert oracle.e4m3_encode(np.array([1.1875]))[0] == 0x3A
    assert oracle.e4m3_encode(np.array([1e9]))[0] == 0x7E
    assert oracle.e4m3_encode(np.array([-1e9]))[0] == 0xFE
    assert oracle.e4m3_encode(np.array([np.nan]))[0] & 0x7F == 0x7F


def test_current_scaling_recipe():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((64, 96)) * 0.02).astype(np.float32)
    codes, amax, s, s_inv = oracle.quantize_e4m3(v)
    assert amax == np.max(np.abs(v))
    assert s == np.float32(np.float32(448.0) / amax)
    assert s_inv == np.float32(np.float32(1.0) / s)
    deq = oracle.dequantize_e4m3(codes, s_inv)
    # the largest element lands on +-448 in the scaled domain
    i = np.unravel_index(np.argmax(np.abs(v)), v.shape)
    assert abs(oracle.e4m3_decode(codes[i])) == 448.0
    # error bound: half a unit in the last place (2^-4 relative) for normals,
    # half the subnormal spacing (2^-10) for subnormals, in the scaled domain
    bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10 * float(s_inv)) * (1 + 1e-6)
    assert np.all(np.abs(deq - v) <= bound)
    z, amax0, s0, _ = oracle.quantize_e4m3(np.zeros(10, np.float32))
    assert amax0 == 0 and s0 == 1.0 and np.all(z == 0)


def test_scale_of_a_tiny_amax_stays_finite():
    """An amax so small that fmax / amax overflows float32 gives a factor of 1
    (current scaling) or keeps the previous factor (delayed scaling), never
    infinity: zeros then quantise to zero codes (not NaN, 0 * inf) and
    scale_inv stays nonzero. The thresholds are fmax / FLT_MAX: about 1.3e-36
    for E4M3 and 1.7e-34 for E5M2."""
    flt_max = float(np.finfo(np.float32).max)
    for fmt, tiny in (("e4m3", 1e-37), ("e5m2", 1e-35)):
        assert oracle.FMAX[fmt] / tiny > flt_max          # the quotient would overflow
        v = np.array([0.0, tiny, -tiny / 2], np.float32)
        amax, s, s_inv = oracle.current_scale(v, fmt)
        assert amax == np.float32(tiny) and s == 1.0 and s_inv == 1.0
        codes = oracle.quantize(v, fmt, s)
        assert not np.any(np.isnan(oracle.dequantize(codes, fmt, s_inv)))
        assert codes[0] == 0
        _, nxt, inv = oracle.delayed_update(np.zeros(2, np.float32), np.float32(tiny),
                                            np.float32(3.0), fmt)
        assert nxt == np.float32(3.0) and inv == np.float32(np.float32(1.0) / np.float32(3.0))
    # just above the threshold the quotient is finite and used
    amax, s, _ = oracle.current_scale(np.array([2e-36], np.float32), "e4m3")
    assert np.isfinite(s) and s == np.float32(np.float32(448.0) / np.float32(2e-36))


# ---------------------------------------------------------------- E5M2
def _torch_e5m2_codes(v):
    t = torch.from_numpy(np.clip(np.asarray(v, np.float32), -57344.0, 57344.0))
    return t.to(torch.float8_e5m2).view(torch.uint8).numpy()


def test_e5m2_golden_points_from_ocp_table():
    with open(os.path.join(GOLDEN, "e5m2_ocp_points.txt")) as fh:
        rows = [ln.split()[:2] for ln in fh if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 13
    for code_s, val_s in rows:
        code = int(code_s, 16)
        dec = oracle.e5m2_decode(np.array([code], np.uint8))[0]
        if val_s == "nan":
            assert np.isnan(dec)
        elif val_s in ("inf", "-inf"):
            assert dec == float(val_s)
            # saturating conversion: infinities become the largest finite value
            assert oracle.e5m2_encode(np.array([float(val_s)]))[0] == (0x7B | (code & 0x80))
        else:
            val = float(val_s)
            assert dec == val and math.copysign(1.0, dec) == math.copysign(1.0, val)
            assert oracle.e5m2_encode(np.array([val]))[0] == code


def test_e5m2_decode_table_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    ours = oracle.e5m2_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.nanmax(ours[np.isfinite(ours)]) == 57344.0


def test_e5m2_encode_matches_torch_cast_and_round_trips():
    rng = np.random.default_rng(321)
    vals = [rng.standard_normal(200000).astype(np.float32) * s for s in (1e-4, 0.01, 1, 300, 20000)]
    grid = oracle.e5m2_decode(np.arange(256, dtype=np.uint8))
    grid = np.unique(grid[np.isfinite(grid)])
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(np.inf)),
                           np.nextafter(mids, np.float32(-np.inf))])
    v = np.concatenate(vals + [grid.astype(np.float32), mids, near])
    assert np.array_equal(oracle.e5m2_encode(v), _torch_e5m2_codes(v))
    finite = np.arange(256, dtype=np.uint8)
    finite = finite[np.isfinite(oracle.e5m2_decode(finite))]
    back = oracle.e5m2_encode(oracle.e5m2_decode(finite))
    assert np.array_equal(back, finite)


def test_e5m2_ties_round_to_even_and_saturate():
    # 1.125 lies halfway between 1.0 (mantissa 0) and 1.25 (mantissa 1): to even
    assert oracle.e5m2_encode(np.array([1.125]))[0] == 0x3C
    # 1.375 between 1.25 (odd) and 1.5 (even): up
    assert oracle.e5m2_encode(np.array([1.375]))[0] == 0x3E
    for big in (57345.0, 60000.0, 61440.0, 1e30, np.inf):
        assert oracle.e5m2_encode(np.array([big]))[0] == 0x7B
        assert oracle.e5m2_encode(np.array([-big]))[0] == 0xFB
    assert oracle.e5m2_encode(np.array([np.nan]))[0] & 0x7F == 0x7F


def test_quantize_error_bounds_both_formats():
    rng = np.random.default_rng(9)
    v = (rng.standard_normal(5000) * 3).astype(np.float32)
    for fmt, mant, sub in (("e4m3", 3, 2.0 ** -9), ("e5m2", 2, 2.0 ** -16)):
        s = np.float32(oracle.FMAX[fmt] / np.max(np.abs(v)))
        deq = oracle.dequantize(oracle.quantize(v, fmt, s), fmt, np.float32(1) / s)
        # half a unit in the last place in the scaled domain
        bound = np.maximum(np.abs(v) * 2.0 ** -(mant + 1), sub / 2 / float(s)) * (1 + 1e-6)
        assert np.all(np.abs(deq - v) <= bound), fmt
        assert np.max(np.abs(deq)) <= np.max(np.abs(v)) * (1 + 2.0 ** -(mant + 1))


def test_delayed_scaling_steps():
    # a history of 4, e4m3: hand-worked steps
    h = np.zeros(4, np.float32)
    s = np.float32(1.0)
    h, s2, sinv = oracle.delayed_update(h, np.float32(2.0), s, "e4m3")
    assert list(h) == [2, 0, 0, 0] and s2 == np.float32(224.0) and sinv == 1.0
    h, s3, sinv = oracle.delayed_update(h, np.float32(8.0), s2, "e4m3")
    assert list(h) == [8, 2, 0, 0] and s3 == np.float32(56.0)
    assert sinv == np.float32(np.float32(1) / np.float32(224))
    h, s4, _ = oracle.delayed_update(h, np.float32(1.0), s3, "e4m3")
    assert list(h) == [1, 8, 2, 0] and s4 == np.float32(56.0)   # the max is still 8
    h, s5, _ = oracle.delayed_update(h, np.float32(1.0), s4, "e4m3")
    h, s6, _ = oracle.delayed_update(h, np.float32(1.0), s5, "e4m3")
    assert list(h) == [1, 1, 1, 8] and s6 == np.float32(56.0)
    h, s7, _ = oracle.delayed_update(h, np.float32(1.0), s6, "e4m3")
    assert list(h) == [1, 1, 1, 1] and s7 == np.float32(448.0)  # 8 has left the window
    # e5m2 uses its own largest finite value
    _, s8, _ = oracle.delayed_update(np.zeros(2, np.float32), np.float32(4.0), s, "e5m2")
    assert s8 == np.float32(14336.0)
    # a zero or non-finite history keeps the previous scale
    _, s9, _ = oracle.delayed_update(np.zeros(3, np.float32), np.float32(0.0), np.float32(7), "e4m3")
    assert s9 == np.float32(7)
    _, s10, _ = oracle.delayed_update(np.zeros(3, np.float32), np.float32(np.inf), np.float32(7), "e4m3")
    assert s10 == np.float32(7)


def test_round_bf16_matches_torch_cast():
    """Round-to-nearest-even float32 -> bfloat16, against torch's CPU cast:
    random magnitudes over many binades, exact ties either side of an even
    and an odd kept part, subnormals and signed zeros."""
    from oracle.fp8_block import round_bf16
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-130, 120, 20000))).astype(np.float32)
    kept = rng.integers(0, 1 << 16, 2000).astype(np.uint32) << 16
    ties = (kept | 0x8000).view(np.float32)          # exactly halfway
    near = np.concatenate([(kept | 0x7FFF), (kept | 0x8001)]).view(np.float32)
    v = np.concatenate([v, ties, near, np.float32([0.0, -0.0, 1e-45, -3e-39])])
    v = v[np.isfinite(v)]
    want = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    got = round_bf16(v)
    assert np.array_equal(got, want) and np.array_equal(np.signbit(got), np.signbit(want))
    # ties go to the even kept part: 1 + 2^-8 -> 1, 1 + 3 * 2^-8 -> 1 + 2^-6
    assert round_bf16(np.float32(1 + 2.0 ** -8)) == 1.0
    assert round_bf16(np.float32(1 + 3 * 2.0 ** -8)) == 1 + 2.0 ** -6


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_fp8_block_is_the_plain_block_within_quantisation_bounds(act):
    """The FP8 block's unquantised intermediates are the plain block's; its
    outputs differ from the plain block by no more than the rounding bound
    of the quantised intermediates (a in E4M3, dH in E5M2) carried through
    the following products."""
    rng = np.random.default_rng(17)
    T, H, Fs = 24, 40, 32
    G = 2 if act == "swiglu" else 1
    x = rng.standard_normal((T, H))
    W1 = rng.standard_normal((G * Fs, H)) * 0.2
    b1 = rng.standard_normal(G * Fs) * 0.1
    W2 = rng.standard_normal((H, Fs)) * 0.2
    dy = rng.standard_normal((T, H))
    f = ob.rank_forward(x, W1, b1, W2, act)
    a_scale = np.float32(448.0 / np.max(np.abs(f["a"])))
    q = oracle.rank_forward_fp8(x, W1, b1, W2, a_scale, act)
    # the unquantised intermediates are the plain block's, float64 throughout
    assert np.allclose(q["h"], f["h"], rtol=0, atol=1e-13)
    assert np.allclose(q["a"], f["a"], rtol=0, atol=1e-13)
    assert q["amax"] == pytest.approx(float(np.max(np.abs(f["a"]))), rel=1e-13)
    da = np.maximum(np.abs(q["a"]) * 2.0 ** -4, 2.0 ** -10 / float(a_scale)) * (1 + 1e-6)
    assert np.all(np.abs(q["a_q"] - q["a"]) <= da)
    assert np.all(np.abs(q["y"] - f["y"]) <= da @ np.abs(W2.T) + 1e-12)
    assert np.any(q["a_q"] != q["a"])               # the quantisation is not a no-op
    g = ob.rank_dgrad(dy, W1, W2, f["h"], act)
    dH_scale = np.float32(57344.0 / np.max(np.abs(g["dH"])) / 4)
    p = oracle.rank_dgrad_fp8(dy, W1, W2, f["h"], dH_scale, act)
    assert np.allclose(p["dH"], g["dH"], rtol=0, atol=1e-12)
    dh = np.maximum(np.abs(g["dH"]) * 2.0 ** -3, 2.0 ** -17 / float(dH_scale)) * (1 + 1e-6)
    assert np.all(np.abs(p["dH_q"] - g["dH"]) <= dh)
    assert np.all(np.abs(p["dx"] - g["dx"]) <= dh @ np.abs(W1) + 1e-12)
    w = oracle.rank_wgrad_fp8(dy, x, q["a_q"], p["dH_q"])
    ref = ob.rank_wgrad(dy, x, f["a"], g["dH"], True)
    assert np.all(np.abs(w["dW2"] - ref["dW2"]) <= np.abs(dy.T) @ da + 1e-12)
    assert np.all(np.abs(w["dW1"] - ref["dW1"]) <= dh.T @ np.abs(x) + 1e-12)
    assert np.all(np.abs(w["db1"] - ref["db1"]) <= dh.sum(axis=0) + 1e-12)
    # with every intermediate exactly representable the FP8 block is the plain one:
    # an all-zero gradient quantises exactly
    z = oracle.rank_dgrad_fp8(np.zeros((T, H)), W1, W2, f["h"], dH_scale, act)
    assert np.all(z["dH_codes"] & 0x7F == 0) and np.all(z["dx"] == 0)
    if act == "swiglu":
        # the gate half of dH carries up * silu'(gate), the up half silu(gate):
        # with up = 0 the gate half vanishes and the up half does not
        fs = Fs
        W1z = W1.copy()
        W1z[fs:] = 0.0
        fz = oracle.rank_forward_fp8(x, W1z, np.concatenate([b1[:fs], np.zeros(fs)]), W2,
                                     a_scale, act)
        assert np.all(fz["a"] == 0) and np.all(fz["a_codes"] & 0x7F == 0)
        gz = oracle.rank_dgrad_fp8(dy, W1z, W2, fz["h"], dH_scale, act)
        assert np.all(gz["dH"][:, :fs] == 0) and np.any(gz["dH"][:, fs:] != 0)
    with pytest.raises(ValueError):
        oracle.rank_forward_fp8(x, W1, b1, W2, a_scale, "relu")


def test_activation_bounds_of_the_fp8_gpu_windows():
    """The slope and curvature bounds the FP8 GPU tests widen their windows
    with hold for the oracle's activations on a fine grid (the maxima of
    |gelu'|, |gelu''|, |silu'|, |silu''|; second derivatives by central
    differences of the first)."""
    from test_gpu_fp8_bwd import GELU_CURV, GELU_SLOPE, SILU_CURV, SILU_SLOPE
    from oracle.activations import gelu_tanh_grad, silu_grad
    z = np.linspace(-30.0, 30.0, 600001)
    e = 1e-5
    for grad, slope, curv in ((gelu_tanh_grad, GELU_SLOPE, GELU_CURV),
                              (silu_grad, SILU_SLOPE, SILU_CURV)):
        g1 = np.abs(grad(z))
        g2 = np.abs((grad(z + e) - grad(z - e)) / (2 * e))
        assert np.max(g1) <= slope and np.max(g1) > 0.97 * slope
        assert np.max(g2) <= curv and np.max(g2) > 0.97 * curv


# ---------------------------------------------------------------- inputs
def test_synth_is_deterministic_and_shaped():
    w = synth.WORKLOADS[2]
    a = synth.make_rank_inputs(w, tokens=16, hidden=32, ffn_shard=24)
    b = synth.make_rank_inputs(w, tokens=16, hidden=32, ffn_shard=24)
    assert a["x"].dtype == torch.bfloat16 and a["x"].shape == (16, 32)
    assert a["W1"].shape == (24, 32) and a["W2"].shape == (32, 24) and a["b1"].shape == (24,)
    for k in ("x", "W1", "W2", "b1", "dy"):
        assert torch.equal(a[k], b[k])
    w4 = synth.WORKLOADS[4]
    s = synth.make_rank_inputs(w4, tokens=8, hidden=16, ffn_shard=12)
    assert s["W1"].shape == (24, 16) and s["b1"] is None
    assert w4.flops() == 6 * 8192 * 4096 * 7168 * 3
    assert synth.WORKLOADS[3].flops() == pytest.approx(3.2985e12, rel=1e-4)
