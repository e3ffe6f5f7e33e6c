"""GPU parity of the FP8 backward and of delayed scaling (OCP E4M3 forward
tensors, OCP E5M2 gradients).

* The E5M2 quantiser is bit-exact against the oracle's encoder (same float32
  product v * scale decides the code).
* Delayed scaling: the history rolls, the call quantises with the scale it
  was given and reports 1 / that scale, and the next scale follows
  fmax / max(history).
* The FP8 block forward + dgrad + wgrad runs through the C ABI on codes the
  GPU quantiser produced (first checked equal to the oracle's own) and is
  compared with the oracle's FP8 block on the dequantised inputs, which
  quantises a (E4M3) and dH (E5M2) at the same given scales.

The codes of a and dH are decided by floating point on both sides, from a
float32 product sum on the device and a float64 one in the oracle, so a
value that falls within that difference of a rounding boundary may take
either neighbour. Such codes are checked for validity: every device code
must be the rounding of some value within delta of the oracle's exact
value, delta being a bound on the device's arithmetic error (for a product
sum, 1.5e-4 of the largest |sum|: the FP8 matrix instructions do not sum
exactly in float32); every code whose value is not that close to a boundary
is then equal to the oracle's. The same holds for h at bf16. Tensors computed from
identical FP8 inputs (the weight gradients given the oracle's codes) are
held to 1e-4 of max |oracle| (float32 accumulation only); tensors after a
quantised intermediate to 6e-2, and the weight gradients of the chained
calls, which take the device's own codes, to the difference those codes make
(exact, element by element) plus 1e-4."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu_helpers import TOL, rel_err, require_gpu, say
from oracle.fp8_block import round_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tp():
    require_gpu()
    import tensor_transformer_mlp_rank_amd as m
    return m


def _f32(x):
    return np.float32(x)


@pytest.mark.parametrize("src", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 1000, 65537, 2 * 1024 * 1024 + 3])
def test_e5m2_quantizer_bit_exact(tp, src, n):
    rng = np.random.default_rng(n + 11)
    v = (rng.standard_normal(n) * rng.choice([1e-4, 0.05, 30.0], size=n)).astype(np.float32)
    if n > 5000:
        # grid points, ties and their neighbours in the scaled domain
        grid = oracle.e5m2_decode(np.arange(256, dtype=np.uint8))
        grid = np.unique(grid[np.isfinite(grid)])
        mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
        sp = np.concatenate([grid.astype(np.float32), mids, np.nextafter(mids, np.float32(np.inf))])
        v[: sp.size] = (sp / 57344.0 * float(np.max(np.abs(v)))).astype(np.float32)
    t = torch.from_numpy(v)
    if src == "bf16":
        t = t.to(torch.bfloat16)
    say(f"quantize e5m2 src={src} n={n}")
    codes, amax, sinv = tp.quantize_e5m2(t.cuda())
    torch.cuda.synchronize()
    vv = t.float().numpy()
    ramax = _f32(np.max(np.abs(vv)))
    rs = _f32(_f32(57344.0) / ramax)
    assert float(amax.cpu()[0]) == float(ramax)
    assert float(sinv.cpu()[0]) == float(_f32(_f32(1.0) / rs))
    rc = oracle.quantize(vv, "e5m2", rs)
    got = codes.cpu().numpy()
    mism = np.nonzero(got != rc)[0]
    assert mism.size == 0, f"{mism.size} codes differ, first at {mism[:5]}"


def _quantized_inputs(tp, inp, with_dy=True):
    """GPU codes of x, W1, W2 (E4M3) and dy (E5M2), each checked equal to the
    oracle's; returns (device codes and scale_inv tensors, dequantised f64)."""
    dev, deq = {}, {}
    fmts = {"x": "e4m3", "W1": "e4m3", "W2": "e4m3"}
    if with_dy:
        fmts["dy"] = "e5m2"
    for k, fmt in fmts.items():
        v = inp[k].float()
        codes, amax, sinv = tp.quantize_e4m3(v.cuda(), e5m2=(fmt == "e5m2"))
        vv = v.numpy()
        s = _f32(_f32(oracle.FMAX[fmt]) / _f32(np.max(np.abs(vv))))
        rc = oracle.quantize(vv, fmt, s)
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy(), rc), k
        assert float(sinv.cpu()[0]) == float(_f32(_f32(1.0) / s)), k
        dev[k] = (codes, sinv)
        deq[k] = oracle.dequantize(rc, fmt, _f32(_f32(1.0) / s))
    return dev, deq


def _scale_for(amax, fmt):
    return _f32(_f32(oracle.FMAX[fmt]) / _f32(amax))


# Error bounds for device results that decide a rounding. The FP8 matrix
# instructions do not sum their products exactly in float32: measured against
# exact sums, their results carry errors up to about 3e-5 of the largest
# |result| of a product (5e-5 with heavy-tailed inputs, and up to 1.1e-4 for
# the gated block's weight gradients over about 100 tokens, whose operands
# are products of Gaussians), some hundred float32 ulps, so the bound on a
# product sum is 1.5e-4 of the largest |sum| in its tensor; on the float32
# activation arithmetic after it, 1e-5 of the value.
SUM_ERR, REL_ERR = 1.5e-4, 1e-5
# products of identical FP8 inputs, against max |oracle|: the same bound
EXACT_TOL = SUM_ERR


def _valid_rounding(got, t, d, rnd):
    """got lies between rnd(t - d) and rnd(t + d): the rounding (monotone)
    of some value within d of t."""
    return (got >= rnd(t - d)) & (got <= rnd(t + d))


def _check_codes(name, codes_dev, t, d, fmt, ref_codes):
    """Device FP8 codes against the exact scaled values t (float64) within
    delta d; reports how many differ in value from the oracle's own codes
    (the codes of +0 and -0 are one value: where the exact GELU slope is a
    tiny negative number the device's underflows to +0, and the two zeros of
    dH then differ in sign only)."""
    got = oracle.dequantize(codes_dev.cpu().numpy(), fmt, 1.0)
    rnd = lambda v: oracle.dequantize(oracle.quantize(v, fmt, 1.0), fmt, 1.0)
    ok = _valid_rounding(got, t, d, rnd)
    n_diff = int(np.count_nonzero(got != oracle.dequantize(ref_codes, fmt, 1.0)))
    say(f"    {name}: {n_diff} of {ref_codes.size} codes are the other neighbour")
    bad = np.argwhere(~ok)
    assert bad.size == 0, (name, bad[:5].tolist(), got[~ok][:5], t[~ok][:5])
    assert n_diff <= max(8, ref_codes.size // 20), (name, n_diff)


def _amax(v):
    return float(np.max(np.abs(v), initial=0.0))


def _check_h(h_dev, h_exact):
    """Stored h (bf16) against the oracle's exact h; returns the bf16 values
    either side of the oracle's range [lo, hi], for the next tolerance."""
    d = REL_ERR * np.abs(h_exact) + SUM_ERR * _amax(h_exact)
    lo, hi = round_bf16(h_exact - d), round_bf16(h_exact + d)
    got = oracle.to_f64(h_dev.cpu())
    ok = (got >= lo) & (got <= hi)
    assert np.all(ok), (np.argwhere(~ok)[:5].tolist(), got[~ok][:5], h_exact[~ok][:5])
    return lo, hi


# The oracle takes the activation of its exact h; the device takes it of h as
# stored in bf16, somewhere in [lo, hi]. Bounds on how far that moves the
# activation and its derivative: |gelu'| <= 1.129 and |gelu''| <= sqrt(2/pi)
# = 0.798 for the tanh form (both maxima found on a fine grid of the oracle's
# functions; the second is gelu''(0)).
GELU_SLOPE, GELU_CURV = 1.13, 0.80
# The same for SiLU: |silu'| <= 1.0998 (near z = 2.4) and |silu''| <= 1/2
# (silu''(0)).
SILU_SLOPE, SILU_CURV = 1.10, 0.50


def _h_span(h, lo, hi):
    """Largest distance from the exact h to a device h in [lo, hi]."""
    return np.maximum(np.abs(hi - h), np.abs(h - lo))


def _a_delta(rf, lo, hi):
    """delta for a (unscaled): float32 error of gelu and gelu's change
    between the exact h and any device h in [lo, hi]."""
    a = rf["a"]
    return REL_ERR * np.abs(a) + 1e-6 * _amax(a) + GELU_SLOPE * _h_span(rf["h"], lo, hi)


def _dH_delta(rg, h, lo, hi):
    """delta for dH (unscaled): the product sum dA's error through gelu'
    (|gelu'| < 1.13), the float32 error of the product, and gelu''s change
    between the exact h and any device h in [lo, hi]."""
    dA = rg["dA"]
    d = REL_ERR * np.abs(rg["dH"]) + GELU_SLOPE * SUM_ERR * _amax(dA)
    return d + np.abs(dA) * GELU_CURV * _h_span(h, lo, hi)


def _halves(v):
    fs = v.shape[1] // 2
    return v[:, :fs], v[:, fs:]


def _a_delta_swiglu(rf, lo, hi):
    """delta for the gated block's a = silu(g) u (unscaled), the device's g
    and u anywhere in their windows: silu(g_d) u_d - silu(g) u =
    (silu(g_d) - silu(g)) u_d + silu(g) (u_d - u), plus the float32 error."""
    g, u = _halves(rf["h"])
    (glo, ulo), (ghi, uhi) = _halves(lo), _halves(hi)
    u_max = np.maximum(np.abs(ulo), np.abs(uhi))
    a = rf["a"]
    return (REL_ERR * np.abs(a) + 1e-6 * _amax(a) + SILU_SLOPE * _h_span(g, glo, ghi) * u_max
            + np.abs(oracle.silu(g)) * _h_span(u, ulo, uhi))


def _dH_delta_swiglu(rg, h, lo, hi):
    """delta for the gated block's dH halves (unscaled), with dA's product-sum
    error e (|e| <= SUM_ERR max|dA|) and the device's g, u in their windows:
      dg: e u_d s'(g_d) + dA (u_d - u) s'(g_d) + dA u (s'(g_d) - s'(g))
      du: e silu(g_d) + dA (silu(g_d) - silu(g))
    (s = silu; |s'| <= SILU_SLOPE, |s''| <= SILU_CURV), plus the float32 error."""
    dA = rg["dA"]
    e = SUM_ERR * _amax(dA)
    g, u = _halves(h)
    (glo, ulo), (ghi, uhi) = _halves(lo), _halves(hi)
    sg, su = _h_span(g, glo, ghi), _h_span(u, ulo, uhi)
    u_max = np.maximum(np.abs(ulo), np.abs(uhi))
    d_g = e * u_max * SILU_SLOPE + np.abs(dA) * su * SILU_SLOPE + np.abs(dA * u) * SILU_CURV * sg
    d_u = e * (np.abs(oracle.silu(g)) + SILU_SLOPE * sg) + np.abs(dA) * SILU_SLOPE * sg
    return REL_ERR * np.abs(rg["dH"]) + np.concatenate([d_g, d_u], axis=1)


def test_delayed_scaling_forward_two_calls(tp):
    """Two forward calls with a history of 3: each quantises a at the scale it
    is given, reports 1 / that scale, rolls the history and sets the next
    scale from it; outputs match the oracle's FP8 block at those scales."""
    T, H, Fs = 300, 528, 272
    w = synth.WORKLOADS[5]
    inp = synth.make_rank_inputs(w, tokens=T, hidden=H, ffn_shard=Fs, seed_base=710)
    dev, deq = _quantized_inputs(tp, inp, with_dy=False)
    b1 = oracle.to_f64(inp["b1"])
    ref0 = oracle.rank_forward(deq["x"], deq["W1"], b1, deq["W2"], "gelu")
    amax_ref = float(np.max(np.abs(ref0["a"])))
    hist = tp.DelayedScaling(3, scale=float(_scale_for(amax_ref, "e4m3") / 2))
    prior = np.array([0.5, 0.25, 0.125], np.float32)          # earlier amaxes
    hist.amax_history.copy_(torch.from_numpy(prior))
    desc = tp.make_desc(T, H, Fs, act="gelu", dtype="e4m3", has_bias=True)
    scales = (dev["x"][1], dev["W1"][1], dev["W2"][1])
    for call in range(2):
        s_in = _f32(hist.scale.cpu()[0])
        h_before = hist.amax_history.cpu().numpy().copy()
        say(f"  delayed forward call {call}: scale {float(s_in):.6g}")
        out = tp.fwd(desc, dev["x"][0], dev["W1"][0], inp["b1"].cuda(), dev["W2"][0],
                     fp8_in_scales=scales, a_history=hist)
        torch.cuda.synchronize()
        h_after = hist.amax_history.cpu().numpy()
        s_out = _f32(hist.scale.cpu()[0])
        sinv = _f32(hist.scale_inv.cpu()[0])
        ref = oracle.rank_forward_fp8(deq["x"], deq["W1"], b1, deq["W2"], s_in)
        # the history rolled and took this call's amax
        assert np.array_equal(h_after[1:], h_before[:-1])
        # 1 / the factor used; the next factor from the whole history
        assert sinv == _f32(_f32(1.0) / s_in)
        assert s_out == _f32(_f32(448.0) / _f32(np.max(h_after)))
        lo, hi = _check_h(out["h"], ref["h_exact"])
        da = _a_delta(ref, lo, hi)
        _check_codes("a", out["a"], ref["a"] * float(s_in), da * float(s_in), "e4m3", ref["a_codes"])
        assert abs(float(h_after[0]) - ref["amax"]) <= float(np.max(da))
        e_y = rel_err(out["y"].cpu(), ref["y"])
        say(f"    rel error y={e_y:.2e}")
        assert e_y <= TOL["e4m3"]


def _check_through_codes(name, got, ref, d_in, M):
    """A bf16 product of the device's own codes against the oracle's product
    of its codes: element by element within the codes' differences d_in
    carried through the product (d_in @ |M|), the bf16 rounding of the
    stored result and the float32 accumulation of identical inputs."""
    g = oracle.to_f64(got.cpu())
    lim = (d_in @ np.abs(M)) * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ref) + EXACT_TOL * _amax(ref)
    excess = np.abs(g - ref) - lim
    assert np.all(excess <= 0), (name, float(np.max(excess)))


def _fp8_block(tp, T, H, Fs, seed, prior=False, act="gelu"):
    """Each entry point on the oracle's own inputs (forward on the quantised
    x, W1, W2; dgrad also on the oracle's stored h; wgrad on the oracle's
    codes of a and dH), then the three chained on the device's own outputs,
    as a training step runs them. act "swiglu": the gated block (no bias),
    with the value distributions of the gated workload."""
    gated = act == "swiglu"
    w = synth.WORKLOADS[4 if gated else 5]
    G = 2 if gated else 1
    inp = synth.make_rank_inputs(w, tokens=T, hidden=H, ffn_shard=Fs, dtype="e4m3",
                                 seed_base=seed)
    dev, deq = _quantized_inputs(tp, inp)
    b1 = None if inp["b1"] is None else oracle.to_f64(inp["b1"])
    b1_dev = None if inp["b1"] is None else inp["b1"].cuda()
    a_delta = _a_delta_swiglu if gated else _a_delta
    dH_delta = _dH_delta_swiglu if gated else _dH_delta
    # the scales a and dH are quantised with (given to both sides): from the
    # plain block's amaxes, halved, so that the test also covers codes that
    # are not at the top of the range
    f0 = oracle.rank_forward(deq["x"], deq["W1"], b1, deq["W2"], act)
    g0 = oracle.rank_dgrad(deq["dy"], deq["W1"], deq["W2"], f0["h"], act)
    a_scale = _f32(_scale_for(np.max(np.abs(f0["a"])), "e4m3") / 2)
    dH_scale = _f32(_scale_for(np.max(np.abs(g0["dH"])), "e5m2") / 2)
    a_sinv, dH_sinv = _f32(_f32(1.0) / a_scale), _f32(_f32(1.0) / dH_scale)
    rf = oracle.rank_forward_fp8(deq["x"], deq["W1"], b1, deq["W2"], a_scale, act)
    rg = oracle.rank_dgrad_fp8(deq["dy"], deq["W1"], deq["W2"], rf["h"], dH_scale, act)
    pr = None
    if prior:
        pr = {"dW1": synth.grad_init(5, (G * Fs, H), 1),
              "db1": None if gated else synth.grad_init(5, (Fs,), 2),
              "dW2": synth.grad_init(5, (H, Fs), 3)}
    prior_args = () if pr is None else tuple(None if pr[k] is None else pr[k].double().numpy()
                                             for k in ("dW1", "db1", "dW2"))
    rw = oracle.rank_wgrad_fp8(deq["dy"], deq["x"], rf["a_q"], rg["dH_q"], *prior_args)
    desc = tp.make_desc(T, H, Fs, act=act, dtype="e4m3", has_bias=not gated)
    wkeys = ("dW1", "dW2") if gated else ("dW1", "db1", "dW2")
    fp8_fwd = (dev["x"][1], dev["W1"][1], dev["W2"][1])
    fp8_dgrad = lambda hist: dict(dy_scale_inv=dev["dy"][1], w1_scale_inv=dev["W1"][1],
                                  w2_scale_inv=dev["W2"][1], dH_history=hist)
    cu = lambda v: torch.tensor([float(v)], dtype=torch.float32, device="cuda")
    fp8_wgrad = lambda a_si, dH_si: dict(dy_scale_inv=dev["dy"][1], x_scale_inv=dev["x"][1],
                                         a_scale_inv=a_si, dH_scale_inv=dH_si)
    acc = lambda: None if pr is None else {k: (None if v is None else v.cuda())
                                           for k, v in pr.items()}
    say(f"  e4m3 {act} block T={T} H={H} Fs={Fs}")

    # forward
    ah = tp.DelayedScaling(2, scale=float(a_scale))
    f = tp.fwd(desc, dev["x"][0], dev["W1"][0], b1_dev, dev["W2"][0],
               fp8_in_scales=fp8_fwd, a_history=ah)
    torch.cuda.synchronize()
    lo, hi = _check_h(f["h"], rf["h_exact"])
    da = a_delta(rf, lo, hi)
    _check_codes("a", f["a"], rf["a"] * float(a_scale), da * float(a_scale), "e4m3", rf["a_codes"])
    assert float(ah.scale_inv.cpu()[0]) == float(a_sinv)
    assert abs(float(ah.amax_history.cpu()[0]) - rf["amax"]) <= float(np.max(da))
    errs = {"y": rel_err(f["y"].cpu(), rf["y"])}
    d_a = np.abs(oracle.dequantize(f["a"].cpu().numpy(), "e4m3", a_sinv) - rf["a_q"])
    _check_through_codes("y", f["y"], rf["y"], d_a, deq["W2"].T)

    # dgrad on the oracle's h, rounded to bf16 (the stored type)
    h_bf = round_bf16(rf["h"])
    h_or = torch.from_numpy(h_bf.astype(np.float32)).to(torch.bfloat16).cuda()
    dh = tp.DelayedScaling(2, scale=float(dH_scale))
    g = tp.bwd_dgrad(desc, dev["dy"][0], dev["W1"][0], dev["W2"][0], h_or, fp8=fp8_dgrad(dh))
    torch.cuda.synchronize()
    ddH = dH_delta(rg, rf["h"], h_bf, h_bf)
    _check_codes("dH", g["dH"], rg["dH"] * float(dH_scale), ddH * float(dH_scale), "e5m2",
                 rg["dH_codes"])
    assert float(dh.scale_inv.cpu()[0]) == float(dH_sinv)
    assert abs(float(dh.amax_history.cpu()[0]) - rg["amax"]) <= float(np.max(ddH))
    errs["dx"] = rel_err(g["dx"].cpu(), rg["dx"])
    d_dH1 = np.abs(oracle.dequantize(g["dH"].cpu().numpy(), "e5m2", dH_sinv) - rg["dH_q"])
    _check_through_codes("dx", g["dx"], rg["dx"], d_dH1, deq["W1"])

    # wgrad on the oracle's codes: identical FP8 inputs
    wg = tp.bwd_wgrad(desc, dev["dy"][0], dev["x"][0],
                      torch.from_numpy(rf["a_codes"]).cuda(), torch.from_numpy(rg["dH_codes"]).cuda(),
                      accumulate_into=acc(), fp8=fp8_wgrad(cu(a_sinv), cu(dH_sinv)))
    torch.cuda.synchronize()
    exact = {k: rel_err(wg[k].cpu(), rw[k]) for k in wkeys}
    # the same from token-contiguous copies of the codes (tpmlp_bwd_wgrad_t)
    codes_t = {"dy": tp.transpose_u8(dev["dy"][0]), "x": tp.transpose_u8(dev["x"][0]),
               "a": tp.transpose_u8(torch.from_numpy(rf["a_codes"]).cuda()),
               "dH": tp.transpose_u8(torch.from_numpy(rg["dH_codes"]).cuda())}
    wt = tp.bwd_wgrad_t(desc, codes_t["dy"], codes_t["x"], codes_t["a"], codes_t["dH"],
                        accumulate_into=acc(), fp8=fp8_wgrad(cu(a_sinv), cu(dH_sinv)))
    torch.cuda.synchronize()
    exact.update({k + " (t)": rel_err(wt[k].cpu(), rw[k]) for k in wkeys})
    say("    given codes: " + " ".join(f"{k}={v:.2e}" for k, v in exact.items()))
    for k, v in exact.items():
        assert v <= EXACT_TOL, (k, v)

    # the chain, on the device's own h, a and dH
    dh2 = tp.DelayedScaling(2, scale=float(dH_scale))
    g2 = tp.bwd_dgrad(desc, dev["dy"][0], dev["W1"][0], dev["W2"][0], f["h"], fp8=fp8_dgrad(dh2))
    wg2 = tp.bwd_wgrad(desc, dev["dy"][0], dev["x"][0], f["a"], g2["dH"], accumulate_into=acc(),
                       fp8=fp8_wgrad(ah.scale_inv, dh2.scale_inv))
    torch.cuda.synchronize()
    _check_codes("dH (chain)", g2["dH"], rg["dH"] * float(dH_scale),
                 dH_delta(rg, rf["h"], lo, hi) * float(dH_scale), "e5m2", rg["dH_codes"])
    errs["dx (chain)"] = rel_err(g2["dx"].cpu(), rg["dx"])
    # The chain's results differ from the oracle's only through the codes of
    # a and dH that took the other neighbour (each a valid rounding, checked
    # above): element by element, by at most those differences carried
    # through the products, plus the float32 accumulation of identical inputs.
    d_dH = np.abs(oracle.dequantize(g2["dH"].cpu().numpy(), "e5m2", dH_sinv) - rg["dH_q"])
    _check_through_codes("dx (chain)", g2["dx"], rg["dx"], d_dH, deq["W1"])
    bound = {"dW2": np.abs(deq["dy"]).T @ d_a, "dW1": d_dH.T @ np.abs(deq["x"]),
             "db1": d_dH.sum(axis=0)}
    chain = {}
    for k in wkeys:
        chain[k] = rel_err(wg2[k].cpu(), rw[k])
        excess = np.abs(oracle.to_f64(wg2[k].cpu()) - rw[k]) - bound[k] - EXACT_TOL * _amax(rw[k])
        assert np.all(excess <= 0), (k, float(np.max(excess)))
    # the chain's weight gradients from token-contiguous copies of its codes
    wt2 = tp.bwd_wgrad_t(desc, codes_t["dy"], codes_t["x"], tp.transpose_u8(f["a"]),
                         tp.transpose_u8(g2["dH"]), accumulate_into=acc(),
                         fp8=fp8_wgrad(ah.scale_inv, dh2.scale_inv))
    torch.cuda.synchronize()
    for k in wkeys:
        e_t = rel_err(wt2[k].cpu(), oracle.to_f64(wg2[k].cpu()))
        assert e_t <= EXACT_TOL, (k, e_t)
    # selective recomputation: a's codes from the saved h at 1 / a_scale_inv;
    # where that factor is the forward's, the codes and so the results are
    # the saved path's bit for bit (dW1 and db1, which do not read a, always)
    wg3 = tp.bwd_wgrad(desc, dev["dy"][0], dev["x"][0], f["h"], g2["dH"], accumulate_into=acc(),
                       fp8=fp8_wgrad(ah.scale_inv, dh2.scale_inv), recompute=True)
    torch.cuda.synchronize()
    same_factor = _f32(_f32(1.0) / a_sinv) == a_scale
    for k in wkeys:
        if same_factor or k != "dW2":
            assert torch.equal(wg3[k], wg2[k]), k
    # otherwise a's recomputed codes differ from the saved ones only where the
    # scaled value lies within a float32 rounding of a code boundary
    rec = rel_err(wg3["dW2"].cpu(), oracle.to_f64(wg2["dW2"].cpu()))
    say("    rel errors (each within the bound of its codes) "
        + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) + " "
        + " ".join(f"{k} (chain)={v:.2e}" for k, v in chain.items())
        + f"; dW2 recomputed against saved {rec:.2e}")
    assert rec <= TOL["e4m3"]


# (200, 384, 272): with 128-element FP8 stages, T=200 ragged with an even
# number of stages (the weight gradients), H=384 a whole but odd number and
# Fs=272 a ragged odd one (each starting with the zero stage). (200, 2304,
# 144): dW1 has 9 tile columns, more than its two stages, so most of the
# workgroups own no stage of db1's column sum
@pytest.mark.parametrize("T,H,Fs", [(300, 528, 272), (64, 256, 512), (37, 48, 32), (513, 1040, 400),
                                    (200, 384, 272), (200, 2304, 144)])
def test_fp8_block_small_and_ragged(tp, T, H, Fs):
    _fp8_block(tp, T, H, Fs, seed=900 + T)


def test_fp8_block_accumulate_and_more_tiles_than_cus(tp):
    """accumulate = 1 into prior fp32 gradients, at a size whose GEMMs have
    more than 256 tiles (ragged in every dimension)."""
    _fp8_block(tp, 4200, 4208, 4112, seed=917, prior=True)



@pytest.mark.parametrize("T,H,Fs", [(32, 1 << 21, 16), (16, 16, 1 << 21)])
def test_fp8_block_widest_rows(tp, T, H, Fs):
    """The widest hidden size and ffn shard the calls accept (2^21): K loops
    of 16384 FP8 stages, operand rows of 2 MiB, 2^21-row weight gradients
    and their token-contiguous forms."""
    _fp8_block(tp, T, H, Fs, seed=960 + T)

# The gated block in E4M3: (300, 528, 272) ragged in T and Fs; (64, 256, 512)
# whole tiles; (37, 48, 32) smaller than one tile; (200, 384, 272) the ragged
# odd stage counts of the GELU cases; (513, 1040, 400) a 3 x 4 pair-tile fc1.
@pytest.mark.parametrize("T,H,Fs", [(300, 528, 272), (64, 256, 512), (37, 48, 32),
                                    (200, 384, 272), (513, 1040, 400)])
def test_fp8_gated_block_small_and_ragged(tp, T, H, Fs):
    _fp8_block(tp, T, H, Fs, seed=930 + T, act="swiglu")


def test_fp8_gated_block_accumulate_and_more_tiles_than_cus(tp):
    """The gated block, accumulate = 1, GEMMs of more than 256 tiles (fc1:
    17 x 17 pair tiles; the weight gradients' last round partial)."""
    _fp8_block(tp, 4200, 4208, 2128, seed=947, prior=True, act="swiglu")


def test_fp8_zero_tokens_still_step_the_histories(tp):
    """T = 0: no products, but each call enters an amax of 0 into its
    history (one entry per call), reports 1 / the factor it was given and
    sets the next factor as the oracle's delayed update does; wgrad without
    accumulation writes zeros."""
    H, Fs = 48, 32
    desc = tp.make_desc(0, H, Fs, act="gelu", dtype="e4m3", has_bias=True)
    one = lambda: torch.ones(1, dtype=torch.float32, device="cuda")
    W1 = torch.zeros((Fs, H), dtype=torch.uint8, device="cuda")
    W2 = torch.zeros((H, Fs), dtype=torch.uint8, device="cuda")
    b1 = torch.zeros((Fs,), dtype=torch.bfloat16, device="cuda")
    anyp = W1  # zero-sized tensors may have no storage: a valid aligned pointer instead
    ws = {c: torch.empty(max(tp.workspace_size(desc, c), 1), dtype=torch.uint8, device="cuda")
          for c in (tp.CALL_FWD, tp.CALL_DGRAD, tp.CALL_WGRAD)}
    for prior in (np.array([3.0, 0.0, 5.0], np.float32), np.zeros(3, np.float32)):
        ah = tp.DelayedScaling(3, scale=2.0)
        dh = tp.DelayedScaling(3, scale=4.0)
        ah.amax_history.copy_(torch.from_numpy(prior))
        dh.amax_history.copy_(torch.from_numpy(prior))
        say(f"  zero tokens, prior history {prior.tolist()}")
        tp.tpmlp_fwd(desc, anyp, W1, b1, W2, anyp, anyp, anyp,
                     fp8=tp.fp8_scales(one(), one(), one(), a_history=ah), workspace=ws[tp.CALL_FWD])
        tp.tpmlp_bwd_dgrad(desc, anyp, W1, W2, anyp, anyp, anyp,
                           fp8=tp.fp8_scales(w1_scale_inv=one(), w2_scale_inv=one(),
                                             dy_scale_inv=one(), dH_history=dh),
                           workspace=ws[tp.CALL_DGRAD])
        dW1 = torch.full((Fs, H), 7.0, device="cuda")
        db1 = torch.full((Fs,), 7.0, device="cuda")
        dW2 = torch.full((H, Fs), 7.0, device="cuda")
        tp.tpmlp_bwd_wgrad(desc, anyp, anyp, anyp, anyp, dW1, db1, dW2, accumulate=False,
                           fp8=tp.fp8_scales(x_scale_inv=one(), a_scale_inv=one(),
                                             dy_scale_inv=one(), dH_scale_inv=one()),
                           workspace=ws[tp.CALL_WGRAD])
        torch.cuda.synchronize()
        for hist, s_in, fmt in ((ah, 2.0, "e4m3"), (dh, 4.0, "e5m2")):
            want_h, want_s, want_si = oracle.delayed_update(prior, np.float32(0.0), np.float32(s_in), fmt)
            assert np.array_equal(hist.amax_history.cpu().numpy(), want_h), fmt
            assert float(hist.scale.cpu()[0]) == float(want_s), fmt
            assert float(hist.scale_inv.cpu()[0]) == float(want_si), fmt
        assert torch.all(dW1 == 0) and torch.all(db1 == 0) and torch.all(dW2 == 0)
        # the token-contiguous entry: the same zeros, and accumulating adds nothing
        for t in (dW1, db1, dW2):
            t.fill_(7.0)
        sc_w = tp.fp8_scales(x_scale_inv=one(), a_scale_inv=one(), dy_scale_inv=one(),
                             dH_scale_inv=one())
        tp.tpmlp_bwd_wgrad_t(desc, anyp, anyp, anyp, anyp, dW1, db1, dW2, accumulate=True,
                             fp8=sc_w)
        torch.cuda.synchronize()
        assert torch.all(dW1 == 7) and torch.all(db1 == 7) and torch.all(dW2 == 7)
        tp.tpmlp_bwd_wgrad_t(desc, anyp, anyp, anyp, anyp, dW1, db1, dW2, accumulate=False,
                             fp8=sc_w)
        torch.cuda.synchronize()
        assert torch.all(dW1 == 0) and torch.all(db1 == 0) and torch.all(dW2 == 0)


@pytest.mark.parametrize("rows,cols", [(1, 16), (37, 48), (64, 64), (300, 528), (513, 1040),
                                       (4200, 4208)])
def test_transpose_u8_exact(tp, rows, cols):
    """The token-contiguous copy: every byte transposed, the padding columns
    [rows, round_up(rows, 16)) zero (including bytes that are NaN codes)."""
    rng = np.random.default_rng(rows * 7 + cols)
    src = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
    say(f"  transpose {rows} x {cols}")
    got = tp.transpose_u8(torch.from_numpy(src).cuda())
    torch.cuda.synchronize()
    ld = (rows + 15) // 16 * 16
    want = np.zeros((cols, ld), np.uint8)
    want[:, :rows] = src.T
    assert got.shape == (cols, ld)
    assert np.array_equal(got.cpu().numpy(), want)


def test_fp8_block_full_size_sampled(tp):
    """The 12288-hidden TP=8 FP8 shard, forward + backward as the benchmark
    runs it (delayed scaling for a and dH): sampled token rows (y, dx, and
    the codes of a and dH) and sampled features (dW1 rows, db1 entries, dW2
    columns), each computed by the oracle from the full inputs."""
    from oracle import block as ob
    w = synth.WORKLOADS[5]
    say("config 5 forward + backward: generating and quantising inputs")
    inp = synth.make_rank_inputs(w)
    dev, deq = _quantized_inputs(tp, inp)
    b1 = oracle.to_f64(inp["b1"])
    rows = np.array([0, 1, 255, 4097, 8191])
    feats = np.array([0, 1, 255, 256, 6143])
    # scales for a and dH from the sampled rows' values, with headroom (both
    # sides quantise at these same factors)
    f0 = oracle.rank_forward(deq["x"][rows], deq["W1"], b1, deq["W2"], "gelu")
    g0 = oracle.rank_dgrad(deq["dy"][rows], deq["W1"], deq["W2"], f0["h"], "gelu")
    a_scale = _scale_for(4 * np.max(np.abs(f0["a"])), "e4m3")
    dH_scale = _scale_for(4 * np.max(np.abs(g0["dH"])), "e5m2")
    T, H, Fs = w.tokens, w.hidden, w.ffn_shard
    desc = tp.make_desc(T, H, Fs, act="gelu", dtype="e4m3", has_bias=True)
    ah = tp.DelayedScaling(16, scale=float(a_scale))
    dh = tp.DelayedScaling(16, scale=float(dH_scale))
    say(f"  e4m3 block T={T} H={H} Fs={Fs}")
    f = tp.fwd(desc, dev["x"][0], dev["W1"][0], inp["b1"].cuda(), dev["W2"][0],
               fp8_in_scales=(dev["x"][1], dev["W1"][1], dev["W2"][1]), a_history=ah)
    g = tp.bwd_dgrad(desc, dev["dy"][0], dev["W1"][0], dev["W2"][0], f["h"],
                     fp8=dict(dy_scale_inv=dev["dy"][1], w1_scale_inv=dev["W1"][1],
                              w2_scale_inv=dev["W2"][1], dH_history=dh))
    wg = tp.bwd_wgrad(desc, dev["dy"][0], dev["x"][0], f["a"], g["dH"],
                      fp8=dict(dy_scale_inv=dev["dy"][1], x_scale_inv=dev["x"][1],
                               a_scale_inv=ah.scale_inv, dH_scale_inv=dh.scale_inv))
    torch.cuda.synchronize()
    # sampled rows
    rf = oracle.rank_forward_fp8(deq["x"][rows], deq["W1"], b1, deq["W2"], a_scale)
    rg = oracle.rank_dgrad_fp8(deq["dy"][rows], deq["W1"], deq["W2"], rf["h"], dH_scale)
    lo, hi = _check_h(f["h"][rows], rf["h_exact"])
    _check_codes("a rows", f["a"][rows], rf["a"] * float(a_scale),
                 _a_delta(rf, lo, hi) * float(a_scale), "e4m3", rf["a_codes"])
    _check_codes("dH rows", g["dH"][rows], rg["dH"] * float(dH_scale),
                 _dH_delta(rg, rf["h"], lo, hi) * float(dH_scale), "e5m2", rg["dH_codes"])
    errs = {"y": rel_err(f["y"][rows].cpu(), rf["y"]), "dx": rel_err(g["dx"][rows].cpu(), rg["dx"])}
    # sampled features over all tokens
    W1s, b1s, W2s = ob.select_features(deq["W1"], b1, deq["W2"], feats, "gelu")
    cf = oracle.rank_forward_fp8(deq["x"], W1s, b1s, W2s, a_scale)
    cg = oracle.rank_dgrad_fp8(deq["dy"], W1s, W2s, cf["h"], dH_scale)
    cw = oracle.rank_wgrad_fp8(deq["dy"], deq["x"], cf["a_q"], cg["dH_q"])
    errs["dW1"] = rel_err(wg["dW1"][feats].cpu(), cw["dW1"])
    errs["db1"] = rel_err(wg["db1"][feats].cpu(), cw["db1"])
    errs["dW2"] = rel_err(wg["dW2"][:, feats].cpu(), cw["dW2"])
    say("    rel errors " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL["e4m3"], (k, v)


def test_fp8_forward_full_size_every_element(tp):
    """The 12288-hidden TP=8 FP8 shard's forward as the benchmark runs it
    (a quantised in fc1's epilogue under delayed scaling): every element of h
    within its bf16 window, every code of a a valid rounding of the oracle's
    exact a (and all but a few equal to the oracle's own codes), y within the
    e4m3 tolerance, and the amax entered into the history."""
    w = synth.WORKLOADS[5]
    say("config 5 forward: generating and quantising inputs")
    inp = synth.make_rank_inputs(w, with_dy=False)
    dev, deq = _quantized_inputs(tp, inp, with_dy=False)
    b1 = oracle.to_f64(inp["b1"])
    T, H, Fs = w.tokens, w.hidden, w.ffn_shard
    say("  oracle forward (plain block for the scale, then the FP8 block)")
    f0 = oracle.rank_forward(deq["x"], deq["W1"], b1, deq["W2"], "gelu")
    a_scale = _scale_for(np.max(np.abs(f0["a"])), "e4m3")
    del f0
    rf = oracle.rank_forward_fp8(deq["x"], deq["W1"], b1, deq["W2"], a_scale)
    desc = tp.make_desc(T, H, Fs, act="gelu", dtype="e4m3", has_bias=True)
    ah = tp.DelayedScaling(16, scale=float(a_scale))
    say(f"  e4m3 forward T={T} H={H} Fs={Fs}")
    f = tp.fwd(desc, dev["x"][0], dev["W1"][0], inp["b1"].cuda(), dev["W2"][0],
               fp8_in_scales=(dev["x"][1], dev["W1"][1], dev["W2"][1]), a_history=ah)
    torch.cuda.synchronize()
    lo, hi = _check_h(f["h"], rf["h"])
    da = _a_delta(rf, lo, hi)
    _check_codes("a", f["a"], rf["a"] * float(a_scale), da * float(a_scale), "e4m3",
                 rf["a_codes"])
    assert abs(float(ah.amax_history.cpu()[0]) - rf["amax"]) <= float(np.max(da))
    e_y = rel_err(f["y"].cpu(), rf["y"])
    say(f"    rel error y={e_y:.2e}")
    assert e_y <= TOL["e4m3"]
