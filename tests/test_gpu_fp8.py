"""GPU parity of the FP8 (OCP E4M3, per-tensor current scaling) path.

* The quantiser is bit-exact against the oracle's encoder: both take the
  decision (the integer code) from the same float32 product v * scale.
* The e4m3 forward is checked against the oracle run on the dequantised
  inputs (the codes the GPU quantiser produced are first checked equal to the
  oracle's own), within 6e-2 of max|oracle|."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu_helpers import TOL, rel_err, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tp():
    require_gpu()
    import tensor_transformer_mlp_rank_amd as m
    return m


def _special_values():
    grid = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    grid = np.unique(grid[np.isfinite(grid)])
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(np.inf)),
                           np.nextafter(mids, np.float32(-np.inf))])
    return np.concatenate([grid.astype(np.float32), mids, near])


@pytest.mark.parametrize("src", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 7, 1000, 65537, 3 * 1024 * 1024 + 5])
def test_quantizer_bit_exact(tp, src, n):
    rng = np.random.default_rng(n)
    v = (rng.standard_normal(n) * rng.choice([1e-3, 0.05, 3.0], size=n)).astype(np.float32)
    if n > 5000:
        sp = _special_values() / 448.0 * float(np.max(np.abs(v)))  # ties in the scaled domain
        v[: sp.size] = sp.astype(np.float32)
    t = torch.from_numpy(v)
    if src == "bf16":
        t = t.to(torch.bfloat16)
    say(f"quantize src={src} n={n}")
    codes, amax, sinv = tp.quantize_e4m3(t.cuda())
    torch.cuda.synchronize()
    vv = t.float().numpy()
    rc, ramax, rs, rsinv = oracle.quantize_e4m3(vv)
    assert float(amax.cpu()[0]) == float(ramax)
    assert float(sinv.cpu()[0]) == float(rsinv)
    got = codes.cpu().numpy()
    mism = np.nonzero(got != rc)[0]
    assert mism.size == 0, f"{mism.size} codes differ, first at {mism[:5]}: {got[mism[:5]]} vs {rc[mism[:5]]}"


def test_quantizer_all_zero_and_empty(tp):
    z = torch.zeros(1000, device="cuda")
    codes, amax, sinv = tp.quantize_e4m3(z)
    torch.cuda.synchronize()
    assert float(amax.cpu()[0]) == 0.0 and float(sinv.cpu()[0]) == 1.0
    assert torch.all(codes == 0)
    e = torch.zeros(0, device="cuda")
    codes, amax, sinv = tp.quantize_e4m3(e)
    torch.cuda.synchronize()
    assert float(amax.cpu()[0]) == 0.0 and float(sinv.cpu()[0]) == 1.0


def _fp8_case(tp, inp, act="gelu"):
    """Quantise x, W1, W2 on the GPU, check codes against the oracle, run the
    e4m3 forward; returns (gpu outputs, oracle dequantised inputs)."""
    q = {}
    deq = {}
    for k in ("x", "W1", "W2"):
        codes, amax, sinv = tp.quantize_e4m3(inp[k].cuda())
        rc, ramax, rs, rsinv = oracle.quantize_e4m3(inp[k].numpy())
        torch.cuda.synchronize()
        assert float(sinv.cpu()[0]) == float(rsinv), k
        assert np.array_equal(codes.cpu().numpy(), rc), k
        q[k] = (codes, sinv)
        deq[k] = oracle.dequantize_e4m3(rc, rsinv)
    T, H = inp["x"].shape
    Fs = inp["W2"].shape[1]
    desc = tp.make_desc(T, H, Fs, act=act, dtype="e4m3", has_bias=inp["b1"] is not None)
    b1 = None if inp["b1"] is None else inp["b1"].cuda()
    say(f"  e4m3 {act} fwd T={T} H={H} Fs={Fs}")
    out = tp.fwd(desc, q["x"][0], q["W1"][0], b1, q["W2"][0],
                 fp8_in_scales=(q["x"][1], q["W1"][1], q["W2"][1]))
    torch.cuda.synchronize()
    return {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in out.items()}, deq


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("T,H,Fs", [(300, 528, 272), (64, 256, 512), (1, 32, 16)])
def test_fp8_forward_small(tp, T, H, Fs, act):
    """Current scaling (a through bf16 and the quantiser); act "swiglu": the
    gated block, with the gated workload's value distributions."""
    w = synth.WORKLOADS[4 if act == "swiglu" else 5]
    inp = synth.make_rank_inputs(w, tokens=T, hidden=H, ffn_shard=Fs, dtype="e4m3",
                                 seed_base=500 + T)
    gpu, deq = _fp8_case(tp, inp, act)
    ref = oracle.rank_forward(deq["x"], deq["W1"], oracle.to_f64(inp["b1"]), deq["W2"], act)
    e_y = rel_err(gpu["y"], ref["y"])
    e_h = rel_err(gpu["h"], ref["h"])
    # the quantised activation, dequantised with the reported scale
    a_deq = oracle.dequantize_e4m3(gpu["a"].numpy(), float(gpu["a_scale_inv"][0]))
    e_a = rel_err(a_deq, ref["a"])
    amax_ref = float(np.max(np.abs(ref["a"])))
    e_amax = abs(float(gpu["a_amax"][0]) - amax_ref) / amax_ref
    say(f"  rel errors y={e_y:.2e} h={e_h:.2e} a={e_a:.2e} amax={e_amax:.2e}")
    assert e_y <= TOL["e4m3"] and e_a <= TOL["e4m3"]
    assert e_h <= TOL["bf16"] and e_amax <= TOL["bf16"]
    # the scale the GPU reports is the recipe's for its own amax
    s = np.float32(np.float32(448.0) / np.float32(gpu["a_amax"][0]))
    assert float(gpu["a_scale_inv"][0]) == float(np.float32(np.float32(1.0) / s))


def test_fp8_forward_full_size_sampled(tp):
    """The 12288-hidden TP=8 shard: sampled token rows of y and h."""
    w = synth.WORKLOADS[5]
    say("config 5: generating inputs")
    inp = synth.make_rank_inputs(w, with_dy=False)
    gpu, deq = _fp8_case(tp, inp)
    rows = np.array([0, 1, 255, 4096, 8191])
    ref = oracle.rank_forward(deq["x"][rows], deq["W1"], oracle.to_f64(inp["b1"]), deq["W2"],
                              "gelu")
    e_y = rel_err(gpu["y"][rows], ref["y"])
    e_h = rel_err(gpu["h"][rows], ref["h"])
    say(f"  rel errors y={e_y:.2e} h={e_h:.2e}")
    assert e_y <= TOL["e4m3"] and e_h <= TOL["bf16"]


def test_fp8_amax_leaves_out_padding_rows(tp):
    """T = 300 is not a multiple of the 256-row tile: the rows past T in the
    last tile hold h = b1, not activations. Here every real h is -3 (tiny
    |gelu|) while gelu(b1) = 29, so amax must stay near |gelu(-3)|."""
    T, H, Fs = 300, 32, 16
    x = torch.ones((T, H), dtype=torch.bfloat16)
    W1 = -torch.ones((Fs, H), dtype=torch.bfloat16)
    W2 = torch.ones((H, Fs), dtype=torch.bfloat16)
    b1 = torch.full((Fs,), 29.0, dtype=torch.bfloat16)
    q = {}
    for k, v in (("x", x), ("W1", W1), ("W2", W2)):
        codes, _, sinv = tp.quantize_e4m3(v.cuda())
        q[k] = (codes, sinv)
    desc = tp.make_desc(T, H, Fs, act="gelu", dtype="e4m3", has_bias=True)
    out = tp.fwd(desc, q["x"][0], q["W1"][0], b1.cuda(), q["W2"][0],
                 fp8_in_scales=(q["x"][1], q["W1"][1], q["W2"][1]))
    torch.cuda.synchronize()
    ref = oracle.rank_forward(oracle.to_f64(x), oracle.to_f64(W1), oracle.to_f64(b1),
                              oracle.to_f64(W2), "gelu")
    amax_ref = float(np.max(np.abs(ref["a"])))
    amax = float(out["a_amax"].cpu()[0])
    say(f"  amax gpu {amax:.6g} oracle {amax_ref:.6g}")
    assert abs(amax - amax_ref) <= TOL["bf16"] * amax_ref


def test_fp8_scales_struct_keeps_its_tensors_alive(tp):
    """A tpmlp_fp8_scales struct built from scale tensors that nothing else
    references: the struct keeps them alive, so new allocations made before
    the call cannot take their memory (regression: the benchmark's FP8 step
    once read a freed x_scale_inv slot holding another tensor's 1.0)."""
    T, H, Fs = 256, 512, 256
    w = synth.WORKLOADS[5]
    inp = synth.make_rank_inputs(w, tokens=T, hidden=H, ffn_shard=Fs, seed_base=77)
    desc = tp.make_desc(T, H, Fs, act="gelu", dtype="e4m3", has_bias=True)
    codes = {}

    def scales():
        sinv = {}
        for k in ("x", "W1", "W2"):
            codes[k], _, sinv[k] = tp.quantize_e4m3(inp[k].cuda())
        return tp.fp8_scales(sinv["x"], sinv["W1"], sinv["W2"], a_history=tp.DelayedScaling(2))

    sc = scales()
    torch.cuda.synchronize()
    import gc
    gc.collect()
    junk = [torch.full((1,), 1.0, device="cuda") for _ in range(64)]   # reuse freed slots
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    h = torch.empty((T, Fs), dtype=torch.bfloat16, device="cuda")
    a = torch.empty((T, Fs), dtype=torch.uint8, device="cuda")
    ws = torch.empty(tp.workspace_size(desc, tp.CALL_FWD), dtype=torch.uint8, device="cuda")
    tp.tpmlp_fwd(desc, codes["x"], codes["W1"], inp["b1"].cuda(), codes["W2"], y, h, a, fp8=sc,
                 workspace=ws)
    torch.cuda.synchronize()
    deq = {}
    for k in ("x", "W1", "W2"):
        rc, _, _, rsinv = oracle.quantize_e4m3(inp[k].numpy())
        deq[k] = oracle.dequantize_e4m3(rc, rsinv)
    ref = oracle.rank_forward(deq["x"], deq["W1"], oracle.to_f64(inp["b1"]), deq["W2"], "gelu")
    e_h = rel_err(h.cpu(), ref["h"])
    say(f"  rel error h={e_h:.2e}")
    assert e_h <= TOL["bf16"]
    del junk
