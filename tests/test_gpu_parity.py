"""GPU parity: the HIP path through the C ABI against the CPU oracle, on the
same seeded inputs, element by element (small and ragged shapes spanning
several tiles) or on sampled outputs (full per-rank shapes).

Tolerance per output tensor, max|gpu - oracle| / max|oracle|:
fp32 1e-5, bf16 inputs with fp32 accumulation 2e-2, e4m3 with per-tensor
scales 6e-2."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu_helpers import (TOL, check, gpu_block, oracle_block, rel_err, require_gpu,
                          sample_gpu, sampled_reference, say, to_dev)

pytestmark = pytest.mark.gpu

ALL = ("y", "h", "a", "dH", "dx", "dW1", "db1", "dW2")


@pytest.fixture(scope="module")
def tp():
    require_gpu()
    import tensor_transformer_mlp_rank_amd as m
    return m


# ------------------------------------------------------------------ tiny fp32, simulated TP=2
@pytest.mark.parametrize("bias_std", [0.0, 0.3])
def test_tiny_fp32_two_simulated_shards(tp, bias_std):
    """Tiny fp32 GELU block (T=128, H=256, F=1024) split into two shards:
    each rank runs on the GPU; the sum of the partial outputs must match the
    unsharded oracle block, and every per-rank tensor its oracle shard."""
    w = synth.WORKLOADS[1]
    full = synth.make_unsharded_inputs(w, b1_std=bias_std)
    ref_full = oracle.unsharded_backward(full["x"], full["W1"], full["b1"], full["W2"], full["dy"],
                                         "gelu")
    ys, dxs = [], []
    for r in range(w.tp):
        W1r, b1r, W2r = oracle.shard_rank(oracle.to_f64(full["W1"]), oracle.to_f64(full["b1"]),
                                          oracle.to_f64(full["W2"]), w.tp, r, "gelu")
        inp = {"x": full["x"], "dy": full["dy"],
               "W1": torch.from_numpy(W1r).float(), "b1": torch.from_numpy(b1r).float(),
               "W2": torch.from_numpy(W2r).float()}
        say(f"rank {r} of {w.tp}")
        gpu = gpu_block(tp, inp, "gelu", "f32", True)
        ref = oracle_block(inp, "gelu", True)
        check(gpu, ref, "f32", ALL)
        ys.append(oracle.to_f64(gpu["y"]))
        dxs.append(oracle.to_f64(gpu["dx"]))
    assert rel_err(sum(ys), ref_full["y"]) <= TOL["f32"]
    assert rel_err(sum(dxs), ref_full["dx"]) <= TOL["f32"]


# ------------------------------------------------------------------ small and ragged shapes
SHAPES = [
    # (T, H, Fs): several tiles of every GEMM and ragged tails in T, H and Fs
    (300, 528, 272),
    (513, 256, 256),
    (64, 1040, 400),
    (1, 16, 16),
    (37, 48, 32),
    # the main loop's forms (64-element stages, run two per iteration; an odd
    # count starts with a zero stage): H=192 and H=320 a whole but odd number
    # of stages (folded K-major loads after the zero stage), Fs=80 and Fs=208
    # ragged with an even number, T=100 ragged and even for the weight
    # gradients, T=192 whole and odd (their zero stage); (300, 528, 272)
    # above has ragged odd counts in every product
    (100, 192, 80),
    (192, 320, 208),
    # one tile, Fs of 17 stages: fc2's forward and fc1's data gradient split K
    # in two, 10 stages and 7 (with the zero stage, 8)
    (256, 256, 1088),
]


@pytest.mark.parametrize("T,H,Fs", SHAPES)
@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_block_small_and_ragged(tp, T, H, Fs, act, dtype):
    w = synth.WORKLOADS[4 if act == "swiglu" else 2]
    inp = synth.make_rank_inputs(w, tokens=T, hidden=H, ffn_shard=Fs, dtype=dtype,
                                 seed_base=100 + T % 97)
    has_bias = act == "gelu"
    gpu = gpu_block(tp, inp, act, dtype, has_bias)
    ref = oracle_block(inp, act, has_bias)
    check(gpu, ref, dtype, ALL)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_block_more_tiles_than_workgroups(tp, act):
    """bf16 block whose GEMMs have 289 (SwiGLU fc1: 561) 256-wide tiles, more
    than the 256 compute units: a CU runs several workgroups in turn, and
    every GEMM has ragged edges in M, N and K. Compared element by element,
    with accumulation into prior gradients."""
    T, H, Fs = 4200, 4208, 4112
    w = synth.WORKLOADS[4 if act == "swiglu" else 2]
    say(f"  T={T} H={H} Fs={Fs} {act}: generating inputs")
    inp = synth.make_rank_inputs(w, tokens=T, hidden=H, ffn_shard=Fs, seed_base=313)
    has_bias = act == "gelu"
    G = 2 if act == "swiglu" else 1
    prior = {"dW1": synth.grad_init(313, (G * Fs, H), 1),
             "db1": synth.grad_init(313, (G * Fs,), 2) if has_bias else None,
             "dW2": synth.grad_init(313, (H, Fs), 3)}
    gpu = gpu_block(tp, inp, act, "bf16", has_bias, accumulate_into=prior)
    say("  oracle")
    ref = oracle_block(inp, act, has_bias, prior=prior)
    check(gpu, ref, "bf16", ALL)


@pytest.mark.parametrize("T,H,Fs", [(192, 2048, 256), (200, 2160, 272), (136, 16400, 64)])
def test_db1_wide_dW1(tp, T, H, Fs):
    """db1 fused into the dW1 product where dW1 has 8 or more tile columns
    (the tile columns share out the k-stages, column bn taking stages bn,
    bn + tiles_n, ...): 8 and 9 columns, and 65, more than the product's
    stages, so that most workgroups own none; an odd whole number of stages
    (T=192, the zero stage), a ragged one (T=200, T=136), and split-K where
    the grid is small. Accumulates into prior gradients; every output
    compared element by element."""
    w = synth.WORKLOADS[2]
    inp = synth.make_rank_inputs(w, tokens=T, hidden=H, ffn_shard=Fs, seed_base=640 + T)
    prior = {"dW1": synth.grad_init(640, (Fs, H), 1),
             "db1": synth.grad_init(640, (Fs,), 2),
             "dW2": synth.grad_init(640, (H, Fs), 3)}
    gpu = gpu_block(tp, inp, "gelu", "bf16", True, accumulate_into=prior)
    ref = oracle_block(inp, "gelu", True, prior=prior)
    check(gpu, ref, "bf16", ALL)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_wgrad_accumulate(tp, dtype, act):
    """accumulate=1 adds into seeded nonzero fp32 buffers."""
    T, H, Fs = 200, 272, 144
    w = synth.WORKLOADS[4 if act == "swiglu" else 2]
    inp = synth.make_rank_inputs(w, tokens=T, hidden=H, ffn_shard=Fs, dtype=dtype, seed_base=77)
    has_bias = act == "gelu"
    G = 2 if act == "swiglu" else 1
    prior = {"dW1": synth.grad_init(77, (G * Fs, H), 1) * 100,
             "db1": synth.grad_init(77, (G * Fs,), 2) * 100 if has_bias else None,
             "dW2": synth.grad_init(77, (H, Fs), 3) * 100}
    gpu = gpu_block(tp, inp, act, dtype, has_bias, accumulate_into=prior)
    ref = oracle_block(inp, act, has_bias, prior=prior)
    check(gpu, ref, dtype, ("dW1", "db1", "dW2"))


@pytest.mark.parametrize("T,H,Fs,act", [
    (1024, 272, 144, "gelu"),     # 16 stages
    (960, 528, 400, "swiglu"),    # 15 stages after the zero stage
    (1088, 256, 256, "gelu"),     # 17 stages after the zero stage
    (1500, 1040, 528, "gelu"),    # several tiles, ragged in every dimension
])
def test_wgrad_accumulate_long_k(tp, T, H, Fs, act):
    """Weight gradients over 15 to 24 stages of tokens accumulating into
    prior gradients of both signs and of a magnitude well above the
    products, compared element by element, with rows and columns past the
    ends of dW1 and dW2."""
    w = synth.WORKLOADS[4 if act == "swiglu" else 2]
    inp = synth.make_rank_inputs(w, tokens=T, hidden=H, ffn_shard=Fs, seed_base=71 + T % 13)
    has_bias = act == "gelu"
    G = 2 if act == "swiglu" else 1
    prior = {"dW1": synth.grad_init(71, (G * Fs, H), 1) * 50,
             "db1": synth.grad_init(71, (G * Fs,), 2) * 50 if has_bias else None,
             "dW2": synth.grad_init(71, (H, Fs), 3) * 50}
    gpu = gpu_block(tp, inp, act, "bf16", has_bias, accumulate_into=prior)
    ref = oracle_block(inp, act, has_bias, prior=prior)
    check(gpu, ref, "bf16", ("dW1", "db1", "dW2"))
    # the sums without the prior, to the same bar: the products are not lost
    # in the prior's magnitude
    for k in ("dW1", "dW2"):
        got = oracle.to_f64(gpu[k]) - oracle.to_f64(prior[k])
        want = ref[k] - oracle.to_f64(prior[k])
        assert rel_err(got, want) <= TOL["bf16"], k


@pytest.mark.parametrize("act,dtype", [("gelu", "bf16"), ("swiglu", "bf16"), ("gelu", "f32"),
                                       ("swiglu", "f32")])
def test_wgrad_recompute(tp, act, dtype):
    """Selective recomputation: tpmlp_bwd_wgrad_recompute forms a from the
    saved h and gives tpmlp_bwd_wgrad's results from the saved a bit for bit
    (the recomputed activation is the forward's), and so the oracle's to the
    tolerance; ragged in every dimension, accumulating into prior
    gradients."""
    T, H, Fs = 1500, 1040, 528
    w = synth.WORKLOADS[4 if act == "swiglu" else 2]
    inp = synth.make_rank_inputs(w, tokens=T, hidden=H, ffn_shard=Fs, dtype=dtype, seed_base=87)
    has_bias = act == "gelu"
    G = 2 if act == "swiglu" else 1
    prior = {"dW1": synth.grad_init(87, (G * Fs, H), 1),
             "db1": synth.grad_init(87, (G * Fs,), 2) if has_bias else None,
             "dW2": synth.grad_init(87, (H, Fs), 3)}
    names = ("dW1", "db1", "dW2") if has_bias else ("dW1", "dW2")
    saved = gpu_block(tp, inp, act, dtype, has_bias, accumulate_into=prior)
    rec = gpu_block(tp, inp, act, dtype, has_bias, accumulate_into=prior, recompute=True)
    for k in names:
        assert torch.equal(saved[k], rec[k]), k
    ref = oracle_block(inp, act, has_bias, prior=prior)
    check(rec, ref, dtype, names)


@pytest.mark.parametrize("act,dtype", [("swiglu", "bf16"), ("gelu", "e4m3")])
def test_wgrad_partial_last_round(tp, act, dtype):
    """Weight gradients whose tile grid leaves a partial last round run its
    tiles as two half-K workgroups that meet in the workspace: dW2 of
    17 x 17 = 289 tiles (32 split), SwiGLU dW1 of 34 x 17 = 578 (64 split).
    Compared with the unsplit product (the minimal workspace) to fp32
    rounding, bit for bit between two runs, and accumulating into priors."""
    T, H, Fs = 2048, 4352, 4352 - 16
    G = 2 if act == "swiglu" else 1
    has_bias = act == "gelu"
    desc = tp.make_desc(T, H, Fs, act=act, dtype=dtype, has_bias=has_bias)
    assert tp.workspace_size(desc, tp.CALL_WGRAD) > 0
    gen = torch.Generator().manual_seed(5)
    if dtype == "e4m3":
        codes = lambda *sh: torch.randint(0, 120, sh, generator=gen, dtype=torch.uint8).cuda()
        dy, x, a, dH = codes(T, H), codes(T, H), codes(T, Fs), codes(T, G * Fs)
        one = torch.ones(1, dtype=torch.float32, device="cuda")
        fp8 = tp.fp8_scales(x_scale_inv=one, a_scale_inv=one, dy_scale_inv=one, dH_scale_inv=one)
    else:
        bf = lambda *sh: torch.randn(*sh, generator=gen).to(torch.bfloat16).cuda()
        dy, x, a, dH = bf(T, H), bf(T, H), bf(T, Fs), bf(T, G * Fs)
        fp8 = None
    prior = {"dW1": torch.randn(G * Fs, H, generator=gen), "dW2": torch.randn(H, Fs, generator=gen),
             "db1": torch.randn(G * Fs, generator=gen) if has_bias else None}

    def run(ws_bytes):
        out = {k: (None if v is None else v.clone().cuda()) for k, v in prior.items()}
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
        tp.tpmlp_bwd_wgrad(desc, dy, x, a, dH, out["dW1"], out["db1"], out["dW2"], accumulate=True,
                           fp8=fp8, workspace=ws if ws_bytes else None)
        torch.cuda.synchronize()
        return {k: v for k, v in out.items() if v is not None}

    full = tp.workspace_size(desc, tp.CALL_WGRAD)
    split1, split2 = run(full), run(full)
    # the minimal workspace: the db1 partial rows only (bias), or none
    plain = run((((H + 255) // 256) * G * Fs * 4 + 255) // 256 * 256 if has_bias else 0)
    for k in split1:
        assert torch.equal(split1[k], split2[k]), k
        assert rel_err(split1[k].cpu(), plain[k].cpu()) <= 1e-5, k
    assert not torch.equal(split1["dW2"], plain["dW2"])  # the split ran (a different sum order)


def test_zero_tokens(tp):
    """T = 0: forward and dgrad enqueue nothing; wgrad overwrites with zeros
    (accumulate = 0) or leaves the buffers alone (accumulate = 1)."""
    H, Fs = 64, 32
    desc = tp.make_desc(0, H, Fs, act="gelu", dtype="bf16", has_bias=True)
    e = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    W1 = torch.zeros((Fs, H), dtype=torch.bfloat16, device="cuda")
    b1 = torch.zeros((Fs,), dtype=torch.bfloat16, device="cuda")
    W2 = torch.zeros((H, Fs), dtype=torch.bfloat16, device="cuda")
    # zero-sized tensors may have no storage: pass a valid aligned pointer instead
    anyp = W1
    tp.tpmlp_fwd(desc, anyp, W1, b1, W2, anyp, anyp, anyp)
    tp.tpmlp_bwd_dgrad(desc, anyp, W1, W2, anyp, anyp, anyp)
    dW1 = torch.full((Fs, H), 7.0, device="cuda")
    db1 = torch.full((Fs,), 7.0, device="cuda")
    dW2 = torch.full((H, Fs), 7.0, device="cuda")
    ws = torch.empty(tp.workspace_size(desc, tp.CALL_WGRAD), dtype=torch.uint8, device="cuda")
    tp.tpmlp_bwd_wgrad(desc, anyp, anyp, anyp, anyp, dW1, db1, dW2, accumulate=True,
                       workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(dW1 == 7) and torch.all(db1 == 7) and torch.all(dW2 == 7)
    tp.tpmlp_bwd_wgrad(desc, anyp, anyp, anyp, anyp, dW1, db1, dW2, accumulate=False,
                       workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(dW1 == 0) and torch.all(db1 == 0) and torch.all(dW2 == 0)
    del e


def test_deterministic(tp):
    """Two runs on the same inputs are bitwise identical (no atomics)."""
    inp = synth.make_rank_inputs(synth.WORKLOADS[2], tokens=520, hidden=512, ffn_shard=384,
                                 seed_base=5)
    a = gpu_block(tp, inp, "gelu", "bf16", True)
    b = gpu_block(tp, inp, "gelu", "bf16", True)
    for k in ALL:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("act,bias", [("gelu", True), ("swiglu", False)])
def test_wgrad_split_k(tp, act, bias):
    """Weight gradients whose tile grid leaves most CUs idle (a few 256 x 256
    tiles, many tokens) are split along K when the workspace has room for the
    partial sums: the result matches the oracle like the unsplit product (a
    workspace with only the db1 partials), and two split runs are bitwise
    identical (the partials are added in a fixed order)."""
    T, H, Fs = 4104, 512, 496
    w = synth.WORKLOADS[2 if act == "gelu" else 4]
    inp = synth.make_rank_inputs(w, tokens=T, hidden=H, ffn_shard=Fs, seed_base=77)
    G = 2 if act == "swiglu" else 1
    desc = tp.make_desc(T, H, Fs, act=act, dtype="bf16", has_bias=bias)
    dv = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    f = tp.fwd(desc, dv["x"], dv["W1"], dv["b1"] if bias else None, dv["W2"])
    g = tp.bwd_dgrad(desc, dv["dy"], dv["W1"], dv["W2"], f["h"])
    full = tp.workspace_size(desc, tp.CALL_WGRAD)
    tiles_n = (H + 255) // 256
    minimum = ((tiles_n * G * Fs * 4 + 255) // 256) * 256 if bias else 0
    assert full > minimum  # this shape is split
    say(f"  wgrad split-K act={act} bias={bias}: workspace {full} bytes, {minimum} unsplit")

    def run(nbytes):
        out = {"dW1": torch.empty((G * Fs, H), device="cuda"),
               "db1": torch.empty((G * Fs,), device="cuda") if bias else None,
               "dW2": torch.empty((H, Fs), device="cuda")}
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        tp.tpmlp_bwd_wgrad(desc, dv["dy"], dv["x"], f["a"], g["dH"], out["dW1"], out["db1"],
                           out["dW2"], accumulate=False, workspace=ws[:nbytes] if nbytes else None)
        torch.cuda.synchronize()
        return {k: (None if v is None else v.cpu()) for k, v in out.items()}

    split1, split2, plain = run(full), run(full), run(minimum)
    ref = oracle_block(inp, act, bias)
    names = ("dW1", "db1", "dW2") if bias else ("dW1", "dW2")
    check(split1, ref, "bf16", names)
    check(plain, ref, "bf16", names)
    for k in names:
        assert torch.equal(split1[k], split2[k]), k
    # the two orders of summation differ only by fp32 rounding
    for k in names:
        assert rel_err(split1[k], plain[k]) <= 1e-5, k


@pytest.mark.parametrize("T,H,Fs,dtype", [
    (1 << 20, 64, 64, "bf16"),       # a million tokens: 4096 M-tiles, weight gradients over K = 2^20
    (256, 1 << 16, 256, "bf16"),     # a 65536-wide hidden dimension: K = 2^16 for fc1 and dgrad
    (1 << 18, 64, 48, "f32"),        # the fp32 kernel over many tokens
    (32, 1 << 21, 16, "bf16"),       # the widest hidden size the calls accept (K = 2^21 for fc1)
    (48, 16, 1 << 21, "bf16"),       # the widest ffn shard they accept (K = 2^21 for fc2)
])
def test_extreme_shapes(tp, T, H, Fs, dtype):
    """Very long token counts and very wide rows (64-bit offsets, large tile
    grids, long K loops, split-K over a million tokens), every output
    compared with the oracle in full."""
    w = synth.WORKLOADS[1 if dtype == "f32" else 2]
    inp = synth.make_rank_inputs(w, tokens=T, hidden=H, ffn_shard=Fs, seed_base=123)
    say(f"  extreme shape T={T} H={H} Fs={Fs} {dtype}")
    gpu = gpu_block(tp, inp, "gelu", dtype, True)
    ref = oracle_block(inp, "gelu", True)
    check(gpu, ref, dtype, ALL)


def test_swiglu_h_layout(tp):
    """The saved pre-activation of the gated block is [gate | up]: the gate
    half is x . W1[:Fs]^T and the up half x . W1[Fs:]^T (checked separately so a
    swapped half cannot pass through a symmetric check)."""
    T, H, Fs = 96, 160, 80
    inp = synth.make_rank_inputs(synth.WORKLOADS[4], tokens=T, hidden=H, ffn_shard=Fs,
                                 seed_base=9)
    gpu = gpu_block(tp, inp, "swiglu", "bf16", False, calls=("fwd",))
    x = oracle.to_f64(inp["x"])
    W1 = oracle.to_f64(inp["W1"])
    assert rel_err(gpu["h"][:, :Fs], x @ W1[:Fs].T) <= TOL["bf16"]
    assert rel_err(gpu["h"][:, Fs:], x @ W1[Fs:].T) <= TOL["bf16"]


# ------------------------------------------------------------------ full per-rank shapes
ROWS = np.array([0, 1, 255, 256, 4097, 8191])
COLS = np.array([0, 1, 127, 128, 1000, 2047])


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_full_size_sampled(tp, cfg):
    """Full per-rank workload in the configuration the benchmark times; the
    oracle checks sampled token rows (y, h, a, dH, dx) and sampled features
    (dW2 columns, dW1 rows, db1 entries)."""
    w = synth.WORKLOADS[cfg]
    say(f"config {cfg} {w.name}: generating inputs")
    inp = synth.make_rank_inputs(w)
    has_bias = w.has_bias
    gpu = gpu_block(tp, inp, w.act, w.dtype, has_bias)
    cols = COLS[COLS < w.ffn_shard]
    ref = sampled_reference(inp, w.act, has_bias, ROWS, cols)
    got = sample_gpu(gpu, w.act, w.ffn_shard, ROWS, cols)
    check(got, ref, w.dtype, ALL)


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_full_size_every_element(tp, cfg):
    """Full per-rank workload in the launch configuration the benchmark times
    (the whole workspace, so split-K where planned; wgrad accumulating into
    prior fp32 gradients): every element of y, h, a, dH, dx, dW1, db1 and dW2
    against one oracle evaluation of the whole shard."""
    w = synth.WORKLOADS[cfg]
    say(f"config {cfg} {w.name}: generating inputs")
    inp = synth.make_rank_inputs(w)
    G, Fs, H = w.gate_mult, w.ffn_shard, w.hidden
    prior = {"dW1": synth.grad_init(cfg, (G * Fs, H), 1),
             "db1": synth.grad_init(cfg, (G * Fs,), 2) if w.has_bias else None,
             "dW2": synth.grad_init(cfg, (H, Fs), 3)}
    gpu = gpu_block(tp, inp, w.act, w.dtype, w.has_bias, accumulate_into=prior)
    say("  oracle on the whole shard")
    ref = oracle_block(inp, w.act, w.has_bias, prior=prior)
    check(gpu, ref, w.dtype, ALL)
