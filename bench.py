"""Benchmark: one tensor-parallel rank's column->row MLP block, forward +
backward (dgrad + wgrad), bf16 inputs with fp32 accumulation, on one MI355X.

One step = tpmlp_fwd + tpmlp_bwd_dgrad + tpmlp_bwd_wgrad over one batch of
synthetic per-rank inputs (default workload: T = 8192 tokens (4 x 2048),
H = 8192, F = 32768 at TP = 8, i.e. Fs = 4096). Inputs and all output
buffers are resident in HBM before the timed region.

Parity comes first: one step in the timed steps' launch configuration runs
before them, and its outputs are compared, tensor by tensor, with the CPU
oracle on the whole workload (max|gpu - oracle| / max|oracle| within 1e-5
for fp32, 2e-2 for bf16, 6e-2 for e4m3) before anything is reported; on a
miss the script exits with status 3 and prints no line.

The timed steps follow untimed warm-up steps (by default as many as fill
100 ms, at least 30: the shader clock ramps up over the first tens of
milliseconds of load), so the line reports the sustained rate.

Then prints one JSON line: TFLOP/s of the whole step (algorithmic FLOPs
6*T*H*Fs*(G+1) over the measured time), its fraction of the vendor peak and
of the peak at the shader clock the kernels measured themselves, the parity
errors, the dominant kernel's roofline (its average launch time from HIP
events recorded on its launch stream during the timed steps) and the CPU
oracle's throughput on a bounded sample.

FP8 (e4m3) steps: x, W1, W2 are E4M3 codes and dy E5M2 codes, quantised
once before the timed region (per-tensor current scaling); inside it the
block quantises a (E4M3) and dH (E5M2) with delayed scaling, the history
update included. ``--calls`` picks the entry points of a step (the 12288-
hidden FP8 shard is forward only unless asked for more); ``--dtype``
overrides the workload's dtype.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK = {"bf16": 2516.6, "f32": 157.3, "e4m3": 5033.2}
# MFMA FLOP per CU per clock (dense), for the peak at a measured clock
FLOP_PER_CU_CLK = {"bf16": 4096, "f32": 256, "e4m3": 8192}
N_CU = 256
# parity tolerance per output tensor, max|gpu - oracle| / max|oracle|
TOL = {"f32": 1e-5, "bf16": 2e-2, "e4m3": 6e-2}
HBM_PEAK_GBS = 8000.0
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
HISTORY_LEN = 1024  # delayed-scaling amax history (the common default length)
# default warm-up: the shader clock ramps up over the first tens of
# milliseconds under load (a 400-step run of the 8192-hidden shard settles
# after about 25 steps, 60 ms, and stays there), so the untimed steps fill
# WARMUP_S of GPU time
WARMUP_S = 0.1
MIN_WARMUP = 30


def traffic_file(name: str) -> str:
    return os.path.join(TRAFFIC_DIR, f"traffic_{name}.json")
COPY_BYTES = 1 << 30  # the calibration copy
KERNEL_SOURCES = ["gemm_mfma.h", "epilogue.h", "common.h", "kernels_mfma.hip"]


def kernel_source_sha() -> str:
    """Hash of the GEMM kernel's code (comments and whitespace left out, so
    that only a change of the code itself marks the counters stale)."""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "tensor_transformer_mlp_rank_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(name: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    runs of workload `name`, or None when absent or when the kernel source
    changed since."""
    try:
        with open(traffic_file(name)) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != kernel_source_sha() or t.get("workload") != name:
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def step_labels(w, calls, wgrad_t=False) -> list:
    """The library's launches in one step (the given entry points among
    forward, dgrad, wgrad), in order, under the names its timing facility
    gives them. wgrad_t: the E4M3 weight gradients from token-contiguous
    operands (a and dH transposed first)."""
    sfx = "." + w.dtype
    fp8 = w.dtype == "e4m3"
    seq = []
    if "fwd" in calls:
        seq += ["fc1_fwd", "a_scale_update", "fc2_fwd"] if fp8 else ["fc1_fwd", "fc2_fwd"]
    if "dgrad" in calls:
        seq += ["fc2_dgrad", "dH_scale_update", "fc1_dgrad"] if fp8 else ["fc2_dgrad", "fc1_dgrad"]
    if "wgrad" in calls:
        if wgrad_t:
            seq += ["transpose_u8", "transpose_u8"]
        seq += ["fc2_wgrad", "fc1_wgrad"]
        if w.has_bias and w.dtype != "f32":
            # adds up the fused column-sum partials, or sums dH's token-contiguous rows
            seq.append("db1_rowsum" if wgrad_t else "db1_reduce")
    return [k if k == "transpose_u8" else k + sfx for k in seq]


def _counter_rows(d: str) -> list:
    import csv
    with open(os.path.join(d, "run_counter_collection.csv")) as fh:
        return sorted(csv.DictReader(fh), key=lambda r: int(r["Dispatch_Id"]))


def write_traffic(name, labels, setup, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir,
                  commands) -> dict:
    """HBM bytes per launch of each kernel of the step, from rocprofv3 --pmc
    FETCH_SIZE and WRITE_SIZE runs of this script (KiB per dispatch), each
    scaled by what the same counter reads for the plain 1 GiB device copy of
    --copy-calibration. Dispatches of the library are matched to step labels
    by launch order; a split-K product's reduce pass counts with its GEMM, and
    the fill that clears a split product's counters with the GEMM after it."""
    import statistics
    copy_bytes = float(COPY_BYTES)

    def copy_kib(d):
        v = [float(r["Counter_Value"]) for r in _counter_rows(d) if "copyBuffer" in r["Kernel_Name"]]
        if not v:
            raise SystemExit(f"no copy kernel dispatch in {d}")
        return statistics.median(v)

    def kname(r):
        return r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]

    scale = {"FETCH_SIZE": copy_bytes / (copy_kib(copy_fetch_dir) * 1024.0),
             "WRITE_SIZE": copy_bytes / (copy_kib(copy_write_dir) * 1024.0)}
    per = {}
    for d, counter in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        rows = [r for r in _counter_rows(d)
                if "tpmlp::" in r["Kernel_Name"] and r["Counter_Name"] == counter]
        rows = rows[setup:]  # one-off set-up launches (the FP8 step quantises its inputs)
        li, step, cur, first = 0, 0, None, True
        sums = {}
        held = []  # fills launched ahead of their product
        for r in rows:
            kn = kname(r)
            if "fill_zero" in kn:
                held.append(r)
                continue
            if "splitk_reduce" in kn and cur is not None:
                lab = cur  # the reduce pass of the product just launched
            else:
                first = step == 0  # the first step records each label's kernels
                lab = labels[li]
                li += 1
                if li == len(labels):
                    li, step = 0, step + 1
                cur = lab
            k = per.setdefault(lab, {"kernels": []})
            for n in [kname(x) for x in held] + [kn]:
                if first:
                    if n not in k["kernels"]:
                        k["kernels"].append(n)
                elif n not in k["kernels"]:
                    raise SystemExit(f"dispatch order does not match the step: {n} as {lab}")
            for x in held + [r]:
                sums.setdefault(lab, []).append(float(x["Counter_Value"]) * 1024.0 * scale[counter])
            held = []
        if li != 0 or step == 0:
            raise SystemExit(f"{d}: {len(rows)} library dispatches after the set-up, not whole "
                             f"steps of {labels}")
        for lab, v in sums.items():
            per[lab][counter] = sum(v) / step
            per[lab]["steps"] = step
    kernels = {}
    for label in labels:
        k = per[label]
        fetch, write = k["FETCH_SIZE"], k["WRITE_SIZE"]
        kernels[label] = {"kernel": " + ".join(k["kernels"]), "dispatches": k["steps"],
                          "fetch_bytes": round(fetch), "write_bytes": round(write),
                          "bytes_per_launch": round(fetch + write)}
    out = {"source_sha": kernel_source_sha(), "workload": name, "labels": list(labels),
           "scale": {"FETCH_SIZE": round(scale["FETCH_SIZE"], 4),
                     "WRITE_SIZE": round(scale["WRITE_SIZE"], 4)},
           "commands": commands, "kernels": kernels}
    with open(traffic_file(name), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    return out

def _cpu_cores() -> int:
    """Threads of the BLAS the oracle runs on (else the affinity count)."""
    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 0) for p in threadpool_info()
                     if p.get("internal_api") in ("openblas", "mkl", "blis")), default=0)
    except Exception:  # threadpoolctl missing: report the affinity count
        cores = 0
    return cores or len(os.sched_getaffinity(0))


def rel_err(got, ref) -> float:
    """max |gpu - oracle| / max |oracle| over one output tensor (the
    tolerance metric of the block)."""
    import numpy as np
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise SystemExit(f"parity: shape {got.shape} against the oracle's {ref.shape}")
    if ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(got - ref)))
    return num / den if den > 0 else num


def parity_report(gpu: dict, ref: dict, tol: dict) -> dict:
    """Per-tensor relative errors of the device's parity step against the
    oracle, and whether every one is within its tolerance."""
    errs = {k: rel_err(gpu[k], ref[k]) for k in tol if gpu.get(k) is not None
            and ref.get(k) is not None}
    bad = {k: v for k, v in errs.items() if not v <= tol[k]}
    return {"max_rel_err": {k: float(f"{v:.3e}") for k, v in errs.items()},
            "tol": {k: tol[k] for k in errs}, "pass": not bad}


def _mlp_oracle(w, calls, x, W1, b1, W2, dy, fp8, a_scale, dH_scale) -> dict:
    """The oracle's outputs for the step's entry points (fp8: its FP8 block
    at the scales the device quantised a and dH with)."""
    import oracle
    out = {}
    if fp8:
        f = oracle.rank_forward_fp8(x, W1, b1, W2, a_scale, w.act)
        out.update(y=f["y"], h=f["h"], a=f["a"])
        if "dgrad" in calls:
            g = oracle.rank_dgrad_fp8(dy, W1, W2, f["h"], dH_scale, w.act)
            out.update(dx=g["dx"])
            if "wgrad" in calls:
                out.update(oracle.rank_wgrad_fp8(dy, x, f["a_q"], g["dH_q"]))
                if not w.has_bias:
                    out["db1"] = None
    else:
        f = oracle.rank_forward(x, W1, b1, W2, w.act)
        out.update(y=f["y"], h=f["h"], a=f["a"])
        if "dgrad" in calls:
            g = oracle.rank_dgrad(dy, W1, W2, f["h"], w.act)
            out.update(dH=g["dH"], dx=g["dx"])
            if "wgrad" in calls:
                out.update(oracle.rank_wgrad(dy, x, f["a"], g["dH"], w.has_bias))
    return out


def cpu_baseline(w, calls, tokens: int, repeats: int = 3, gpu=None) -> dict:
    """The CPU oracle (fp64 NumPy, as it stands) on the first `tokens` tokens
    of the same per-rank shard: the step's entry points (for e4m3, the
    oracle's FP8 block on the dequantised codes). With `gpu` (the outputs of
    the device's parity step on the whole shard, and for e4m3 the scales it
    quantised a and dH with), the oracle also runs once on the whole shard and
    every output is compared with the device's: the result's "parity"."""
    import numpy as np
    import oracle
    import synth
    cores = _cpu_cores()
    fp8 = w.dtype == "e4m3"
    tol = {"y": TOL[w.dtype], "h": TOL["bf16" if fp8 else w.dtype], "a": TOL[w.dtype],
           "dH": TOL[w.dtype], "dx": TOL[w.dtype], "dW1": TOL[w.dtype], "db1": TOL[w.dtype],
           "dW2": TOL[w.dtype]}
    if fp8:
        tol.pop("dH")  # E5M2 codes: checked through dx, dW1 and db1 (one code step exceeds 6e-2)

    def inputs(n):
        inp = synth.make_rank_inputs(w, tokens=n)
        x, W1, W2, dy = (oracle.to_f64(inp[k]) for k in ("x", "W1", "W2", "dy"))
        b1 = oracle.to_f64(inp["b1"]) if w.has_bias else None
        if fp8:
            # the codes the device is given (per-tensor current scaling), dequantised
            def deq(v, fmt):
                _, s, s_inv = oracle.current_scale(v, fmt)
                return oracle.dequantize(oracle.quantize(v, fmt, s), fmt, s_inv)
            x, W1, W2 = deq(x, "e4m3"), deq(W1, "e4m3"), deq(W2, "e4m3")
            dy = deq(dy, "e5m2")
        return x, W1, b1, W2, dy

    parity = None
    times = []
    if gpu is not None:
        full = inputs(w.tokens)
        t0 = time.perf_counter()
        ref = _mlp_oracle(w, calls, *full, fp8, gpu.get("a_scale"), gpu.get("dH_scale"))
        dt_full = time.perf_counter() - t0
        parity = parity_report(gpu, ref, tol)
        ref = full = None
        if tokens == w.tokens:
            times.append(dt_full)  # the whole shard is also the timed sample
    if tokens <= 0:
        return None, parity
    x, W1, b1, W2, dy = inputs(tokens)
    a_scale = dH_scale = None
    if fp8:
        # the scales of a and dH as delayed scaling would settle on them
        f0 = oracle.rank_forward(x, W1, b1, W2, w.act)
        a_scale = np.float32(448.0 / np.max(np.abs(f0["a"])))
        dH_scale = np.float32(57344.0 / np.max(np.abs(
            oracle.rank_dgrad(dy, W1, W2, f0["h"], w.act)["dH"]))) if "dgrad" in calls else None
        del f0
    while len(times) < repeats:
        t0 = time.perf_counter()
        _mlp_oracle(w, calls, x, W1, b1, W2, dy, fp8, a_scale, dH_scale)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    flops = w.flops(tokens=tokens, calls=calls)
    res = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
           "kind": "oracle",
           "sample": f"{'+'.join(calls)} of the first {tokens} of {w.tokens} tokens of the "
                     f"{w.name} shard in fp64 NumPy, median of {repeats} runs "
                     f"({flops / 1e12:.3f} TFLOP per run, {dt:.2f} s, {sum(times):.1f} s total)"}
    return res, parity


def _attn_oracle(x, W, b, Wo, dy, ctx, dqkv) -> dict:
    from oracle import attention as oa
    dWqkv, dbqkv = oa.qkv_wgrad(dqkv, x, has_bias=b is not None)
    return {"qkv": oa.qkv_forward(x, W, b), "y": oa.out_forward(ctx, Wo),
            "dctx": oa.out_dgrad(dy, Wo), "dWo": oa.out_wgrad(dy, ctx),
            "dx": oa.qkv_dgrad(dqkv, W), "dWqkv": dWqkv, "dbqkv": dbqkv}


def attn_cpu_baseline(w, tokens: int, repeats: int = 3, gpu=None) -> dict:
    """The CPU oracle's per-rank attention projections (fp64 NumPy, as it
    stands) on the first `tokens` tokens: the six products of a step. With
    `gpu`, also compared on the whole shard with the device's parity step."""
    import oracle
    import synth
    cores = _cpu_cores()

    def inputs(n):
        inp = synth.make_attn_inputs(w, tokens=n)
        x, W, Wo, dy, ctx, dqkv = (oracle.to_f64(inp[k])
                                   for k in ("x", "Wqkv", "Wo", "dy", "ctx", "dqkv"))
        b = oracle.to_f64(inp["bqkv"]) if inp["bqkv"] is not None else None
        return x, W, b, Wo, dy, ctx, dqkv

    parity, times = None, []
    if gpu is not None:
        full = inputs(w.tokens)
        t0 = time.perf_counter()
        ref = _attn_oracle(*full)
        dt_full = time.perf_counter() - t0
        parity = parity_report(gpu, ref, {k: TOL[w.dtype] for k in ref})
        ref = full = None
        if tokens == w.tokens:
            times.append(dt_full)
    if tokens <= 0:
        return None, parity
    args = inputs(tokens)
    while len(times) < repeats:
        t0 = time.perf_counter()
        _attn_oracle(*args)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    flops = w.flops(tokens=tokens)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"the six projection products of the first {tokens} of {w.tokens} tokens of "
                      f"the {w.name} shard in fp64 NumPy, median of {repeats} runs "
                      f"({flops / 1e12:.3f} TFLOP per run, {dt:.2f} s, {sum(times):.1f} s total)"}, parity


def host_outputs(dev: dict) -> dict:
    """The parity step's device outputs on the host: arrays, and the scales
    as float32 scalars."""
    import numpy as np
    out = {}
    for k, v in dev.items():
        if v is None:
            out[k] = None
        elif k.endswith("_scale"):
            out[k] = np.float32(v.item())
        else:
            out[k] = v.cpu().numpy()
    return out


class Job:
    """One benchmark step: its calls (name, function), the library launches
    they make in order, algorithmic FLOPs, and what the JSON line reports."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def mlp_job(tp, torch, w, calls, dev, wgrad_t=False) -> Job:
    """The MLP block: forward, dgrad, wgrad (accumulate) on one rank's shard.
    wgrad_t (E4M3): the weight gradients through tpmlp_bwd_wgrad_t, with x
    and dy given token-contiguous as well (transposed with the inputs'
    quantisation, before the timed steps) and a and dH transposed inside the
    step."""
    import synth
    inp = synth.make_rank_inputs(w)
    d = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    T, H, Fs, G = w.tokens, w.hidden, w.ffn_shard, w.gate_mult
    desc = tp.make_desc(T, H, Fs, act=w.act, dtype=w.dtype, has_bias=w.has_bias)
    fp8 = w.dtype == "e4m3"
    at = torch.bfloat16 if w.dtype in ("bf16", "e4m3") else torch.float32
    qt = torch.uint8 if fp8 else at  # a and dH: FP8 codes in the e4m3 step
    buf = {
        "y": torch.empty((T, H), dtype=at, device=dev),
        "h": torch.empty((T, G * Fs), dtype=at, device=dev),
        "a": torch.empty((T, Fs), dtype=qt, device=dev),
        "dH": torch.empty((T, G * Fs), dtype=qt, device=dev),
        "dx": torch.empty((T, H), dtype=at, device=dev),
        "dW1": torch.zeros((G * Fs, H), dtype=torch.float32, device=dev),
        "db1": torch.zeros((G * Fs,), dtype=torch.float32, device=dev) if w.has_bias else None,
        "dW2": torch.zeros((H, Fs), dtype=torch.float32, device=dev),
    }
    ws = {}
    for c, code in (("fwd", tp.CALL_FWD), ("dgrad", tp.CALL_DGRAD), ("wgrad", tp.CALL_WGRAD)):
        n = tp.workspace_size(desc, code)
        ws[c] = torch.empty(n, dtype=torch.uint8, device=dev) if n else None
    sc = {"fwd": None, "dgrad": None, "wgrad": None}
    if fp8:
        # inputs as FP8 codes (current scaling, once); a and dH under delayed scaling
        sinv = {}
        for k, e5 in (("x", False), ("W1", False), ("W2", False), ("dy", True)):
            codes, _, sinv[k] = tp.quantize_e4m3(d[k], stream=torch.cuda.current_stream(), e5m2=e5)
            d[k] = codes
        a_hist, dH_hist = tp.DelayedScaling(HISTORY_LEN), tp.DelayedScaling(HISTORY_LEN)
        sc["fwd"] = tp.fp8_scales(sinv["x"], sinv["W1"], sinv["W2"], a_history=a_hist)
        sc["dgrad"] = tp.fp8_scales(w1_scale_inv=sinv["W1"], w2_scale_inv=sinv["W2"],
                                    dy_scale_inv=sinv["dy"], dH_history=dH_hist)
        sc["wgrad"] = tp.fp8_scales(x_scale_inv=sinv["x"], a_scale_inv=a_hist.scale_inv,
                                    dy_scale_inv=sinv["dy"], dH_scale_inv=dH_hist.scale_inv)
        if wgrad_t:
            d["x_t"], d["dy_t"] = tp.transpose_u8(d["x"]), tp.transpose_u8(d["dy"])
            buf["a_t"] = torch.empty((Fs, tp.token_ld(T)), dtype=torch.uint8, device=dev)
            buf["dH_t"] = torch.empty((G * Fs, tp.token_ld(T)), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
    elif wgrad_t:
        raise SystemExit("--wgrad-t: E4M3 workloads only")
    stream = torch.cuda.current_stream()

    def fwd():
        tp.tpmlp_fwd(desc, d["x"], d["W1"], d["b1"], d["W2"], buf["y"], buf["h"], buf["a"],
                     fp8=sc["fwd"], workspace=ws["fwd"], stream=stream)

    def dgrad():
        tp.tpmlp_bwd_dgrad(desc, d["dy"], d["W1"], d["W2"], buf["h"], buf["dH"], buf["dx"],
                           fp8=sc["dgrad"], workspace=ws["dgrad"], stream=stream)

    def wgrad():
        if wgrad_t:
            tp.tpmlp_transpose_u8(buf["a"], T, Fs, buf["a_t"], stream=stream)
            tp.tpmlp_transpose_u8(buf["dH"], T, G * Fs, buf["dH_t"], stream=stream)
            tp.tpmlp_bwd_wgrad_t(desc, d["dy_t"], d["x_t"], buf["a_t"], buf["dH_t"], buf["dW1"],
                                 buf["db1"], buf["dW2"], accumulate=True, fp8=sc["wgrad"],
                                 stream=stream)
            return
        tp.tpmlp_bwd_wgrad(desc, d["dy"], d["x"], buf["a"], buf["dH"], buf["dW1"], buf["db1"],
                           buf["dW2"], accumulate=True, fp8=sc["wgrad"], workspace=ws["wgrad"],
                           stream=stream)

    fns = {"fwd": fwd, "dgrad": dgrad, "wgrad": wgrad}

    def parity_step() -> dict:
        """One step on zeroed gradient buffers (accumulating into zeros is
        the plain result), in the timed steps' launch configuration; float32
        copies of its outputs on the device (the FP8 codes of a dequantised,
        and the scales a and dH were quantised at), for host_outputs() after
        the timed steps."""
        for k in ("dW1", "db1", "dW2"):
            if buf[k] is not None:
                buf[k].zero_()
        out = {}
        if fp8:
            out = {"a_scale": a_hist.scale.clone(), "dH_scale": dH_hist.scale.clone()}
        for c in calls:
            fns[c]()
        dev32 = lambda t: None if t is None else t.float().clone()
        out.update(y=dev32(buf["y"]), h=dev32(buf["h"]))
        if fp8:
            out["a"] = buf["a"].view(torch.float8_e4m3fn).float() * a_hist.scale_inv
        else:
            out["a"] = dev32(buf["a"])
        if "dgrad" in calls:
            out["dx"] = dev32(buf["dx"])
            if not fp8:
                out["dH"] = dev32(buf["dH"])
            if "wgrad" in calls:
                out.update(dW1=dev32(buf["dW1"]), dW2=dev32(buf["dW2"]), db1=dev32(buf["db1"]))
        return out

    what = "fwd+bwd" if calls == ("fwd", "dgrad", "wgrad") else "+".join(calls)
    return Job(
        name=w.name, dtype=w.dtype, stream=stream,
        fns=[(c, fns[c]) for c in calls], parity_step=parity_step,
        labels=step_labels(w, calls, wgrad_t), flops=w.flops(calls=calls),
        # fc1's GEMMs have T*H*G*Fs multiply-adds each, fc2's T*H*Fs
        gemm_flops=lambda lab: 2.0 * T * H * Fs * (G if lab.startswith("fc1") else 1),
        metric=f"TFLOP/s per-rank TP-MLP {what} ({w.dtype}) and % of MFMA peak, 1 MI355X",
        config={"workload": w.name, "tokens": T, "batch": w.batch, "seq_len": w.seq,
                "hidden": H, "ffn": w.ffn, "tp": w.tp, "ffn_shard": Fs, "act": w.act,
                "parallelism": "one TP rank's shard on one GPU",
                **({"wgrad_operands": "token-contiguous"} if wgrad_t else {})},
        cpu=lambda n, gpu: cpu_baseline(w, calls, n, gpu=gpu))


def attn_job(tp, torch, w, dev) -> Job:
    """The attention block's two projections, forward and backward, on one
    rank's shard: packed QKV, output projection, their dgrads and wgrads
    (accumulate). The core attention between them is not the library's and
    is not run; its output ctx and input gradient dqkv are synthetic."""
    import synth
    inp = synth.make_attn_inputs(w)
    d = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    T, H, N, D = w.tokens, w.hidden, w.nqkv, w.d
    has_bias = w.b_std is not None
    desc = tp.make_attn_desc(T, H, w.q_heads_rank, w.kv_heads_rank, w.head_dim, dtype=w.dtype,
                             has_bias=has_bias)
    at = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    buf = {"qkv": torch.empty((T, N), dtype=at, device=dev),
           "y": torch.empty((T, H), dtype=at, device=dev),
           "dctx": torch.empty((T, D), dtype=at, device=dev),
           "dx": torch.empty((T, H), dtype=at, device=dev),
           "dWo": torch.zeros((H, D), dtype=torch.float32, device=dev),
           "dWqkv": torch.zeros((N, H), dtype=torch.float32, device=dev),
           "dbqkv": torch.zeros((N,), dtype=torch.float32, device=dev) if has_bias else None}
    n = tp.attn_workspace_size(desc)
    ws = torch.empty(n, dtype=torch.uint8, device=dev) if n else None
    stream = torch.cuda.current_stream()

    def fwd():
        tp.tpmlp_attn_qkv_fwd(desc, d["x"], d["Wqkv"], d["bqkv"], buf["qkv"], stream=stream)
        tp.tpmlp_attn_out_fwd(desc, d["ctx"], d["Wo"], buf["y"], stream=stream)

    def bwd():
        tp.tpmlp_attn_out_bwd_dgrad(desc, d["dy"], d["Wo"], buf["dctx"], ws, stream=stream)
        tp.tpmlp_attn_out_bwd_wgrad(desc, d["dy"], d["ctx"], buf["dWo"], True, ws, stream=stream)
        tp.tpmlp_attn_qkv_bwd_dgrad(desc, d["dqkv"], d["Wqkv"], buf["dx"], stream=stream)
        tp.tpmlp_attn_qkv_bwd_wgrad(desc, d["dqkv"], d["x"], buf["dWqkv"], buf["dbqkv"], True,
                                    ws, stream=stream)

    def parity_step() -> dict:
        for k in ("dWo", "dWqkv", "dbqkv"):
            if buf[k] is not None:
                buf[k].zero_()
        fwd()
        bwd()
        return {k: (None if v is None else v.float().clone()) for k, v in
                (("qkv", buf["qkv"]), ("y", buf["y"]), ("dctx", buf["dctx"]), ("dWo", buf["dWo"]),
                 ("dx", buf["dx"]), ("dWqkv", buf["dWqkv"]), ("dbqkv", buf["dbqkv"]))}

    sfx = "." + w.dtype
    labels = [k + sfx for k in ("qkv_fwd", "out_fwd", "out_dgrad", "out_wgrad", "qkv_dgrad",
                                "qkv_wgrad")]
    if has_bias and w.dtype != "f32":
        labels.append("dbqkv_reduce" + sfx)
    return Job(
        name=w.name, dtype=w.dtype, stream=stream, fns=[("fwd", fwd), ("bwd", bwd)],
        parity_step=parity_step,
        labels=labels, flops=w.flops(),
        gemm_flops=lambda lab: 2.0 * T * H * (N if lab.startswith("qkv") else D),
        metric=f"TFLOP/s per-rank TP attention projections fwd+bwd ({w.dtype}) and % of MFMA "
               f"peak, 1 MI355X",
        config={"workload": w.name, "tokens": T, "batch": w.batch, "seq_len": w.seq,
                "hidden": H, "heads": w.heads, "kv_heads": w.kv_heads, "head_dim": w.head_dim,
                "tp": w.tp, "qkv_shard": N, "ctx_shard": D,
                "parallelism": "one TP rank's shard on one GPU"},
        cpu=lambda n, gpu: attn_cpu_baseline(w, n, gpu=gpu))


def moe_labels(w) -> list:
    labels = ["moe_fc1_fwd", "moe_fc2_fwd", "moe_fc2_dgrad", "moe_fc1_dgrad", "moe_fc2_wgrad",
              "moe_fc1_wgrad"]
    if w.has_bias:
        labels.append("moe_db1_reduce")
    return [k + "." + w.dtype for k in labels]


def moe_job(tp, torch, w, dev) -> Job:
    """The local experts of a mixture-of-experts layer: grouped forward,
    dgrad, wgrad (accumulate) over the rows of a seeded synthetic routing.
    The dispatch and combine around them are not the library's and are not
    run."""
    import synth
    import numpy as np
    counts = synth.moe_counts(w)
    inp = synth.make_moe_inputs(w, counts)
    d = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    T, H, Fs, G, E = int(counts.sum()), w.hidden, w.ffn_shard, w.gate_mult, w.experts
    desc = tp.make_moe_desc(T, H, Fs, E, act=w.act, dtype=w.dtype, has_bias=w.has_bias)
    bf = torch.bfloat16
    buf = {"y": torch.empty((T, H), dtype=bf, device=dev),
           "h": torch.empty((T, G * Fs), dtype=bf, device=dev),
           "a": torch.empty((T, Fs), dtype=bf, device=dev),
           "dH": torch.empty((T, G * Fs), dtype=bf, device=dev),
           "dx": torch.empty((T, H), dtype=bf, device=dev),
           "dW1": torch.zeros((E, G * Fs, H), dtype=torch.float32, device=dev),
           "db1": torch.zeros((E, G * Fs), dtype=torch.float32, device=dev) if w.has_bias else None,
           "dW2": torch.zeros((E, H, Fs), dtype=torch.float32, device=dev)}
    n = tp.moe_workspace_size(desc)
    ws = torch.empty(n, dtype=torch.uint8, device=dev) if n else None
    stream = torch.cuda.current_stream()
    c = d["counts"]

    def fwd():
        tp.tpmlp_moe_fwd(desc, c, d["x"], d["W1"], d["b1"], d["W2"], buf["y"], buf["h"], buf["a"],
                         stream=stream)

    def dgrad():
        tp.tpmlp_moe_bwd_dgrad(desc, c, d["dy"], d["W1"], d["W2"], buf["h"], buf["dH"], buf["dx"],
                               stream=stream)

    def wgrad():
        tp.tpmlp_moe_bwd_wgrad(desc, c, d["dy"], d["x"], buf["a"], buf["dH"], buf["dW1"],
                               buf["db1"], buf["dW2"], True, ws, stream=stream)

    def parity_step() -> dict:
        for k in ("dW1", "db1", "dW2"):
            if buf[k] is not None:
                buf[k].zero_()
        fwd()
        dgrad()
        wgrad()
        return {k: (None if v is None else v.float().clone()) for k, v in buf.items()}

    return Job(
        name=w.name, dtype=w.dtype, stream=stream, parity_step=parity_step,
        fns=[("fwd", fwd), ("dgrad", dgrad), ("wgrad", wgrad)], labels=moe_labels(w),
        flops=w.flops(T),
        gemm_flops=lambda lab: 2.0 * T * H * Fs * (G if lab.startswith("moe_fc1") else 1),
        metric=f"TFLOP/s per-rank MoE expert MLPs fwd+bwd ({w.dtype}) and % of MFMA peak, "
               f"1 MI355X",
        config={"workload": w.name, "tokens": w.tokens, "routed_rows": T, "experts": E,
                "topk": w.topk, "hidden": H, "expert_ffn_shard": Fs, "act": w.act,
                "rows_per_expert_min": int(np.min(counts)),
                "rows_per_expert_max": int(np.max(counts)),
                "parallelism": "one rank's local experts on one GPU"},
        cpu=lambda nt, gpu: moe_cpu_baseline(w, counts, nt, gpu=gpu))


def _moe_oracle(x, dy, W1, b1, W2, counts, act, has_bias) -> dict:
    from oracle import moe as om
    f = om.grouped_forward(x, counts, W1, b1, W2, act)
    g = om.grouped_dgrad(dy, counts, W1, W2, f["h"], act)
    wg = om.grouped_wgrad(dy, x, f["a"], g["dH"], counts, has_bias)
    return {**f, **g, **wg}


def moe_cpu_baseline(w, counts, rows: int, repeats: int = 3, gpu=None) -> dict:
    """The CPU oracle's grouped block (fp64 NumPy, as it stands) on the
    first `rows` routed rows (the leading experts' groups, the last one cut).
    With `gpu`, also compared on every routed row with the device's parity
    step."""
    import numpy as np
    import oracle
    import synth
    cores = _cpu_cores()
    cum = np.cumsum(counts)
    sub = [int(min(c, max(rows - (s - c), 0))) for c, s in zip(counts, cum)]
    k = max(i + 1 for i, c in enumerate(sub) if c > 0) if any(sub) else 1
    sub = sub[:k]  # the experts the sample reaches
    inp = synth.make_moe_inputs(w, counts)
    n = sum(sub)
    parity, times = None, []
    if gpu is not None:
        full = (oracle.to_f64(inp["x"]), oracle.to_f64(inp["dy"]), oracle.to_f64(inp["W1"]),
                oracle.to_f64(inp["b1"]) if w.has_bias else None, oracle.to_f64(inp["W2"]))
        t0 = time.perf_counter()
        ref = _moe_oracle(*full, counts, w.act, w.has_bias)
        dt_full = time.perf_counter() - t0
        parity = parity_report(gpu, ref, {k2: TOL[w.dtype] for k2 in ref})
        ref = full = None
        if n == int(np.sum(counts)):
            times.append(dt_full)
    if rows <= 0:
        return None, parity
    x, dy = oracle.to_f64(inp["x"][:n]), oracle.to_f64(inp["dy"][:n])
    W1, W2 = oracle.to_f64(inp["W1"][:k]), oracle.to_f64(inp["W2"][:k])
    b1 = oracle.to_f64(inp["b1"][:k]) if w.has_bias else None
    while len(times) < repeats:
        t0 = time.perf_counter()
        _moe_oracle(x, dy, W1, b1, W2, sub, w.act, w.has_bias)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    flops = w.flops(n)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"fwd+dgrad+wgrad of the first {n} of {int(np.sum(counts))} routed rows "
                      f"(experts 0..{k - 1}) of the {w.name} layer in fp64 NumPy, median of "
                      f"{repeats} runs "
                      f"({flops / 1e12:.3f} TFLOP per run, {dt:.2f} s, {sum(times):.1f} s total)"}, parity


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: as many as take "
                         f"{WARMUP_S * 1e3:.0f} ms, at least {MIN_WARMUP}: the shader clock "
                         "ramps up over the first tens of milliseconds of load)")
    ap.add_argument("--workload", type=int, default=3,
                    help="workload id (3: H=8192 TP=8 MLP shard; 6, 7: attention projections; "
                         "8, 9: mixture-of-experts expert MLPs)")
    ap.add_argument("--wgrad-t", action="store_true",
                    help="E4M3 MLP: weight gradients from token-contiguous operands "
                         "(tpmlp_bwd_wgrad_t; a and dH transposed inside the step)")
    ap.add_argument("--calls", default=None,
                    help="MLP: entry points of a step, comma-separated among fwd,dgrad,wgrad "
                         "(default: the workload's)")
    ap.add_argument("--dtype", default=None, choices=["f32", "bf16", "e4m3"],
                    help="override the workload's dtype")
    ap.add_argument("--cpu-tokens", type=int, default=8192,
                    help="tokens in the CPU oracle's timed sample (0: no cpu_baseline; the "
                         "parity check on the whole workload runs either way)")
    ap.add_argument("--breakdown", action="store_true", help="print per-kernel times to stderr")
    ap.add_argument("--cold", action="store_true",
                    help="also time the steps with caches flushed before each (a 512 MiB buffer "
                         "is written between steps, outside the timed spans)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the reference "
                         "kernel for scaling HBM byte counters)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="no GPU: write profiles/traffic_<workload>.json from four rocprofv3 "
                         "--pmc output folders (FETCH_SIZE and WRITE_SIZE of this benchmark, then "
                         "of --copy-calibration)")
    ap.add_argument("--command", action="append", default=[],
                    help="with --write-traffic: the commands that made the folders (recorded)")
    args = ap.parse_args()
    import dataclasses
    import synth
    attn = args.workload in synth.ATTN_WORKLOADS
    moe = args.workload in synth.MOE_WORKLOADS
    if moe:
        w = synth.MOE_WORKLOADS[args.workload]
        if (args.dtype and args.dtype != w.dtype) or args.calls:
            raise SystemExit("the expert workloads run bf16 forward + backward")
        calls = ("fwd", "dgrad", "wgrad")
    elif attn:
        w = synth.ATTN_WORKLOADS[args.workload]
        if args.dtype and args.dtype != w.dtype:
            if args.dtype == "e4m3":
                raise SystemExit("the attention projections have no FP8 path")
            w = dataclasses.replace(w, dtype=args.dtype, name=w.name.replace(w.dtype, args.dtype))
        if args.calls:
            raise SystemExit("--calls applies to the MLP workloads")
        calls = ("fwd", "bwd")
    else:
        w = synth.WORKLOADS[args.workload]
        if args.dtype and args.dtype != w.dtype:
            w = dataclasses.replace(w, dtype=args.dtype, name=w.name.replace(w.dtype, args.dtype))
        calls = tuple(args.calls.split(",")) if args.calls else w.calls
        if not calls or any(c not in ("fwd", "dgrad", "wgrad") for c in calls) \
                or calls[0] != "fwd" or ("wgrad" in calls and "dgrad" not in calls):
            raise SystemExit("--calls: fwd, then optionally dgrad, then optionally wgrad")
    if args.write_traffic:
        if moe:
            labels, setup = moe_labels(w), 0
        elif attn:
            sfx = "." + w.dtype
            labels = [k + sfx for k in ("qkv_fwd", "out_fwd", "out_dgrad", "out_wgrad",
                                        "qkv_dgrad", "qkv_wgrad")]
            if w.b_std is not None and w.dtype != "f32":
                labels.append("dbqkv_reduce" + sfx)
            setup = 0
        else:
            labels = step_labels(w, calls, args.wgrad_t)
            # the FP8 step quantises its four inputs (and with --wgrad-t
            # transposes x and dy)
            setup = (10 if args.wgrad_t else 8) if w.dtype == "e4m3" else 0
        out = write_traffic(w.name, labels, setup, *args.write_traffic, args.command)
        print(json.dumps(out["kernels"], indent=1))
        return
    if args.copy_calibration:
        import torch
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4,
                          "launches": 5}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library computes one tensor-parallel rank's "
              "share and has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import tensor_transformer_mlp_rank_amd as tp

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if moe:
        job = moe_job(tp, torch, w, dev)
    elif attn:
        job = attn_job(tp, torch, w, dev)
    else:
        job = mlp_job(tp, torch, w, calls, dev, args.wgrad_t)
    stream = job.stream

    # parity first: one step in the timed steps' launch configuration, its
    # outputs kept on the host. They are compared with the oracle on the whole
    # workload after the timed steps (so that the GPU does not sit idle for the
    # oracle's seconds of CPU work right before them), and no number is
    # reported unless every tensor is within its tolerance.
    gpu_out = job.parity_step()

    def step(ev=None):
        # ev: events recorded on the launch stream before the first call and
        # after each call (they add no work to the step)
        if ev is not None:
            ev[0].record(stream)
        for j, (_, f) in enumerate(job.fns):
            f()
            if ev is not None:
                ev[j + 1].record(stream)

    def new_events():
        return [[torch.cuda.Event(enable_timing=True) for _ in range(len(job.fns) + 1)]
                for _ in range(args.steps)]

    def span_stats(ev) -> dict:
        """median / p10 / p90 of the step and the median of each call, in ms"""
        import statistics

        def q(v, f):
            v = sorted(v)
            return round(v[min(len(v) - 1, int(f * len(v)))], 4)
        st = [e[0].elapsed_time(e[-1]) for e in ev]
        return {"step_ms": {"median": round(statistics.median(st), 4), "p10": q(st, 0.1),
                            "p90": q(st, 0.9)},
                "call_ms": {c: round(statistics.median(e[j].elapsed_time(e[j + 1]) for e in ev), 4)
                            for j, (c, _) in enumerate(job.fns)}}

    # warm-up; its last (up to three) steps time every kernel, to find the
    # dominant one (the first step, with its one-off costs, only if it is the
    # only one)
    if args.warmup is None:
        # two steps to estimate a step's time, then as many as fill WARMUP_S
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        per_step = (time.perf_counter() - t) / 2
        args.warmup = max(MIN_WARMUP, 2 + math.ceil(max(WARMUP_S - 2 * per_step, 0.0) / per_step))
        nwarm = args.warmup - 2
    else:
        nwarm = max(args.warmup, 1)
    probe_from = max(1, nwarm - 3) if nwarm > 1 else 0
    for i in range(nwarm):
        if i == probe_from:
            tp.timing_enable(True)
        step()
    torch.cuda.synchronize()
    per = tp.timing_collect()
    probe_mhz = {k: round(tp.timing_clock_mhz(k), 1) for k in per}
    tp.timing_enable(False)
    # (a label launched twice in a step, the transposes of --wgrad-t, is one entry)
    if list(per) != list(dict.fromkeys(job.labels)):
        raise SystemExit(f"unexpected launch sequence {list(per)}")
    dominant = max(per, key=lambda k: per[k][1])
    breakdown = {k: round(v[1] / v[0], 4) for k, v in per.items()}
    if args.breakdown:
        print("per-kernel ms (warm-up):", json.dumps(breakdown), file=sys.stderr)

    # timed region: live events around the dominant kernel only
    tp.timing_enable(True, dominant)
    torch.cuda.synchronize()
    ev = new_events()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dom = tp.timing_collect()[dominant]
    # every GEMM kernel's clock over the timed steps (the clock capture covers
    # all of them; events bracket the dominant kernel only)
    timed_mhz = {k: round(tp.timing_clock_mhz(k), 1) for k in per}
    dom_mhz = timed_mhz.get(dominant, 0.0)
    tp.timing_enable(False)
    spans = span_stats(ev)
    cold = None
    if args.cold:
        # caches flushed before each step: 512 MiB written (more than the 256 MB
        # MALL and the 8 x 4 MB L2), outside the event spans
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cev = new_events()
        for i in range(args.steps):
            flush.fill_(i & 0xFF)
            step(cev[i])
        torch.cuda.synchronize()
        cold = span_stats(cev)
        del flush

    ms = (t1 - t0) * 1e3 / args.steps
    value = job.flops / (ms * 1e-3) / 1e12
    dom_ms = dom[1] / dom[0]
    achieved = job.gemm_flops(dominant) / (dom_ms * 1e-3) / 1e12
    peak = PEAK[job.dtype]
    # measured shader clocks (the library's workgroups read the clock and
    # real-time counters) over the timed steps: the step's is each GEMM
    # kernel's weighted by its share of the step's time (from the warm-up)
    gemm_ms = {k: v[1] for k, v in per.items() if timed_mhz.get(k, 0) > 0}
    step_mhz = (sum(timed_mhz[k] * t for k, t in gemm_ms.items()) / sum(gemm_ms.values())
                if gemm_ms else None)
    at_clock = lambda mhz: None if not mhz else N_CU * FLOP_PER_CU_CLK[job.dtype] * mhz * 1e-6
    line = {
        "metric": job.metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": job.dtype,
        "data": "synthetic (seeded PCG64 normals; per-rank shard shapes)",
        "config": job.config,
        "pct_of_peak": round(100 * value / peak, 2),
        "clock_mhz": {"step": None if step_mhz is None else round(step_mhz, 1),
                      "dominant_kernel": round(dom_mhz, 1) if dom_mhz else None,
                      "per_kernel": timed_mhz,
                      "per_kernel_warmup": probe_mhz,
                      "source": "shader clock counter over the 100 MHz real-time counter, "
                                "per workgroup of the GEMM kernels"},
        "pct_of_peak_at_clock": None if step_mhz is None else round(100 * value / at_clock(step_mhz), 2),
        "parity": None,
        "roofline": {"bound": "mfma", "kernel": dominant, "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "frac_at_clock": None if not dom_mhz else round(achieved / at_clock(dom_mhz), 4),
                     "traffic": measured_traffic(job.name, dominant),
                     "traffic_unit": "L2-to-fabric bytes per launch (rocprofv3 FETCH_SIZE + "
                                     "WRITE_SIZE, copy-calibrated; Infinity Cache hits count "
                                     "as fetched)",
                     "launches": dom[0], "avg_ms": round(dom_ms, 4)},
        "kernel_ms": breakdown,
        "spans": spans,
    }
    if cold is not None:
        line["spans_cold"] = cold
    st = [e[0].elapsed_time(e[-1]) for e in ev]
    print("step ms: " + " ".join(f"{v:.3f}" for v in st), file=sys.stderr)
    baseline, parity = job.cpu(args.cpu_tokens, host_outputs(gpu_out))
    gpu_out = None
    if not parity["pass"]:
        print(json.dumps({"parity_failed": parity, "workload": job.name}), file=sys.stderr)
        sys.exit(3)
    line["parity"] = parity
    if baseline is not None:
        line["cpu_baseline"] = baseline
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
