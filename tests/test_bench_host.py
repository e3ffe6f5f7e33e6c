"""Host-side logic of bench.py that needs no GPU: the one-GPU rule of its
command line, the launch sequences it expects from the library, and the
conversion of rocprofv3 counter files into HBM bytes per kernel (copy
calibration, split-K reduce passes counted with their product, set-up
launches skipped)."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_step_labels():
    w3, w5 = synth.WORKLOADS[3], synth.WORKLOADS[5]
    assert bench.step_labels(w3, ("fwd", "dgrad", "wgrad")) == [
        "fc1_fwd.bf16", "fc2_fwd.bf16", "fc2_dgrad.bf16", "fc1_dgrad.bf16", "fc2_wgrad.bf16",
        "fc1_wgrad.bf16", "db1_reduce.bf16"]
    assert bench.step_labels(w5, ("fwd",)) == ["fc1_fwd.e4m3", "a_scale_update.e4m3",
                                               "fc2_fwd.e4m3"]
    assert bench.moe_labels(synth.MOE_WORKLOADS[8])[-1] == "moe_fc1_wgrad.bf16"   # no bias
    assert bench.moe_labels(synth.MOE_WORKLOADS[9])[-1] == "moe_db1_reduce.bf16"


def _write_counters(d, rows):
    os.makedirs(d)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                            "Counter_Value"])
        wr.writeheader()
        for i, (k, c, v) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i + 1, "Kernel_Name": k, "Counter_Name": c,
                         "Counter_Value": v})


def test_write_traffic_maps_dispatches_to_labels(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_DIR", str(tmp_path))
    labels = ["a.bf16", "b.bf16", "c.bf16"]
    gemm = "void tpmlp::gemm_mfma_kernel<x>(tpmlp::GemmArgs, tpmlp::EpiArgs)"
    red = "tpmlp::(anonymous namespace)::splitk_reduce_kernel(float const*)"
    other = "void tpmlp::colsum_reduce_kernel(float const*)"
    setup = "void tpmlp::quantize_kernel<float, false>(float const*)"
    # one set-up launch, then two steps: a, b (split: GEMM + reduce), c
    seq = [(setup, 1.0)] + [(gemm, 10.0), (gemm, 20.0), (red, 4.0), (other, 2.0)] * 2
    for counter, sub in (("FETCH_SIZE", "f"), ("WRITE_SIZE", "w")):
        _write_counters(tmp_path / sub, [(k, counter, v) for k, v in seq])
    # the copy: 1 GiB read (FETCH_SIZE counts half of it), 1 GiB written
    _write_counters(tmp_path / "cf", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 512 * 1024)])
    _write_counters(tmp_path / "cw", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024 * 1024)])
    out = bench.write_traffic("toy", labels, 1, str(tmp_path / "f"), str(tmp_path / "w"),
                              str(tmp_path / "cf"), str(tmp_path / "cw"), ["cmd"])
    k = out["kernels"]
    assert out["scale"] == {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
    assert k["a.bf16"]["fetch_bytes"] == 10 * 1024 * 2 and k["a.bf16"]["write_bytes"] == 10 * 1024
    assert k["b.bf16"]["fetch_bytes"] == 24 * 1024 * 2       # GEMM and its reduce pass
    assert "splitk_reduce_kernel" in k["b.bf16"]["kernel"]
    assert k["c.bf16"]["bytes_per_launch"] == 2 * 1024 * 3
    assert all(v["dispatches"] == 2 for v in k.values())
    saved = json.load(open(tmp_path / "traffic_toy.json"))
    assert saved["workload"] == "toy" and saved["source_sha"] == bench.kernel_source_sha()
    assert bench.measured_traffic("toy", "b.bf16") == k["b.bf16"]["bytes_per_launch"]
    # a partial step is an error
    for counter, sub in (("FETCH_SIZE", "f2"), ("WRITE_SIZE", "w2")):
        _write_counters(tmp_path / sub, [(k_, counter, v) for k_, v in seq[:-1]])
    with pytest.raises(SystemExit):
        bench.write_traffic("toy2", labels, 1, str(tmp_path / "f2"), str(tmp_path / "w2"),
                            str(tmp_path / "cf"), str(tmp_path / "cw"), [])


def _small(cfg, **kw):
    import dataclasses
    return dataclasses.replace(synth.WORKLOADS[cfg], **kw)


@pytest.mark.parametrize("cfg,dtype", [(2, "bf16"), (4, "bf16"), (5, "e4m3")])
def test_parity_gate_passes_the_oracle_and_catches_a_wrong_tensor(cfg, dtype):
    """bench.py's parity gate on a small shard: device outputs equal to the
    oracle's (rounded to the storage types) pass; one output tensor off by
    10% fails, naming that tensor. Host only: the 'device' outputs are made
    here from the oracle."""
    import numpy as np
    import oracle
    w = _small(cfg, tokens=64, hidden=48, ffn=synth.WORKLOADS[cfg].tp * 32)
    calls = ("fwd", "dgrad", "wgrad")
    inp = synth.make_rank_inputs(w)
    f64 = {k: (None if v is None else oracle.to_f64(v)) for k, v in inp.items()}
    fp8 = dtype == "e4m3"
    extra = {}
    if fp8:
        def deq(v, fmt):
            _, s, s_inv = oracle.current_scale(v, fmt)
            return oracle.dequantize(oracle.quantize(v, fmt, s), fmt, s_inv)
        for k, fmt in (("x", "e4m3"), ("W1", "e4m3"), ("W2", "e4m3"), ("dy", "e5m2")):
            f64[k] = deq(f64[k], fmt)
        extra = {"a_scale": np.float32(64.0), "dH_scale": np.float32(2048.0)}
    ref = bench._mlp_oracle(w, calls, f64["x"], f64["W1"], f64["b1"], f64["W2"], f64["dy"],
                            fp8, extra.get("a_scale"), extra.get("dH_scale"))
    import torch
    bf = lambda v: torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).float().numpy()
    gpu = {k: (None if v is None else (bf(v) if k in ("y", "h", "a", "dH", "dx") else
                                      np.asarray(v, np.float32)))
           for k, v in ref.items()}
    gpu.update(extra)
    base, par = bench.cpu_baseline(w, calls, 0, gpu=gpu)
    assert base is None and par["pass"], par
    assert set(par["max_rel_err"]) >= {"y", "dx", "dW1", "dW2"}
    gpu["dW1"] = gpu["dW1"] * 1.1
    _, par = bench.cpu_baseline(w, calls, 0, gpu=gpu)
    assert not par["pass"] and par["max_rel_err"]["dW1"] > par["tol"]["dW1"]
