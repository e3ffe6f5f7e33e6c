"""Seeded sweep of random shapes through the C ABI, each compared with the
oracle element by element: sizes drawn at random (any T; H and Fs multiples
of 16) reach combinations of ragged tile edges, odd and even stage counts,
zero stages, split-K plans and accumulation that the fixed cases do not list
one by one. The draws are fixed by the seed, so a failure names its case."""
import numpy as np
import pytest
import torch

import synth
from _gpu_helpers import check, gpu_block, oracle_block, require_gpu, say

pytestmark = pytest.mark.gpu

ALL = ("y", "h", "a", "dH", "dx", "dW1", "db1", "dW2")


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 1400))]))
        H = 16 * int(rng.integers(1, 96))
        Fs = 16 * int(rng.integers(1, 72))
        act = "swiglu" if rng.random() < 0.5 else "gelu"
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        acc = bool(rng.random() < 0.5)
        out.append((i, T, H, Fs, act, dtype, acc))
    return out


@pytest.fixture(scope="module")
def tp():
    require_gpu()
    import tensor_transformer_mlp_rank_amd as m
    return m


@pytest.mark.parametrize("i,T,H,Fs,act,dtype,acc", _cases(24, 2026))
def test_random_shapes(tp, i, T, H, Fs, act, dtype, acc):
    w = synth.WORKLOADS[4 if act == "swiglu" else 2]
    inp = synth.make_rank_inputs(w, tokens=T, hidden=H, ffn_shard=Fs, dtype=dtype,
                                 seed_base=700 + i)
    has_bias = act == "gelu"
    G = 2 if act == "swiglu" else 1
    prior = None
    if acc:
        prior = {"dW1": synth.grad_init(700 + i, (G * Fs, H), 1),
                 "db1": synth.grad_init(700 + i, (G * Fs,), 2) if has_bias else None,
                 "dW2": synth.grad_init(700 + i, (H, Fs), 3)}
    say(f"  case {i}: T={T} H={H} Fs={Fs} {act} {dtype} accumulate={acc}")
    gpu = gpu_block(tp, inp, act, dtype, has_bias, accumulate_into=prior)
    ref = oracle_block(inp, act, has_bias, prior=prior)
    check(gpu, ref, dtype, ALL)
    torch.cuda.empty_cache()


def _fp8_cases(n, seed):
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(1, 900)), 16 * int(rng.integers(1, 80)),
             16 * int(rng.integers(1, 56)), "swiglu" if rng.random() < 0.5 else "gelu",
             bool(rng.random() < 0.5)) for i in range(n)]


@pytest.mark.parametrize("i,T,H,Fs,act,acc", _fp8_cases(8, 2027))
def test_random_shapes_e4m3(tp, i, T, H, Fs, act, acc):
    """The E4M3 block's checks (codes as valid roundings, products of the
    device's codes within the bound of their differences, both weight
    gradient forms, the recomputing one) at random shapes."""
    from test_gpu_fp8_bwd import _fp8_block
    say(f"  e4m3 case {i}: T={T} H={H} Fs={Fs} {act} accumulate={acc}")
    _fp8_block(tp, T, H, Fs, seed=800 + i, prior=acc, act=act)
    torch.cuda.empty_cache()
