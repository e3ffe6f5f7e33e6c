"""Seeded synthetic inputs for the per-rank tensor-parallel MLP block.

This module holds the workload table and the random-number recipe, and
nothing of the block's arithmetic: no GEMM, no activation, no sharding, no
quantisation. Both the CPU oracle (``oracle/``) and the GPU library's callers
(tests, ``bench.py``) draw their inputs from here, so the two sides see the
same bits while sharing no code that computes the block.

Recipe (one rule for every tensor):

* generator ``numpy.random.Generator(PCG64(seed))`` with
  ``seed = 1000 * config_id + tensor_id`` where tensor ids are
  x=1, W1=2, b1=3, W2=4, dy=5, dW_init=6 (initial fp32 gradient buffers for the
  accumulate mode);
* draw standard normals in float32, multiply by the tensor's standard
  deviation in float32;
* for bf16 workloads, cast to ``torch.bfloat16`` with torch's own
  round-to-nearest-even cast (a library routine); fp32 workloads keep the
  float32 values; fp8 workloads keep float32 values and leave the e4m3
  encoding to the code under test (the library's quantiser on the GPU side,
  the oracle's encoder on the CPU side).

The shapes are the per-rank shard shapes of the five workloads: a tiny fp32
GELU block split into two simulated shards, GELU shards at TP=4 and TP=8,
a gated SwiGLU shard at TP=2 and an fp8 GELU shard at TP=8. The block
structure (column-parallel fc1, activation, row-parallel fc2) follows the
Megatron code tour, section "The Transformer Stack".

The attention-projection workloads (``ATTN_WORKLOADS``) use the same rule
with their own tensor ids: x=1, Wqkv=2, bqkv=3, Wo=4, dy=5, dW_init=6,
ctx=7 (the core attention's output, the input of the output projection) and
dqkv=8 (the core attention's input gradient). The per-rank packed weight is
drawn directly at its shard shape [(nq + 2 nkv) hn, H].

The mixture-of-experts workloads (``MOE_WORKLOADS``) draw the per-expert
token counts from a seeded synthetic routing (``moe_counts``): router logits
N(0, 1) per token and expert plus a per-expert offset N(0, 0.5) (so the
experts are unevenly loaded, as trained routers are), each token sent to its
top-k experts; the counts are the histogram of those choices. The grouped
rows themselves (x, dy) are drawn directly at [sum(counts), H] with tensor
ids x=1, W1=2, b1=3, W2=4, dy=5, dW_init=6, routing=9; expert weights are
[E, ...] stacks.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

TENSOR_IDS = {"x": 1, "W1": 2, "b1": 3, "W2": 4, "dy": 5, "dW_init": 6,
              "Wqkv": 2, "bqkv": 3, "Wo": 4, "ctx": 7, "dqkv": 8, "routing": 9}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One per-rank workload: shapes, activation, dtype and value scales."""

    cfg_id: int
    name: str
    tokens: int          # T = micro-batch x sequence length
    batch: int
    seq: int
    hidden: int          # H
    ffn: int             # F, unsharded intermediate size
    tp: int              # tensor-parallel degree
    act: str             # "gelu" or "swiglu"
    dtype: str           # "f32", "bf16" or "e4m3"
    x_std: float
    w1_std: float
    w2_std: float
    b1_std: float | None  # None: no bias; 0.0: bias present and zero
    calls: tuple = ("fwd", "dgrad", "wgrad")

    @property
    def ffn_shard(self) -> int:
        return self.ffn // self.tp

    @property
    def gate_mult(self) -> int:
        """G: 2 for the gated SwiGLU block (gate and up halves), 1 otherwise."""
        return 2 if self.act == "swiglu" else 1

    @property
    def has_bias(self) -> bool:
        return self.b1_std is not None

    def flops(self, tokens: int | None = None, calls=None) -> float:
        """Algorithmic FLOPs of the per-rank GEMMs (epilogues not counted)."""
        t = self.tokens if tokens is None else tokens
        calls = self.calls if calls is None else calls
        per_gemm_pair = 2.0 * t * self.hidden * self.ffn_shard * (self.gate_mult + 1)
        n = 0
        for c in calls:
            n += 1 if c in ("fwd", "dgrad", "wgrad") else 0
        return per_gemm_pair * n


# Standard deviation of fc2 weights at the 8192-hidden shard: 0.02/sqrt(2*80).
_W2_SCALED = 0.02 / math.sqrt(2 * 80)

WORKLOADS = {
    1: Workload(1, "gelu_f32_tiny_tp2", 128, 1, 128, 256, 1024, 2, "gelu", "f32",
                1.0, 0.02, 0.02, 0.0),
    2: Workload(2, "gelu_bf16_h2048_tp4", 8192, 4, 2048, 2048, 8192, 4, "gelu", "bf16",
                1.0, 0.02, 0.02, 0.01),
    3: Workload(3, "gelu_bf16_h8192_tp8", 8192, 4, 2048, 8192, 32768, 8, "gelu", "bf16",
                1.0, 0.02, _W2_SCALED, 0.01),
    4: Workload(4, "swiglu_bf16_h4096_tp2", 8192, 2, 4096, 4096, 14336, 2, "swiglu", "bf16",
                1.0, 0.02, 0.02, None),
    5: Workload(5, "gelu_e4m3_h12288_tp8", 8192, 2, 4096, 12288, 49152, 8, "gelu", "e4m3",
                1.0, 0.02, 0.02, 0.01, calls=("fwd",)),
}


def seed_for(cfg_id: int, tensor: str) -> int:
    return 1000 * cfg_id + TENSOR_IDS[tensor]


def normal_f32(seed: int, shape, std: float) -> np.ndarray:
    """Seeded N(0, std^2) draw in float32 (PCG64)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = rng.standard_normal(size=shape, dtype=np.float32)
    out *= np.float32(std)
    return out


def _cast(arr: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(arr)
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    return t  # f32, and e4m3 workloads keep float32 values for the quantiser


def shard_shapes(w: Workload, tokens: int | None = None, hidden: int | None = None,
                 ffn_shard: int | None = None) -> dict:
    t = w.tokens if tokens is None else tokens
    h = w.hidden if hidden is None else hidden
    fs = w.ffn_shard if ffn_shard is None else ffn_shard
    g = w.gate_mult
    return {"x": (t, h), "W1": (g * fs, h), "b1": (g * fs,), "W2": (h, fs), "dy": (t, h)}


def make_rank_inputs(w: Workload, tokens: int | None = None, hidden: int | None = None,
                     ffn_shard: int | None = None, dtype: str | None = None,
                     seed_base: int | None = None, with_dy: bool = True) -> dict:
    """Per-rank shard inputs on the CPU, drawn directly at shard shape.

    ``tokens``/``hidden``/``ffn_shard`` override the workload's sizes (used for
    small and ragged test shapes with the same value distributions).
    ``seed_base`` replaces ``cfg_id`` in the seed rule.
    Returns torch CPU tensors keyed x, W1, b1 (or None), W2, dy.
    """
    dt = w.dtype if dtype is None else dtype
    cid = w.cfg_id if seed_base is None else seed_base
    shapes = shard_shapes(w, tokens, hidden, ffn_shard)
    out = {
        "x": _cast(normal_f32(seed_for(cid, "x"), shapes["x"], w.x_std), dt),
        "W1": _cast(normal_f32(seed_for(cid, "W1"), shapes["W1"], w.w1_std), dt),
        "W2": _cast(normal_f32(seed_for(cid, "W2"), shapes["W2"], w.w2_std), dt),
        "b1": None,
    }
    if w.has_bias:
        if w.b1_std == 0.0:
            b = np.zeros(shapes["b1"], dtype=np.float32)
        else:
            b = normal_f32(seed_for(cid, "b1"), shapes["b1"], w.b1_std)
        # the bias of an e4m3 workload is carried in bf16
        out["b1"] = _cast(b, "bf16" if dt == "e4m3" else dt)
    if with_dy:
        out["dy"] = _cast(normal_f32(seed_for(cid, "dy"), shapes["dy"], 1.0), dt)
    return out


def make_unsharded_inputs(w: Workload, tokens: int | None = None, hidden: int | None = None,
                          ffn: int | None = None, dtype: str | None = None,
                          seed_base: int | None = None, b1_std: float | None = -1.0) -> dict:
    """Unsharded block inputs (for simulated multi-shard runs on tiny shapes).

    W1 is [G*F, H]; for the gated block rows [0, F) are the gate projection and
    rows [F, 2F) the up projection. ``b1_std=-1`` keeps the workload's bias
    rule; any other value overrides it (``None`` drops the bias).
    """
    dt = w.dtype if dtype is None else dtype
    cid = w.cfg_id if seed_base is None else seed_base
    t = w.tokens if tokens is None else tokens
    h = w.hidden if hidden is None else hidden
    f = w.ffn if ffn is None else ffn
    g = w.gate_mult
    bstd = w.b1_std if b1_std == -1.0 else b1_std
    out = {
        "x": _cast(normal_f32(seed_for(cid, "x"), (t, h), w.x_std), dt),
        "W1": _cast(normal_f32(seed_for(cid, "W1"), (g * f, h), w.w1_std), dt),
        "W2": _cast(normal_f32(seed_for(cid, "W2"), (h, f), w.w2_std), dt),
        "dy": _cast(normal_f32(seed_for(cid, "dy"), (t, h), 1.0), dt),
        "b1": None,
    }
    if bstd is not None:
        b = (np.zeros((g * f,), np.float32) if bstd == 0.0
             else normal_f32(seed_for(cid, "b1"), (g * f,), bstd))
        out["b1"] = _cast(b, dt)
    return out


def grad_init(cfg_id: int, shape, salt: int = 0) -> torch.Tensor:
    """Seeded nonzero fp32 buffer used as the prior content of a gradient
    accumulator when testing the accumulate mode."""
    return torch.from_numpy(normal_f32(seed_for(cfg_id, "dW_init") + 7919 * salt, shape, 1e-3))


# ---------------------------------------------------------------- attention projections
@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    """One rank's share of the attention block's projections."""

    cfg_id: int
    name: str
    tokens: int          # T = micro-batch x sequence length
    batch: int
    seq: int
    hidden: int          # H
    heads: int           # query heads, unsharded
    kv_heads: int        # key/value heads, unsharded (= heads without grouped queries)
    head_dim: int        # hn
    tp: int
    dtype: str           # "f32" or "bf16"
    x_std: float
    w_std: float
    b_std: float | None  # None: no QKV bias

    @property
    def q_heads_rank(self) -> int:
        return self.heads // self.tp

    @property
    def kv_heads_rank(self) -> int:
        return self.kv_heads // self.tp

    @property
    def nqkv(self) -> int:
        return (self.q_heads_rank + 2 * self.kv_heads_rank) * self.head_dim

    @property
    def d(self) -> int:
        return self.q_heads_rank * self.head_dim

    def flops(self, tokens: int | None = None) -> float:
        """Algorithmic FLOPs of the two projections forward + backward (six GEMMs)."""
        t = self.tokens if tokens is None else tokens
        return 3 * 2.0 * t * self.hidden * (self.nqkv + self.d)


ATTN_WORKLOADS = {
    # the pages' example model (hidden 1024, 16 heads, TP 2, micro-batch 2 x seq 2048)
    6: AttnWorkload(6, "attn_bf16_h1024_tp2", 4096, 2, 2048, 1024, 16, 16, 64, 2, "bf16",
                    1.0, 0.02, 0.01),
    # the 8192-hidden shard of the MLP workloads' model: 64 heads of 128, TP 8
    7: AttnWorkload(7, "attn_bf16_h8192_tp8", 8192, 4, 2048, 8192, 64, 64, 128, 8, "bf16",
                    1.0, 0.02, 0.01),
}


def make_attn_inputs(w: AttnWorkload, tokens: int | None = None, hidden: int | None = None,
                     q_heads: int | None = None, kv_heads: int | None = None,
                     head_dim: int | None = None, dtype: str | None = None,
                     seed_base: int | None = None) -> dict:
    """Per-rank inputs of the two projections on the CPU: x, Wqkv, bqkv (or
    None), Wo, dy, ctx, dqkv. Sizes override the workload's per-rank ones."""
    dt = w.dtype if dtype is None else dtype
    cid = w.cfg_id if seed_base is None else seed_base
    t = w.tokens if tokens is None else tokens
    h = w.hidden if hidden is None else hidden
    nq = w.q_heads_rank if q_heads is None else q_heads
    nkv = w.kv_heads_rank if kv_heads is None else kv_heads
    hn = w.head_dim if head_dim is None else head_dim
    nqkv, d = (nq + 2 * nkv) * hn, nq * hn
    out = {
        "x": _cast(normal_f32(seed_for(cid, "x"), (t, h), w.x_std), dt),
        "Wqkv": _cast(normal_f32(seed_for(cid, "Wqkv"), (nqkv, h), w.w_std), dt),
        "Wo": _cast(normal_f32(seed_for(cid, "Wo"), (h, d), w.w_std), dt),
        "dy": _cast(normal_f32(seed_for(cid, "dy"), (t, h), 1.0), dt),
        "ctx": _cast(normal_f32(seed_for(cid, "ctx"), (t, d), 1.0), dt),
        "dqkv": _cast(normal_f32(seed_for(cid, "dqkv"), (t, nqkv), 1.0), dt),
        "bqkv": None,
    }
    if w.b_std is not None:
        out["bqkv"] = _cast(normal_f32(seed_for(cid, "bqkv"), (nqkv,), w.b_std), dt)
    return out


# ---------------------------------------------------------------- mixture of experts
@dataclasses.dataclass(frozen=True)
class MoeWorkload:
    """One rank's local experts of a mixture-of-experts layer."""

    cfg_id: int
    name: str
    tokens: int          # tokens entering the layer (batch x sequence)
    batch: int
    seq: int
    hidden: int          # H
    experts: int         # local experts E
    topk: int            # experts per token
    ffn_shard: int       # Fs per expert (its expert-tensor-parallel share)
    act: str             # "gelu" or "swiglu"
    dtype: str
    x_std: float
    w_std: float
    b1_std: float | None

    @property
    def gate_mult(self) -> int:
        return 2 if self.act == "swiglu" else 1

    @property
    def has_bias(self) -> bool:
        return self.b1_std is not None

    def flops(self, rows: int) -> float:
        """Algorithmic FLOPs of forward + backward over `rows` routed rows."""
        return 3 * 2.0 * rows * self.hidden * self.ffn_shard * (self.gate_mult + 1)


MOE_WORKLOADS = {
    # Mixtral-style: 8 experts, top-2, SwiGLU, hidden 4096, expert ffn 14336 (all local)
    8: MoeWorkload(8, "moe_swiglu_bf16_h4096_e8", 4096, 1, 4096, 4096, 8, 2, 14336, "swiglu",
                   "bf16", 1.0, 0.02, None),
    # fine-grained: 64 experts, top-6, GELU with bias, hidden 2048, expert ffn 1408
    9: MoeWorkload(9, "moe_gelu_bf16_h2048_e64", 4096, 1, 4096, 2048, 64, 6, 1408, "gelu",
                   "bf16", 1.0, 0.02, 0.01),
}


def moe_counts(w: MoeWorkload, tokens: int | None = None, seed_base: int | None = None) -> np.ndarray:
    """Rows per local expert (int32 [E]) from a seeded synthetic top-k routing."""
    t = w.tokens if tokens is None else tokens
    cid = w.cfg_id if seed_base is None else seed_base
    rng = np.random.Generator(np.random.PCG64(seed_for(cid, "routing")))
    bias = rng.standard_normal(w.experts).astype(np.float32) * np.float32(0.5)
    logits = rng.standard_normal((t, w.experts), dtype=np.float32) + bias
    top = np.argpartition(-logits, w.topk - 1, axis=1)[:, :w.topk]
    return np.bincount(top.reshape(-1), minlength=w.experts).astype(np.int32)


def make_moe_inputs(w: MoeWorkload, counts, hidden: int | None = None,
                    ffn_shard: int | None = None, experts: int | None = None,
                    dtype: str | None = None, seed_base: int | None = None) -> dict:
    """Grouped rows and expert stacks on the CPU: x, dy [sum(counts), H];
    W1 [E, G*Fs, H], b1 [E, G*Fs] or None, W2 [E, H, Fs]; counts (int32)."""
    dt = w.dtype if dtype is None else dtype
    cid = w.cfg_id if seed_base is None else seed_base
    h = w.hidden if hidden is None else hidden
    fs = w.ffn_shard if ffn_shard is None else ffn_shard
    e = w.experts if experts is None else experts
    rows = int(np.sum(counts))
    g = w.gate_mult
    out = {
        "counts": torch.from_numpy(np.asarray(counts, dtype=np.int32)),
        "x": _cast(normal_f32(seed_for(cid, "x"), (rows, h), w.x_std), dt),
        "W1": _cast(normal_f32(seed_for(cid, "W1"), (e, g * fs, h), w.w_std), dt),
        "W2": _cast(normal_f32(seed_for(cid, "W2"), (e, h, fs), w.w_std), dt),
        "dy": _cast(normal_f32(seed_for(cid, "dy"), (rows, h), 1.0), dt),
        "b1": None,
    }
    if w.has_bias:
        out["b1"] = _cast(normal_f32(seed_for(cid, "b1"), (e, g * fs), w.b1_std), dt)
    return out
