"""CPU oracle for one tensor-parallel rank's share of the column->row MLP block.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the GPU
library (``tensor_transformer_mlp_rank_amd``); both draw inputs from the
separate ``synth`` module.

Everything is plain float64 NumPy (SciPy's logistic function for the sigmoid),
written as the definitions stated by the pages:

* the block: a column-parallel fc1 (weight split along its output features),
  a fused bias+GELU or the gated SwiGLU variant, then a row-parallel fc2 that
  yields this rank's partial sum -- Megatron-LM code tour (pyshine.com),
  sections "The Tensor-Parallel Primitives" and "The Transformer Stack";
* the conjugate operators f (identity forward, all-reduce backward) and g
  (all-reduce forward, identity backward) that fix which tensors are
  replicated and which are partial -- "Megatron-LM / Megatron-Core" concept
  note, section "Key math / How it works";
* FP8 (OCP E4M3 for the forward tensors, OCP E5M2 for the gradients;
  per-tensor current or delayed scaling) -- code tour, "Honest Limits";
  concept note, "Key math / How it works";
* the attention projections (``attention``): the packed QKV projection,
  column-parallel, and the row-parallel output projection, split by heads --
  code tour, "The Transformer Stack"; concept note, "Key math / How it
  works";
* the expert MLPs of a mixture-of-experts layer over ragged token groups
  (``moe``) -- onegen.ai overview, "Key Features"; concept note, "Key math /
  How it works".

Where the pages are silent (activation formulas, gated layout, scaling
recipe) the readings are the textbook ones, each stated in the header of the
module that takes it.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle.py``, ``tests/test_oracle_attention.py`` and
``tests/test_oracle_moe.py`` (library
routines, closed forms, finite differences, the shard-sum invariant of the
MLP and of the attention block, brute force, the OCP E4M3 and E5M2 tables).
"""
from .activations import gelu_tanh, gelu_tanh_grad, silu, silu_grad, sigmoid
from .block import (shard_rank, select_features, rank_forward, rank_dgrad, rank_wgrad,
                    unsharded_forward, unsharded_backward, block_loss, to_f64)
from .fp8 import (E4M3_MAX, E5M2_MAX, FMAX, e4m3_decode, e4m3_encode, e5m2_decode, e5m2_encode,
                  current_scale, quantize_e4m3, dequantize_e4m3, quantize, dequantize,
                  delayed_update)
from .fp8_block import rank_forward_fp8, rank_dgrad_fp8, rank_wgrad_fp8
from . import attention
from . import moe

__all__ = [
    "gelu_tanh", "gelu_tanh_grad", "silu", "silu_grad", "sigmoid",
    "shard_rank", "select_features", "rank_forward", "rank_dgrad", "rank_wgrad",
    "unsharded_forward", "unsharded_backward", "block_loss", "to_f64",
    "E4M3_MAX", "E5M2_MAX", "FMAX", "e4m3_decode", "e4m3_encode", "e5m2_decode", "e5m2_encode",
    "quantize", "dequantize", "delayed_update",
    "rank_forward_fp8", "rank_dgrad_fp8", "rank_wgrad_fp8",
    "current_scale", "quantize_e4m3",
    "dequantize_e4m3", "attention", "moe",
]
