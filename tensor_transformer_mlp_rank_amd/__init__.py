"""Python binding of libtpmlp: one tensor-parallel rank's share of the
column->row MLP block (fc1 column-parallel, bias+GELU or SwiGLU, fc2
row-parallel partial sum), forward and backward, on MI355X.

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the block runs in the library's HIP kernels
(``libtpmlp.so``, built in-tree by ``build.py``). If the library is missing
this module raises on import -- there is no fallback path.

The C entry points keep their names here (``tpmlp_fwd``, ``tpmlp_bwd_dgrad``,
``tpmlp_bwd_wgrad``, ``tpmlp_quantize_e4m3``, ``tpmlp_quantize_e5m2``, and the
attention projections ``tpmlp_attn_*`` and the expert MLPs ``tpmlp_moe_*``) and
take preallocated output
tensors; ``fwd``, ``bwd_dgrad``, ``bwd_wgrad`` and ``attn_*`` are
conveniences that allocate the outputs with torch and call them. Layouts are
those of ``include/tpmlp.h``.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtpmlp.so")

F32, BF16, E4M3 = 0, 1, 2
GELU, SWIGLU = 0, 1
CALL_FWD, CALL_DGRAD, CALL_WGRAD, CALL_WGRAD_RECOMPUTE = 0, 1, 2, 3

STATUS = {0: "OK", 1: "E_NULL", 2: "E_SHAPE", 3: "E_DTYPE", 4: "E_ALIGN", 5: "E_UNSUPPORTED",
          6: "E_WORKSPACE", 7: "E_HIP", 8: "E_SCRATCH"}

_DTYPE_CODES = {"f32": F32, "bf16": BF16, "e4m3": E4M3}
_ACT_CODES = {"gelu": GELU, "swiglu": SWIGLU}
_TORCH = {F32: torch.float32, BF16: torch.bfloat16, E4M3: torch.uint8}


class Desc(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("ffn_shard", ctypes.c_int64), ("act", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("has_bias", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("has_bias", ctypes.c_int32), ("reserved", ctypes.c_int32)]

    @property
    def nqkv(self) -> int:
        return (self.q_heads + 2 * self.kv_heads) * self.head_dim

    @property
    def d(self) -> int:
        return self.q_heads * self.head_dim


class MoeDesc(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("ffn_shard", ctypes.c_int64), ("experts", ctypes.c_int32),
                ("act", ctypes.c_int32), ("dtype", ctypes.c_int32), ("has_bias", ctypes.c_int32),
                ("reserved0", ctypes.c_int32), ("reserved1", ctypes.c_int32)]


class Fp8History(ctypes.Structure):
    _fields_ = [("amax_history", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("scale_inv", ctypes.c_void_p), ("len", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class Fp8Scales(ctypes.Structure):
    _fields_ = [("x_scale_inv", ctypes.c_void_p), ("w1_scale_inv", ctypes.c_void_p),
                ("w2_scale_inv", ctypes.c_void_p), ("a_amax", ctypes.c_void_p),
                ("a_scale_inv", ctypes.c_void_p), ("a_history", ctypes.POINTER(Fp8History)),
                ("dy_scale_inv", ctypes.c_void_p), ("dH_history", ctypes.POINTER(Fp8History)),
                ("dH_scale_inv", ctypes.c_void_p)]


class DelayedScaling:
    """Device state of one tensor under delayed scaling (tpmlp_fp8_history):
    an amax history of ``length`` floats (newest first), the scale the next
    call quantises with and the 1/scale of the last call."""

    def __init__(self, length: int, device="cuda", scale: float = 1.0):
        self.amax_history = torch.zeros(length, dtype=torch.float32, device=device)
        self.scale = torch.full((1,), float(scale), dtype=torch.float32, device=device)
        self.scale_inv = torch.zeros(1, dtype=torch.float32, device=device)
        self.struct = Fp8History(_ptr(self.amax_history), _ptr(self.scale), _ptr(self.scale_inv),
                                 int(length), 0)


def fp8_scales(x_scale_inv=None, w1_scale_inv=None, w2_scale_inv=None, a_amax=None,
               a_scale_inv=None, a_history: DelayedScaling | None = None, dy_scale_inv=None,
               dH_history: DelayedScaling | None = None, dH_scale_inv=None) -> Fp8Scales:
    """tpmlp_fp8_scales from one-element float32 device tensors (None: NULL)."""
    sc = Fp8Scales(_ptr(x_scale_inv), _ptr(w1_scale_inv), _ptr(w2_scale_inv), _ptr(a_amax),
                   _ptr(a_scale_inv), None if a_history is None else ctypes.pointer(a_history.struct),
                   _ptr(dy_scale_inv),
                   None if dH_history is None else ctypes.pointer(dH_history.struct),
                   _ptr(dH_scale_inv))
    # the struct holds raw device pointers: keep the tensors they point into
    # alive as long as the struct (a freed scale tensor's memory would be
    # handed to the next allocation and the call would read that instead)
    sc._keep = (x_scale_inv, w1_scale_inv, w2_scale_inv, a_amax, a_scale_inv, a_history,
                dy_scale_inv, dH_history, dH_scale_inv)
    return sc


class TpmlpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)} ({lib.tpmlp_strerror(status).decode()})"
        if status == 7:
            msg += f": {lib.tpmlp_last_hip_error().decode()}"
        super().__init__(msg)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(or python tensor_transformer_mlp_rank_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pdesc = ctypes.POINTER(Desc)
    L.tpmlp_fwd.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(Fp8Scales), vp, sz, vp]
    psc = ctypes.POINTER(Fp8Scales)
    L.tpmlp_bwd_dgrad.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, psc, vp, sz, vp]
    L.tpmlp_bwd_wgrad.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, vp, i32, psc, vp, sz, vp]
    L.tpmlp_bwd_wgrad_noalloc.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, vp, i32, psc, vp]
    L.tpmlp_bwd_wgrad_recompute.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, vp, i32, psc, vp, sz,
                                            vp]
    L.tpmlp_bwd_wgrad_t.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, vp, i32, psc, vp]
    L.tpmlp_transpose_u8.argtypes = [vp, i64, i64, vp, vp]
    L.tpmlp_quantize_e4m3.argtypes = [i32, vp, i64, vp, vp, vp, vp, sz, vp]
    L.tpmlp_quantize_e5m2.argtypes = [i32, vp, i64, vp, vp, vp, vp, sz, vp]
    L.tpmlp_quantize_workspace_size.argtypes = [i64]
    L.tpmlp_quantize_workspace_size.restype = sz
    L.tpmlp_workspace_size.argtypes = [pdesc, i32]
    L.tpmlp_workspace_size.restype = sz
    pa = ctypes.POINTER(AttnDesc)
    L.tpmlp_attn_qkv_fwd.argtypes = [pa, vp, vp, vp, vp, vp]
    L.tpmlp_attn_out_fwd.argtypes = [pa, vp, vp, vp, vp]
    L.tpmlp_attn_out_bwd_dgrad.argtypes = [pa, vp, vp, vp, vp, sz, vp]
    L.tpmlp_attn_out_bwd_wgrad.argtypes = [pa, vp, vp, vp, i32, vp, sz, vp]
    L.tpmlp_attn_qkv_bwd_dgrad.argtypes = [pa, vp, vp, vp, vp]
    L.tpmlp_attn_qkv_bwd_wgrad.argtypes = [pa, vp, vp, vp, vp, i32, vp, sz, vp]
    L.tpmlp_attn_workspace_size.argtypes = [pa]
    L.tpmlp_attn_workspace_size.restype = sz
    pm = ctypes.POINTER(MoeDesc)
    L.tpmlp_moe_fwd.argtypes = [pm, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.tpmlp_moe_bwd_dgrad.argtypes = [pm, vp, vp, vp, vp, vp, vp, vp, vp]
    L.tpmlp_moe_bwd_wgrad.argtypes = [pm, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    L.tpmlp_moe_workspace_size.argtypes = [pm]
    L.tpmlp_moe_workspace_size.restype = sz
    for f in ("tpmlp_fwd", "tpmlp_bwd_dgrad", "tpmlp_bwd_wgrad", "tpmlp_bwd_wgrad_noalloc",
              "tpmlp_bwd_wgrad_recompute", "tpmlp_bwd_wgrad_t", "tpmlp_transpose_u8",
              "tpmlp_quantize_e4m3",
              "tpmlp_quantize_e5m2", "tpmlp_timing_enable", "tpmlp_attn_qkv_fwd",
              "tpmlp_attn_out_fwd", "tpmlp_attn_out_bwd_dgrad", "tpmlp_attn_out_bwd_wgrad",
              "tpmlp_attn_qkv_bwd_dgrad", "tpmlp_attn_qkv_bwd_wgrad", "tpmlp_moe_fwd",
              "tpmlp_moe_bwd_dgrad", "tpmlp_moe_bwd_wgrad"):
        getattr(L, f).restype = i32
    L.tpmlp_strerror.argtypes = [i32]
    L.tpmlp_strerror.restype = ctypes.c_char_p
    L.tpmlp_last_hip_error.restype = ctypes.c_char_p
    L.tpmlp_abi_version.restype = i32
    L.tpmlp_timing_enable.argtypes = [i32, ctypes.c_char_p]
    L.tpmlp_timing_collect.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(i64),
                                       ctypes.POINTER(ctypes.c_double), i32]
    L.tpmlp_timing_collect.restype = i32
    L.tpmlp_timing_clock_mhz.argtypes = [ctypes.c_char_p]
    L.tpmlp_timing_clock_mhz.restype = ctypes.c_double
    return L


lib = _load()


# ------------------------------------------------------------------ marshalling
def make_desc(tokens: int, hidden: int, ffn_shard: int, act="gelu", dtype="bf16",
              has_bias: bool = True) -> Desc:
    a = _ACT_CODES[act] if isinstance(act, str) else int(act)
    d = _DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)
    return Desc(int(tokens), int(hidden), int(ffn_shard), a, d, int(bool(has_bias)), 0)


def make_attn_desc(tokens: int, hidden: int, q_heads: int, kv_heads: int, head_dim: int,
                   dtype="bf16", has_bias: bool = True) -> AttnDesc:
    d = _DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)
    return AttnDesc(int(tokens), int(hidden), int(q_heads), int(kv_heads), int(head_dim), d,
                    int(bool(has_bias)), 0)


def make_moe_desc(tokens: int, hidden: int, ffn_shard: int, experts: int, act="gelu",
                  dtype="bf16", has_bias: bool = True) -> MoeDesc:
    a = _ACT_CODES[act] if isinstance(act, str) else int(act)
    d = _DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)
    return MoeDesc(int(tokens), int(hidden), int(ffn_shard), int(experts), a, d,
                   int(bool(has_bias)), 0, 0)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensors passed to libtpmlp must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libtpmlp must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, where: str):
    if status != 0:
        raise TpmlpError(status, where)


def workspace_size(desc: Desc, call: int) -> int:
    return int(lib.tpmlp_workspace_size(ctypes.byref(desc), call))


def tpmlp_fwd(desc, x, W1, b1, W2, y, h, a, fp8=None, workspace=None, stream=None):
    ws = _ptr(workspace)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sc = None if fp8 is None else ctypes.byref(fp8)
    _check(lib.tpmlp_fwd(ctypes.byref(desc), _ptr(x), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(y),
                         _ptr(h), _ptr(a), sc, ws, nbytes, _stream(stream)), "tpmlp_fwd")


def tpmlp_bwd_dgrad(desc, dy, W1, W2, h, dH, dx, fp8=None, workspace=None, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sc = None if fp8 is None else ctypes.byref(fp8)
    _check(lib.tpmlp_bwd_dgrad(ctypes.byref(desc), _ptr(dy), _ptr(W1), _ptr(W2), _ptr(h),
                               _ptr(dH), _ptr(dx), sc, _ptr(workspace), nbytes, _stream(stream)),
           "tpmlp_bwd_dgrad")


def tpmlp_bwd_wgrad(desc, dy, x, a, dH, dW1, db1, dW2, accumulate=False, fp8=None,
                    workspace=None, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sc = None if fp8 is None else ctypes.byref(fp8)
    _check(lib.tpmlp_bwd_wgrad(ctypes.byref(desc), _ptr(dy), _ptr(x), _ptr(a), _ptr(dH),
                               _ptr(dW1), _ptr(db1), _ptr(dW2), int(bool(accumulate)), sc,
                               _ptr(workspace), nbytes, _stream(stream)), "tpmlp_bwd_wgrad")


def tpmlp_bwd_wgrad_recompute(desc, dy, x, h, dH, dW1, db1, dW2, accumulate=False, fp8=None,
                              workspace=None, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sc = None if fp8 is None else ctypes.byref(fp8)
    _check(lib.tpmlp_bwd_wgrad_recompute(ctypes.byref(desc), _ptr(dy), _ptr(x), _ptr(h),
                                         _ptr(dH), _ptr(dW1), _ptr(db1), _ptr(dW2),
                                         int(bool(accumulate)), sc, _ptr(workspace), nbytes,
                                         _stream(stream)), "tpmlp_bwd_wgrad_recompute")


def tpmlp_bwd_wgrad_noalloc(desc, dy, x, a, dH, dW1, db1, dW2, accumulate=False, fp8=None,
                            stream=None):
    sc = None if fp8 is None else ctypes.byref(fp8)
    _check(lib.tpmlp_bwd_wgrad_noalloc(ctypes.byref(desc), _ptr(dy), _ptr(x), _ptr(a), _ptr(dH),
                                       _ptr(dW1), _ptr(db1), _ptr(dW2), int(bool(accumulate)), sc,
                                       _stream(stream)), "tpmlp_bwd_wgrad_noalloc")


def tpmlp_bwd_wgrad_t(desc, dy_t, x_t, a_t, dH_t, dW1, db1, dW2, accumulate=False, fp8=None,
                      stream=None):
    sc = None if fp8 is None else ctypes.byref(fp8)
    _check(lib.tpmlp_bwd_wgrad_t(ctypes.byref(desc), _ptr(dy_t), _ptr(x_t), _ptr(a_t),
                                 _ptr(dH_t), _ptr(dW1), _ptr(db1), _ptr(dW2),
                                 int(bool(accumulate)), sc, _stream(stream)), "tpmlp_bwd_wgrad_t")


def tpmlp_transpose_u8(src, rows, cols, dst, stream=None):
    _check(lib.tpmlp_transpose_u8(_ptr(src), rows, cols, _ptr(dst), _stream(stream)),
           "tpmlp_transpose_u8")


SCRATCH_BYTES = 8 << 20  # TPMLP_SCRATCH_BYTES


def _quantize(fn, name, src, dst, amax, scale_inv, workspace, stream):
    dt = BF16 if src.dtype == torch.bfloat16 else F32 if src.dtype == torch.float32 else -1
    nbytes = workspace.numel() * workspace.element_size()
    _check(fn(dt, _ptr(src), src.numel(), _ptr(dst), _ptr(amax), _ptr(scale_inv),
              _ptr(workspace), nbytes, _stream(stream)), name)


def tpmlp_quantize_e4m3(src, dst, amax, scale_inv, workspace, stream=None):
    _quantize(lib.tpmlp_quantize_e4m3, "tpmlp_quantize_e4m3", src, dst, amax, scale_inv,
              workspace, stream)


def tpmlp_quantize_e5m2(src, dst, amax, scale_inv, workspace, stream=None):
    _quantize(lib.tpmlp_quantize_e5m2, "tpmlp_quantize_e5m2", src, dst, amax, scale_inv,
              workspace, stream)


# ------------------------------------------------------------------ conveniences
def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


def fwd(desc, x, W1, b1, W2, save_h=True, fp8_in_scales=None, a_history=None, stream=None):
    """Run the forward; returns dict y, h (or None), a, and for E4M3 a_amax,
    a_scale_inv. ``fp8_in_scales`` = (x_scale_inv, w1_scale_inv, w2_scale_inv)
    one-element fp32 device tensors. With ``a_history`` (DelayedScaling), a
    is quantised with delayed scaling and a_scale_inv is the history's."""
    dev = x.device
    T, H, Fs = desc.tokens, desc.hidden, desc.ffn_shard
    G = 2 if desc.act == SWIGLU else 1
    act_t = torch.bfloat16 if desc.dtype in (BF16, E4M3) else torch.float32
    out = {"y": _empty((T, H), act_t, dev),
           "h": _empty((T, G * Fs), act_t, dev) if save_h else None,
           "a": _empty((T, Fs), torch.uint8 if desc.dtype == E4M3 else act_t, dev)}
    sc = None
    if desc.dtype == E4M3:
        xs, w1s, w2s = fp8_in_scales
        if a_history is None:
            out["a_amax"] = torch.zeros(1, dtype=torch.float32, device=dev)
            out["a_scale_inv"] = torch.zeros(1, dtype=torch.float32, device=dev)
            sc = fp8_scales(xs, w1s, w2s, out["a_amax"], out["a_scale_inv"])
        else:
            out["a_scale_inv"] = a_history.scale_inv
            sc = fp8_scales(xs, w1s, w2s, a_history=a_history)
    n = workspace_size(desc, CALL_FWD)
    ws = _empty((max(n, 1),), torch.uint8, dev) if n else None
    tpmlp_fwd(desc, x, W1, b1, W2, out["y"], out["h"], out["a"], sc, ws, stream)
    return out


def bwd_dgrad(desc, dy, W1, W2, h, fp8=None, stream=None):
    """dH and dx_partial. For E4M3, ``fp8`` = dict dy_scale_inv, w1_scale_inv,
    w2_scale_inv (device tensors) and dH_history (DelayedScaling); dH is
    E5M2 codes and dx_partial bfloat16."""
    dev = dy.device
    T, H, Fs = desc.tokens, desc.hidden, desc.ffn_shard
    G = 2 if desc.act == SWIGLU else 1
    t = _TORCH[desc.dtype]
    out = {"dH": _empty((T, G * Fs), t, dev),
           "dx": _empty((T, H), torch.bfloat16 if desc.dtype == E4M3 else t, dev)}
    sc = None if fp8 is None else fp8_scales(**fp8)
    n = workspace_size(desc, CALL_DGRAD)
    ws = _empty((n,), torch.uint8, dev) if n else None
    tpmlp_bwd_dgrad(desc, dy, W1, W2, h, out["dH"], out["dx"], sc, ws, stream)
    return out


def bwd_wgrad(desc, dy, x, a, dH, accumulate_into=None, fp8=None, stream=None, recompute=False):
    """fp32 weight gradients. ``accumulate_into`` = dict dW1, db1, dW2 of
    existing fp32 buffers to add into (accumulate mode). For E4M3, ``fp8`` =
    dict dy_scale_inv, x_scale_inv, a_scale_inv, dH_scale_inv. With
    ``recompute``, ``a`` is the saved pre-activation h and the call recomputes
    the activation from it (tpmlp_bwd_wgrad_recompute)."""
    dev = dy.device
    H, Fs = desc.hidden, desc.ffn_shard
    G = 2 if desc.act == SWIGLU else 1
    if accumulate_into is not None:
        out = accumulate_into
    else:
        out = {"dW1": _empty((G * Fs, H), torch.float32, dev),
               "db1": _empty((G * Fs,), torch.float32, dev) if desc.has_bias else None,
               "dW2": _empty((H, Fs), torch.float32, dev)}
    n = workspace_size(desc, CALL_WGRAD_RECOMPUTE if recompute else CALL_WGRAD)
    ws = _empty((n,), torch.uint8, dev) if n else None
    sc = None if fp8 is None else fp8_scales(**fp8)
    call = tpmlp_bwd_wgrad_recompute if recompute else tpmlp_bwd_wgrad
    call(desc, dy, x, a, dH, out["dW1"], out.get("db1"), out["dW2"],
         accumulate=accumulate_into is not None, fp8=sc, workspace=ws, stream=stream)
    return out


def token_ld(T):
    """Row length of the token-contiguous layout: T rounded up to 16."""
    return (T + 15) // 16 * 16


def transpose_u8(src, stream=None):
    """The token-contiguous copy [cols, token_ld(rows)] of a [rows, cols]
    uint8 tensor of FP8 codes (tpmlp_transpose_u8)."""
    rows, cols = src.shape
    dst = _empty((cols, token_ld(rows)), torch.uint8, src.device)
    tpmlp_transpose_u8(src, rows, cols, dst, stream)
    return dst


def bwd_wgrad_t(desc, dy_t, x_t, a_t, dH_t, accumulate_into=None, fp8=None, stream=None):
    """bwd_wgrad for E4M3 from token-contiguous operands (tpmlp_bwd_wgrad_t)."""
    dev = dy_t.device
    H, Fs = desc.hidden, desc.ffn_shard
    G = 2 if desc.act == SWIGLU else 1
    if accumulate_into is not None:
        out = accumulate_into
    else:
        out = {"dW1": _empty((G * Fs, H), torch.float32, dev),
               "db1": _empty((G * Fs,), torch.float32, dev) if desc.has_bias else None,
               "dW2": _empty((H, Fs), torch.float32, dev)}
    sc = None if fp8 is None else fp8_scales(**fp8)
    tpmlp_bwd_wgrad_t(desc, dy_t, x_t, a_t, dH_t, out["dW1"], out.get("db1"), out["dW2"],
                      accumulate=accumulate_into is not None, fp8=sc, stream=stream)
    return out


def quantize_e4m3(src, stream=None, e5m2=False):
    """E4M3 (or E5M2) codes (uint8, same shape) plus one-element amax and
    scale_inv, per-tensor current scaling."""
    dev = src.device
    dst = _empty(src.shape, torch.uint8, dev)
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    sinv = torch.zeros(1, dtype=torch.float32, device=dev)
    n = int(lib.tpmlp_quantize_workspace_size(src.numel()))
    ws = _empty((max(n, 256),), torch.uint8, dev)
    (tpmlp_quantize_e5m2 if e5m2 else tpmlp_quantize_e4m3)(src, dst, amax, sinv, ws, stream)
    return dst, amax, sinv


def quantize_e5m2(src, stream=None):
    return quantize_e4m3(src, stream, e5m2=True)


# ------------------------------------------------------------------ timing
# ------------------------------------------------------------------ attention projections
def attn_workspace_size(desc: AttnDesc) -> int:
    return int(lib.tpmlp_attn_workspace_size(ctypes.byref(desc)))


def tpmlp_attn_qkv_fwd(desc, x, Wqkv, bqkv, qkv, stream=None):
    _check(lib.tpmlp_attn_qkv_fwd(ctypes.byref(desc), _ptr(x), _ptr(Wqkv), _ptr(bqkv), _ptr(qkv),
                                  _stream(stream)), "tpmlp_attn_qkv_fwd")


def tpmlp_attn_out_fwd(desc, ctx, Wo, y, stream=None):
    _check(lib.tpmlp_attn_out_fwd(ctypes.byref(desc), _ptr(ctx), _ptr(Wo), _ptr(y),
                                  _stream(stream)), "tpmlp_attn_out_fwd")


def _nbytes(workspace):
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def tpmlp_attn_out_bwd_dgrad(desc, dy, Wo, dctx, workspace=None, stream=None):
    _check(lib.tpmlp_attn_out_bwd_dgrad(ctypes.byref(desc), _ptr(dy), _ptr(Wo), _ptr(dctx),
                                        _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "tpmlp_attn_out_bwd_dgrad")


def tpmlp_attn_out_bwd_wgrad(desc, dy, ctx, dWo, accumulate=False, workspace=None, stream=None):
    _check(lib.tpmlp_attn_out_bwd_wgrad(ctypes.byref(desc), _ptr(dy), _ptr(ctx), _ptr(dWo),
                                        int(bool(accumulate)), _ptr(workspace),
                                        _nbytes(workspace), _stream(stream)),
           "tpmlp_attn_out_bwd_wgrad")


def tpmlp_attn_qkv_bwd_dgrad(desc, dqkv, Wqkv, dx, stream=None):
    _check(lib.tpmlp_attn_qkv_bwd_dgrad(ctypes.byref(desc), _ptr(dqkv), _ptr(Wqkv), _ptr(dx),
                                        _stream(stream)), "tpmlp_attn_qkv_bwd_dgrad")


def tpmlp_attn_qkv_bwd_wgrad(desc, dqkv, x, dWqkv, dbqkv, accumulate=False, workspace=None,
                             stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.tpmlp_attn_qkv_bwd_wgrad(ctypes.byref(desc), _ptr(dqkv), _ptr(x), _ptr(dWqkv),
                                        _ptr(dbqkv), int(bool(accumulate)), _ptr(workspace),
                                        nbytes, _stream(stream)), "tpmlp_attn_qkv_bwd_wgrad")


def _act_t(desc):
    return torch.float32 if desc.dtype == F32 else torch.bfloat16


def attn_qkv_fwd(desc, x, Wqkv, bqkv=None, stream=None):
    """Packed projection; returns (qkv, q, k, v), q/k/v column views of qkv."""
    qkv = _empty((desc.tokens, desc.nqkv), _act_t(desc), x.device)
    tpmlp_attn_qkv_fwd(desc, x, Wqkv, bqkv, qkv, stream)
    a, b = desc.d, desc.d + desc.kv_heads * desc.head_dim
    return qkv, qkv[:, :a], qkv[:, a:b], qkv[:, b:]


def attn_out_fwd(desc, ctx, Wo, stream=None):
    y = _empty((desc.tokens, desc.hidden), _act_t(desc), ctx.device)
    tpmlp_attn_out_fwd(desc, ctx, Wo, y, stream)
    return y


def _attn_ws(desc, device):
    n = attn_workspace_size(desc)
    return _empty((n,), torch.uint8, device) if n else None


def attn_out_bwd(desc, dy, Wo, ctx, dWo=None, stream=None):
    """(dctx, dWo); with a given dWo the gradient is added into it."""
    dctx = _empty((desc.tokens, desc.d), _act_t(desc), dy.device)
    ws = _attn_ws(desc, dy.device)
    tpmlp_attn_out_bwd_dgrad(desc, dy, Wo, dctx, ws, stream)
    acc = dWo is not None
    if not acc:
        dWo = _empty((desc.hidden, desc.d), torch.float32, dy.device)
    tpmlp_attn_out_bwd_wgrad(desc, dy, ctx, dWo, acc, ws, stream)
    return dctx, dWo


def attn_qkv_bwd(desc, dqkv, Wqkv, x, dWqkv=None, dbqkv=None, stream=None):
    """(dx_partial, dWqkv, dbqkv or None); with given dWqkv (and dbqkv) the
    gradients are added into them."""
    dx = _empty((desc.tokens, desc.hidden), _act_t(desc), dqkv.device)
    tpmlp_attn_qkv_bwd_dgrad(desc, dqkv, Wqkv, dx, stream)
    acc = dWqkv is not None
    if not acc:
        dWqkv = _empty((desc.nqkv, desc.hidden), torch.float32, dqkv.device)
        dbqkv = _empty((desc.nqkv,), torch.float32, dqkv.device) if desc.has_bias else None
    tpmlp_attn_qkv_bwd_wgrad(desc, dqkv, x, dWqkv, dbqkv, acc, _attn_ws(desc, dqkv.device), stream)
    return dx, dWqkv, dbqkv


# ------------------------------------------------------------------ mixture of experts
def moe_workspace_size(desc: MoeDesc) -> int:
    return int(lib.tpmlp_moe_workspace_size(ctypes.byref(desc)))


def _counts(counts):
    if counts.dtype != torch.int32:
        raise ValueError("counts must be an int32 device tensor")
    return counts


def tpmlp_moe_fwd(desc, counts, x, W1, b1, W2, y, h, a, stream=None):
    _check(lib.tpmlp_moe_fwd(ctypes.byref(desc), _ptr(_counts(counts)), _ptr(x), _ptr(W1),
                             _ptr(b1), _ptr(W2), _ptr(y), _ptr(h), _ptr(a), _stream(stream)),
           "tpmlp_moe_fwd")


def tpmlp_moe_bwd_dgrad(desc, counts, dy, W1, W2, h, dH, dx, stream=None):
    _check(lib.tpmlp_moe_bwd_dgrad(ctypes.byref(desc), _ptr(_counts(counts)), _ptr(dy), _ptr(W1),
                                   _ptr(W2), _ptr(h), _ptr(dH), _ptr(dx), _stream(stream)),
           "tpmlp_moe_bwd_dgrad")


def tpmlp_moe_bwd_wgrad(desc, counts, dy, x, a, dH, dW1, db1, dW2, accumulate=False,
                        workspace=None, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.tpmlp_moe_bwd_wgrad(ctypes.byref(desc), _ptr(_counts(counts)), _ptr(dy), _ptr(x),
                                   _ptr(a), _ptr(dH), _ptr(dW1), _ptr(db1), _ptr(dW2),
                                   int(bool(accumulate)), _ptr(workspace), nbytes,
                                   _stream(stream)), "tpmlp_moe_bwd_wgrad")


def moe_fwd(desc, counts, x, W1, b1, W2, stream=None):
    """dict y, h, a of the grouped rows (rows past the sum of counts unset)."""
    G = 2 if desc.act == SWIGLU else 1
    T, H, Fs = desc.tokens, desc.hidden, desc.ffn_shard
    out = {"y": _empty((T, H), torch.bfloat16, x.device),
           "h": _empty((T, G * Fs), torch.bfloat16, x.device),
           "a": _empty((T, Fs), torch.bfloat16, x.device)}
    tpmlp_moe_fwd(desc, counts, x, W1, b1, W2, out["y"], out["h"], out["a"], stream)
    return out


def moe_bwd_dgrad(desc, counts, dy, W1, W2, h, stream=None):
    G = 2 if desc.act == SWIGLU else 1
    T, H, Fs = desc.tokens, desc.hidden, desc.ffn_shard
    out = {"dH": _empty((T, G * Fs), torch.bfloat16, dy.device),
           "dx": _empty((T, H), torch.bfloat16, dy.device)}
    tpmlp_moe_bwd_dgrad(desc, counts, dy, W1, W2, h, out["dH"], out["dx"], stream)
    return out


def moe_bwd_wgrad(desc, counts, dy, x, a, dH, accumulate_into=None, stream=None):
    """Per-expert fp32 dW1 [E, G*Fs, H], db1 [E, G*Fs], dW2 [E, H, Fs]."""
    G = 2 if desc.act == SWIGLU else 1
    E, H, Fs = desc.experts, desc.hidden, desc.ffn_shard
    if accumulate_into is not None:
        out = accumulate_into
    else:
        out = {"dW1": _empty((E, G * Fs, H), torch.float32, dy.device),
               "db1": _empty((E, G * Fs), torch.float32, dy.device) if desc.has_bias else None,
               "dW2": _empty((E, H, Fs), torch.float32, dy.device)}
    n = moe_workspace_size(desc)
    ws = _empty((n,), torch.uint8, dy.device) if n else None
    tpmlp_moe_bwd_wgrad(desc, counts, dy, x, a, dH, out["dW1"], out.get("db1"), out["dW2"],
                        accumulate_into is not None, ws, stream)
    return out


def timing_enable(enable: bool, name_filter: str | None = None):
    _check(lib.tpmlp_timing_enable(int(bool(enable)),
                                   None if name_filter is None else name_filter.encode()),
           "tpmlp_timing_enable")


def timing_clock_mhz(name: str) -> float:
    """Mean shader clock (MHz) of the GEMM launches `name` timed before the
    last timing_collect(); 0.0 if none."""
    return float(lib.tpmlp_timing_clock_mhz(name.encode()))


def timing_collect(cap: int = 64) -> dict:
    names = (ctypes.c_char_p * cap)()
    counts = (ctypes.c_int64 * cap)()
    tot = (ctypes.c_double * cap)()
    n = lib.tpmlp_timing_collect(names, counts, tot, cap)
    if n < 0:
        raise RuntimeError("tpmlp_timing_collect failed")
    return {names[i].decode(): (int(counts[i]), float(tot[i])) for i in range(min(n, cap))}


__all__ = ["Desc", "Fp8Scales", "Fp8History", "DelayedScaling", "fp8_scales", "TpmlpError",
           "make_desc", "workspace_size", "tpmlp_fwd", "tpmlp_bwd_dgrad", "tpmlp_bwd_wgrad",
           "tpmlp_bwd_wgrad_noalloc", "tpmlp_bwd_wgrad_recompute", "SCRATCH_BYTES",
           "tpmlp_bwd_wgrad_t", "tpmlp_transpose_u8", "token_ld", "transpose_u8", "bwd_wgrad_t",
           "CALL_FWD", "CALL_DGRAD", "CALL_WGRAD", "CALL_WGRAD_RECOMPUTE",
           "tpmlp_quantize_e4m3", "tpmlp_quantize_e5m2", "fwd", "bwd_dgrad", "bwd_wgrad",
           "quantize_e4m3", "quantize_e5m2", "timing_enable", "timing_collect", "timing_clock_mhz",
           "lib", "LIB_PATH",
           "F32", "BF16", "E4M3", "GELU", "SWIGLU",
           "AttnDesc", "make_attn_desc", "attn_workspace_size", "tpmlp_attn_qkv_fwd",
           "tpmlp_attn_out_fwd", "tpmlp_attn_out_bwd_dgrad", "tpmlp_attn_out_bwd_wgrad",
           "tpmlp_attn_qkv_bwd_dgrad", "tpmlp_attn_qkv_bwd_wgrad", "attn_qkv_fwd",
           "attn_out_fwd", "attn_out_bwd", "attn_qkv_bwd",
           "MoeDesc", "make_moe_desc", "moe_workspace_size", "tpmlp_moe_fwd",
           "tpmlp_moe_bwd_dgrad", "tpmlp_moe_bwd_wgrad", "moe_fwd", "moe_bwd_dgrad",
           "moe_bwd_wgrad"]
