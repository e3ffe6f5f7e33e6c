"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/tpmlp.h, and rejects invalid arguments with the documented
status codes before any HIP call (fake device addresses are never touched,
because validation fails first)."""
import ctypes
import os
import re

import pytest

import tensor_transformer_mlp_rank_amd as tp

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "tpmlp.h")
OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_UNSUP, E_WS, E_HIP, E_SCRATCH = range(9)
P = 0x100000          # fake, 16-byte aligned "device" address (never dereferenced)
MIS = 0x100008        # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tpmlp_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"tpmlp_fwd", "tpmlp_bwd_dgrad", "tpmlp_bwd_wgrad"} <= set(names)
    for n in names:
        assert hasattr(tp.lib, n), n


def test_version_and_strings():
    assert tp.lib.tpmlp_abi_version() == 9
    for s in range(9):
        assert len(tp.lib.tpmlp_strerror(s)) > 5
    assert tp.lib.tpmlp_last_hip_error() == b""


def fwd(desc, x=P, W1=P, b1=P, W2=P, y=P, h=P, a=P, fp8=None, ws=None, nbytes=0):
    d = None if desc is None else ctypes.byref(desc)
    sc = None if fp8 is None else ctypes.byref(fp8)
    return tp.lib.tpmlp_fwd(d, x, W1, b1, W2, y, h, a, sc, ws, nbytes, None)


def dgrad(desc, dy=P, W1=P, W2=P, h=P, dH=P, dx=P, fp8=None, ws=None, nbytes=0):
    sc = None if fp8 is None else ctypes.byref(fp8)
    return tp.lib.tpmlp_bwd_dgrad(ctypes.byref(desc), dy, W1, W2, h, dH, dx, sc, ws, nbytes, None)


def wgrad(desc, dy=P, x=P, a=P, dH=P, dW1=P, db1=P, dW2=P, acc=0, fp8=None, ws=None, nbytes=0):
    sc = None if fp8 is None else ctypes.byref(fp8)
    return tp.lib.tpmlp_bwd_wgrad(ctypes.byref(desc), dy, x, a, dH, dW1, db1, dW2, acc, sc, ws,
                                  nbytes, None)


def D(**kw):
    base = dict(tokens=64, hidden=256, ffn_shard=128, act="gelu", dtype="bf16", has_bias=True)
    base.update(kw)
    return tp.make_desc(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(tokens=-1), E_SHAPE), (dict(hidden=0), E_SHAPE), (dict(ffn_shard=-16), E_SHAPE),
    (dict(hidden=264), E_SHAPE), (dict(ffn_shard=136), E_SHAPE), (dict(hidden=1 << 23), E_SHAPE),
    (dict(tokens=1 << 30, hidden=1 << 21), E_SHAPE),   # a tile grid past 2^31 workgroups
    (dict(ffn_shard=(1 << 22) - 16 + 32, act="swiglu", has_bias=False), E_SHAPE),
    (dict(dtype=9), E_DTYPE), (dict(act=4), E_DTYPE),
    (dict(act="swiglu", has_bias=True), E_UNSUP),
    (dict(act="swiglu", dtype="e4m3", has_bias=True), E_UNSUP),
])
def test_desc_validation(kw, code):
    assert fwd(D(**kw)) == code


def test_desc_null_and_reserved_and_flags():
    assert fwd(None) == E_NULL
    d = D()
    d.reserved = 1
    assert fwd(d) == E_DTYPE
    d = D()
    d.has_bias = 2
    assert fwd(d) == E_DTYPE


@pytest.mark.parametrize("name", ["x", "W1", "W2", "y", "a"])
def test_fwd_required_pointers(name):
    assert fwd(D(), **{name: None}) == E_NULL
    assert fwd(D(), **{name: MIS}) == E_ALIGN


def test_fwd_bias_and_h_rules():
    assert fwd(D(has_bias=True), b1=None) == E_NULL
    assert fwd(D(has_bias=True), b1=MIS) == E_ALIGN
    assert fwd(D(), h=MIS) == E_ALIGN


def test_fp8_rules():
    d8 = D(dtype="e4m3")
    sc = tp.Fp8Scales(P, P, P, P, P)
    assert fwd(d8) == E_NULL                           # scales required
    assert fwd(D(), fp8=sc) == E_DTYPE                 # scales only for e4m3
    assert fwd(d8, fp8=tp.Fp8Scales(P, None, P, P, P)) == E_NULL
    assert fwd(d8, fp8=tp.Fp8Scales(P, P, P, None, P)) == E_NULL   # current scaling: amax out
    need = tp.workspace_size(d8, tp.CALL_FWD)
    assert need >= 64 * 128 * 2
    assert fwd(d8, fp8=sc) == E_WS
    assert fwd(d8, fp8=sc, ws=P, nbytes=need - 1) == E_WS
    assert fwd(d8, fp8=sc, ws=MIS, nbytes=need) == E_ALIGN
    assert dgrad(d8) == E_NULL                         # fp8 scales required
    assert wgrad(d8) == E_NULL
    assert dgrad(D(), fp8=sc) == E_DTYPE
    assert wgrad(D(), fp8=sc) == E_DTYPE
    # the gated block in E4M3: the same checks (its workspace has the pair
    # tiles' amax partials)
    d8g = D(dtype="e4m3", act="swiglu", has_bias=False)
    need_g = tp.workspace_size(d8g, tp.CALL_FWD)
    assert need_g >= 64 * 128 * 2
    assert fwd(d8g, fp8=sc) == E_WS
    assert fwd(d8g, fp8=sc, ws=P, nbytes=need_g - 1) == E_WS
    assert dgrad(d8g) == E_NULL


def _hist(length=4, reserved=0, ptrs=True):
    return tp.Fp8History(P if ptrs else None, P, P, length, reserved)


def test_fp8_delayed_and_backward_rules():
    d8 = D(dtype="e4m3")
    h = _hist()
    # forward with delayed scaling: no amax output needed; the history is checked
    ok_fwd = tp.Fp8Scales(P, P, P, None, None, ctypes.pointer(h))
    need = tp.workspace_size(d8, tp.CALL_FWD)
    assert fwd(d8, fp8=ok_fwd) == E_WS                 # passes validation up to the workspace
    for bad in (_hist(0), _hist(4097), _hist(4, reserved=1)):
        sc = tp.Fp8Scales(P, P, P, None, None, ctypes.pointer(bad))
        assert fwd(d8, fp8=sc, ws=P, nbytes=need) == E_SHAPE
    sc = tp.Fp8Scales(P, P, P, None, None, ctypes.pointer(_hist(ptrs=False)))
    assert fwd(d8, fp8=sc, ws=P, nbytes=need) == E_NULL
    # dgrad: dy, W1, W2 scales and the dH history are required; workspace = amax partials
    need_d = tp.workspace_size(d8, tp.CALL_DGRAD)
    assert need_d >= 4
    full = dict(x_scale_inv=None, w1_scale_inv=P, w2_scale_inv=P, a_amax=None, a_scale_inv=None,
                a_history=None, dy_scale_inv=P, dH_history=ctypes.pointer(h), dH_scale_inv=None)
    assert dgrad(d8, fp8=tp.Fp8Scales(**full)) == E_WS
    assert dgrad(d8, fp8=tp.Fp8Scales(**full), ws=P, nbytes=need_d - 1) == E_WS
    for k in ("w1_scale_inv", "w2_scale_inv", "dy_scale_inv", "dH_history"):
        assert dgrad(d8, fp8=tp.Fp8Scales(**dict(full, **{k: None})), ws=P, nbytes=need_d) == E_NULL
    bad = ctypes.pointer(_hist(0))
    assert dgrad(d8, fp8=tp.Fp8Scales(**dict(full, dH_history=bad)), ws=P, nbytes=need_d) == E_SHAPE
    # wgrad: dy, x, a, dH scales are required
    need_w = tp.workspace_size(d8, tp.CALL_WGRAD)
    assert need_w == 1 * 128 * 4                       # db1 partials, as for bf16
    wfull = dict(x_scale_inv=P, a_scale_inv=P, dy_scale_inv=P, dH_scale_inv=P)
    assert wgrad(d8, fp8=tp.Fp8Scales(**wfull)) == E_WS
    for k in wfull:
        assert wgrad(d8, fp8=tp.Fp8Scales(**dict(wfull, **{k: None})), ws=P, nbytes=need_w) == E_NULL


def test_workspace_sizes():
    assert tp.workspace_size(D(), tp.CALL_FWD) == 0
    assert tp.workspace_size(D(), tp.CALL_DGRAD) == 0
    assert tp.workspace_size(D(dtype="e4m3"), tp.CALL_DGRAD) == 256  # one amax partial, padded
    # bf16 wgrad with bias: one fp32 row of db1 partials per 256-column tile of H
    assert tp.workspace_size(D(), tp.CALL_WGRAD) == 1 * 128 * 4
    assert tp.workspace_size(D(hidden=4096, ffn_shard=1000 - 1000 % 16), tp.CALL_WGRAD) == \
        (16 * 992 * 4 + 255) // 256 * 256
    assert tp.workspace_size(D(has_bias=False), tp.CALL_WGRAD) == 0
    assert tp.workspace_size(D(dtype="f32"), tp.CALL_WGRAD) == 0
    assert tp.workspace_size(D(hidden=3), tp.CALL_FWD) == 0      # invalid desc
    assert tp.workspace_size(D(dtype="e4m3"), 7) == 0            # invalid call
    # E4M3 forward: bf16 a (current scaling), then one amax partial per fc1
    # workgroup: 32 x 8 tiles of 256 x 256 for GELU, 32 x 16 pair tiles of
    # 256 x 128 for the gated block
    a_bytes = 8192 * 2048 * 2
    for act, parts in (("gelu", 32 * 8), ("swiglu", 32 * 16)):
        d = D(tokens=8192, hidden=4096, ffn_shard=2048, dtype="e4m3", act=act,
              has_bias=act == "gelu")
        assert tp.workspace_size(d, tp.CALL_FWD) == a_bytes + (parts * 4 + 4 + 255) // 256 * 256
        assert tp.workspace_size(d, tp.CALL_DGRAD) == (32 * 8 * 4 + 4 + 255) // 256 * 256


def _colsum_bytes(H, GFs, splits=1):
    return ((splits * ((H + 255) // 256) * GFs * 4 + 255) // 256) * 256


def test_split_k_plans_through_workspace_sizes():
    """The wgrad workspace adds split-K partial planes exactly where the tile
    grid would leave CUs idle: the 2048-hidden TP=4 shard (64 tiles of
    256 x 256 over K = 8192 tokens) splits four ways; the 8192-hidden TP=8
    shard (512 tiles, two full rounds) does not; FP8 and fp32 never do."""
    H = Fs = 2048
    got = tp.workspace_size(D(tokens=8192, hidden=H, ffn_shard=Fs), tp.CALL_WGRAD)
    planes = 4 * H * Fs * 4                      # four fp32 partial planes of the larger product
    assert got == _colsum_bytes(H, Fs, 4) + planes
    big = D(tokens=8192, hidden=8192, ffn_shard=4096)
    assert tp.workspace_size(big, tp.CALL_WGRAD) == _colsum_bytes(8192, 4096)
    # FP8 never splits along K (its 64-tile dW2 takes the partial-round split instead)
    assert tp.workspace_size(D(tokens=8192, hidden=H, ffn_shard=Fs, dtype="e4m3"),
                             tp.CALL_WGRAD) == _colsum_bytes(H, Fs) + _tail_bytes(64)
    assert tp.workspace_size(D(tokens=8192, hidden=H, ffn_shard=Fs, dtype="f32"),
                             tp.CALL_WGRAD) == 0
    # too few stages to split (K = 512 tokens): the colsum rows only
    assert tp.workspace_size(D(tokens=512, hidden=H, ffn_shard=Fs), tp.CALL_WGRAD) == \
        _colsum_bytes(H, Fs)
    # without bias the planes alone
    assert tp.workspace_size(D(tokens=8192, hidden=H, ffn_shard=Fs, has_bias=False),
                             tp.CALL_WGRAD) == planes
    # the attention out-projection backward at the 8192-hidden shard (128 tiles) splits in two
    a = tp.make_attn_desc(8192, 8192, 8, 8, 128, dtype="bf16", has_bias=True)
    assert tp.attn_workspace_size(a) >= 2 * 8192 * 1024 * 4


def _tail_bytes(tiles):
    return (tiles * 4 + 255) // 256 * 256 + tiles * 2 * 256 * 256 * 4


def test_partial_last_round_plans_through_workspace_sizes():
    """Weight gradients whose tiles leave a last round of 8 to 128 workgroups
    on the 256 compute units run that many tiles (rounded down to a multiple
    of 8) as two half-K workgroups each; the halves meet in the workspace (a
    counter per tile, then two 256 x 256 fp32 dumps). At the SwiGLU
    4096-hidden TP=2 shard (T = 8192, Fs = 7168) fc1's weight gradient
    (56 x 16 = 896 tiles) splits 128 tiles; fc2's (448 tiles: a last round of
    192) does not, nor do the other calls' products."""
    sw = D(tokens=8192, hidden=4096, ffn_shard=7168, act="swiglu", has_bias=False)
    assert tp.workspace_size(sw, tp.CALL_WGRAD) == _tail_bytes(128)
    assert tp.workspace_size(sw, tp.CALL_DGRAD) == 0
    assert tp.workspace_size(sw, tp.CALL_FWD) == 0
    # with bias fc1's product (896 tiles) carries the fused column sum and does not
    # split; fc2's (16 x 56 = 896 tiles) does
    assert tp.workspace_size(D(tokens=8192, hidden=4096, ffn_shard=14336), tp.CALL_WGRAD) == \
        _colsum_bytes(4096, 14336) + _tail_bytes(128)
    # whole rounds (the 8192-hidden TP=8 shard): nothing to split
    big = D(tokens=8192, hidden=8192, ffn_shard=4096)
    assert tp.workspace_size(big, tp.CALL_WGRAD) == _colsum_bytes(8192, 4096)
    # fewer than 16 stages of K: no split (K = T = 960 tokens is 15 stages of 64; 1024 is 16)
    short = dict(hidden=4096, ffn_shard=7168, act="swiglu", has_bias=False)
    assert tp.workspace_size(D(tokens=960, **short), tp.CALL_WGRAD) == 0
    assert tp.workspace_size(D(tokens=1024, **short), tp.CALL_WGRAD) == _tail_bytes(128)
    # a last round of 4 tiles (13 x 20 = 260): no split; of 12 (4 x 67 = 268): 8 of them split
    assert tp.workspace_size(D(tokens=4096, hidden=13 * 256, ffn_shard=20 * 256, has_bias=False),
                             tp.CALL_WGRAD) == 0
    assert tp.workspace_size(D(tokens=4096, hidden=4 * 256, ffn_shard=67 * 256, has_bias=False),
                             tp.CALL_WGRAD) == _tail_bytes(8)
    # the fp32 kernel never splits
    assert tp.workspace_size(D(tokens=8192, dtype="f32", **short), tp.CALL_WGRAD) == 0
    # the allocation-free call never splits either: it needs no workspace without bias
    assert tp.workspace_size(sw, tp.CALL_WGRAD) > 0


@pytest.mark.parametrize("name", ["dy", "W1", "W2", "h", "dH", "dx"])
def test_dgrad_pointers(name):
    assert dgrad(D(), **{name: None}) == E_NULL
    assert dgrad(D(), **{name: MIS}) == E_ALIGN


@pytest.mark.parametrize("name", ["dy", "x", "a", "dH", "dW1", "dW2"])
def test_wgrad_pointers(name):
    assert wgrad(D(), **{name: None}) == E_NULL
    assert wgrad(D(), **{name: MIS}) == E_ALIGN


def test_wgrad_bias_and_flag():
    assert wgrad(D(has_bias=True), db1=None) == E_NULL
    assert wgrad(D(), acc=2) == E_DTYPE


def test_wgrad_workspace():
    need = tp.workspace_size(D(), tp.CALL_WGRAD)
    args = (ctypes.byref(D()), P, P, P, P, P, P, P, 0, None)
    assert tp.lib.tpmlp_bwd_wgrad(*args, None, 0, None) == E_WS
    assert tp.lib.tpmlp_bwd_wgrad(*args, P, need - 1, None) == E_WS
    assert tp.lib.tpmlp_bwd_wgrad(*args, MIS, need, None) == E_ALIGN


def wgrad_recompute(desc, dy=P, x=P, h=P, dH=P, dW1=P, db1=P, dW2=P, acc=0, fp8=None, ws=P,
                    nbytes=1 << 40):
    sc = None if fp8 is None else ctypes.byref(fp8)
    return tp.lib.tpmlp_bwd_wgrad_recompute(ctypes.byref(desc), dy, x, h, dH, dW1, db1, dW2, acc,
                                            sc, ws, nbytes, None)


@pytest.mark.parametrize("name", ["dy", "x", "h", "dH", "dW1", "dW2"])
def test_wgrad_recompute_validation(name):
    """The recomputing weight gradient checks its arguments as
    tpmlp_bwd_wgrad does (h_saved in a_saved's place), then its workspace."""
    assert wgrad_recompute(D(), **{name: None}) == E_NULL
    assert wgrad_recompute(D(), **{name: MIS}) == E_ALIGN
    assert wgrad_recompute(D(has_bias=True), db1=None) == E_NULL
    assert wgrad_recompute(D(), acc=2) == E_DTYPE
    assert wgrad_recompute(D(dtype="e4m3")) == E_NULL  # FP8 without scales
    need = tp.workspace_size(D(), tp.CALL_WGRAD_RECOMPUTE)
    assert wgrad_recompute(D(), ws=None, nbytes=0) == E_WS
    assert wgrad_recompute(D(), nbytes=need - 1) == E_WS
    assert wgrad_recompute(D(), ws=MIS, nbytes=need) == E_ALIGN


def wgrad_t(desc, dy=P, x=P, a=P, dH=P, dW1=P, db1=P, dW2=P, acc=0, fp8=None):
    sc = None if fp8 is None else ctypes.byref(fp8)
    return tp.lib.tpmlp_bwd_wgrad_t(ctypes.byref(desc), dy, x, a, dH, dW1, db1, dW2, acc, sc,
                                    None)


@pytest.mark.parametrize("name", ["dy", "x", "a", "dH", "dW1", "dW2"])
def test_wgrad_t_validation(name):
    """The token-contiguous weight gradient checks its arguments as
    tpmlp_bwd_wgrad does; it is E4M3 only and takes no workspace."""
    d8 = D(dtype="e4m3")
    full = dict(dy_scale_inv=P, x_scale_inv=P, a_scale_inv=P, dH_scale_inv=P)
    sc = tp.Fp8Scales(**full)
    assert wgrad_t(d8, fp8=sc, **{name: None}) == E_NULL
    assert wgrad_t(d8, fp8=sc, **{name: MIS}) == E_ALIGN
    assert wgrad_t(d8, fp8=sc, db1=None) == E_NULL          # bias without db1
    assert wgrad_t(d8, fp8=sc, acc=2) == E_DTYPE
    assert wgrad_t(d8) == E_NULL                            # FP8 without scales
    for k in full:
        assert wgrad_t(d8, fp8=tp.Fp8Scales(**dict(full, **{k: None}))) == E_NULL
    assert wgrad_t(D(), fp8=None) == E_UNSUP                # bf16: not this entry
    assert wgrad_t(D(dtype="f32")) == E_UNSUP
    assert wgrad_t(D(hidden=3), fp8=sc) == E_SHAPE
    # token-contiguous rows past 2^23 - 256 bytes: 256 of them overflow 32-bit offsets
    assert wgrad_t(D(dtype="e4m3", tokens=(1 << 23) - 255), fp8=sc) == E_SHAPE


def test_transpose_u8_validation():
    """Sizes: cols a multiple of 16, neither negative; empty arrays are a
    no-op (nothing enqueued, NULL pointers accepted)."""
    T = tp.lib.tpmlp_transpose_u8
    assert T(P, 4, 24, P, None) == E_SHAPE
    assert T(P, -1, 16, P, None) == E_SHAPE
    assert T(P, 4, -16, P, None) == E_SHAPE
    assert T(None, 0, 16, None, None) == 0
    assert T(None, 7, 0, None, None) == 0
    assert T(None, 4, 16, P, None) == E_NULL
    assert T(P, 4, 16, MIS, None) == E_ALIGN
    assert tp.token_ld(0) == 0 and tp.token_ld(1) == 16 and tp.token_ld(32) == 32


def test_wgrad_recompute_workspace_size():
    """The recomputed activation ([T][Fs] of the call's element type, rounded
    up to 256 bytes) in front of the weight gradient's own workspace."""
    for dt, es in (("bf16", 2), ("f32", 4), ("e4m3", 1)):
        for act, bias in (("gelu", True), ("swiglu", False)):
            d = D(tokens=100, ffn_shard=144, dtype=dt, act=act, has_bias=bias)
            a = (100 * 144 * es + 255) // 256 * 256
            assert tp.workspace_size(d, tp.CALL_WGRAD_RECOMPUTE) == \
                a + tp.workspace_size(d, tp.CALL_WGRAD), (dt, act)
    assert tp.workspace_size(D(tokens=0), tp.CALL_WGRAD_RECOMPUTE) == \
        tp.workspace_size(D(tokens=0), tp.CALL_WGRAD)
    assert tp.workspace_size(D(), 4) == 0                         # invalid call


def wgrad_noalloc(desc, dy=P, x=P, a=P, dH=P, dW1=P, db1=P, dW2=P, acc=0, fp8=None):
    sc = None if fp8 is None else ctypes.byref(fp8)
    return tp.lib.tpmlp_bwd_wgrad_noalloc(ctypes.byref(desc), dy, x, a, dH, dW1, db1, dW2, acc,
                                          sc, None)


@pytest.mark.parametrize("name", ["dy", "x", "a", "dH", "dW1", "dW2"])
def test_wgrad_noalloc_validation(name):
    """The allocation-free weight gradient checks its arguments as
    tpmlp_bwd_wgrad does, before anything else."""
    assert wgrad_noalloc(D(), **{name: None}) == E_NULL
    assert wgrad_noalloc(D(), **{name: MIS}) == E_ALIGN
    assert wgrad_noalloc(D(has_bias=True), db1=None) == E_NULL
    assert wgrad_noalloc(D(), acc=2) == E_DTYPE
    assert wgrad_noalloc(D(dtype="e4m3")) == E_NULL  # FP8 without scales


def test_wgrad_noalloc_rejects_what_the_scratch_cannot_hold():
    """db1 partial sums of ceil(H / 256) * G * Fs floats beyond
    TPMLP_SCRATCH_BYTES: TPMLP_E_SCRATCH, before any HIP call."""
    assert tp.SCRATCH_BYTES == 8 << 20
    fits = D(tokens=64, hidden=8192, ffn_shard=8192)          # 32 * 8192 * 4 = 1 MiB
    big = D(tokens=64, hidden=65536, ffn_shard=16384)         # 256 * 16384 * 4 = 16 MiB
    gated = D(tokens=64, hidden=65536, ffn_shard=4112, act="swiglu", has_bias=False)
    assert tp.workspace_size(fits, tp.CALL_WGRAD) > 0
    assert wgrad_noalloc(big) == E_SCRATCH
    # no bias: no partial sums, no scratch needed (validated like any call)
    assert wgrad_noalloc(gated, db1=None, dW1=MIS) == E_ALIGN


def test_quantize_validation():
    q = tp.lib.tpmlp_quantize_e4m3
    ws = int(tp.lib.tpmlp_quantize_workspace_size(1000))
    assert ws >= 4
    assert q(5, P, 1000, P, P, P, P, ws, None) == E_DTYPE
    assert q(tp.BF16, P, -1, P, P, P, P, ws, None) == E_SHAPE
    assert q(tp.BF16, P, 1000, P, None, P, P, ws, None) == E_NULL
    assert q(tp.BF16, None, 1000, P, P, P, P, ws, None) == E_NULL
    assert q(tp.BF16, MIS, 1000, P, P, P, P, ws, None) == E_ALIGN
    assert q(tp.BF16, P, 1000, P, P, P, None, ws, None) == E_WS
    assert q(tp.BF16, P, 1000, P, P, P, P, ws - 1, None) == E_WS


def test_timing_facility_without_records():
    assert tp.lib.tpmlp_timing_enable(1, b"fc1") == 0
    assert tp.timing_collect() == {}
    assert tp.lib.tpmlp_timing_enable(0, None) == 0


# ------------------------------------------------------------------ attention projections
def A(**kw):
    base = dict(tokens=64, hidden=256, q_heads=8, kv_heads=2, head_dim=64, dtype="bf16",
                has_bias=True)
    base.update(kw)
    return tp.make_attn_desc(**base)


def attn_calls(d, p=P, acc=0, ws=None, nbytes=0, bias=P):
    """status of each of the six attention calls with every pointer = p"""
    b = ctypes.byref(d) if d is not None else None
    L = tp.lib
    return [L.tpmlp_attn_qkv_fwd(b, p, p, bias, p, None),
            L.tpmlp_attn_out_fwd(b, p, p, p, None),
            L.tpmlp_attn_out_bwd_dgrad(b, p, p, p, None, 0, None),
            L.tpmlp_attn_out_bwd_wgrad(b, p, p, p, acc, None, 0, None),
            L.tpmlp_attn_qkv_bwd_dgrad(b, p, p, p, None),
            L.tpmlp_attn_qkv_bwd_wgrad(b, p, p, p, bias, acc, ws, nbytes, None)]


@pytest.mark.parametrize("kw,code", [
    (dict(tokens=-1), E_SHAPE), (dict(hidden=0), E_SHAPE), (dict(hidden=264), E_SHAPE),
    (dict(q_heads=0), E_SHAPE), (dict(kv_heads=0), E_SHAPE), (dict(kv_heads=3), E_SHAPE),
    (dict(head_dim=72), E_SHAPE), (dict(head_dim=-16), E_SHAPE),
    (dict(q_heads=1 << 16, kv_heads=1 << 16), E_SHAPE), (dict(hidden=1 << 23), E_SHAPE),
    (dict(tokens=1 << 30, hidden=1 << 21, q_heads=16, kv_heads=16, head_dim=64), E_SHAPE),
    (dict(dtype=9), E_DTYPE), (dict(dtype="e4m3"), E_UNSUP),
])
def test_attn_desc_validation(kw, code):
    assert attn_calls(A(**kw)) == [code] * 6


def test_attn_null_reserved_pointers_alignment():
    assert attn_calls(None) == [E_NULL] * 6
    d = A()
    d.reserved = 1
    assert attn_calls(d) == [E_DTYPE] * 6
    d = A()
    d.has_bias = 2
    assert attn_calls(d) == [E_DTYPE] * 6
    assert attn_calls(A(), p=None) == [E_NULL] * 6
    assert attn_calls(A(), p=MIS) == [E_ALIGN] * 6


# Each case below fails validation; calls that would pass it are never made
# (their fake addresses must not reach a kernel).
def test_attn_bias_and_accumulate_rules():
    L, d = tp.lib, A()
    b = ctypes.byref(d)
    # the bias pointer is required with has_bias
    assert L.tpmlp_attn_qkv_fwd(b, P, P, None, P, None) == E_NULL
    assert L.tpmlp_attn_qkv_bwd_wgrad(b, P, P, P, None, 0, P, 1 << 20, None) == E_NULL
    assert L.tpmlp_attn_qkv_fwd(b, P, P, MIS, P, None) == E_ALIGN
    # accumulate is 0 or 1
    assert L.tpmlp_attn_out_bwd_wgrad(b, P, P, P, 2, None, 0, None) == E_DTYPE
    # a workspace given must be aligned
    assert L.tpmlp_attn_out_bwd_dgrad(b, P, P, P, MIS, 1 << 20, None) == E_ALIGN
    assert L.tpmlp_attn_out_bwd_wgrad(b, P, P, P, 0, MIS, 1 << 20, None) == E_ALIGN
    assert L.tpmlp_attn_qkv_bwd_wgrad(b, P, P, P, P, -1, P, 1 << 20, None) == E_DTYPE


def test_attn_workspace():
    d = A(tokens=1000, hidden=512, q_heads=8, kv_heads=8, head_dim=64)
    n = tp.attn_workspace_size(d)
    nqkv = (8 + 16) * 64
    tiles_n = (512 + 255) // 256
    need = ((tiles_n * nqkv * 4 + 255) // 256) * 256   # dbqkv partials of an unsplit product
    assert n >= need and n % 256 == 0
    assert tp.attn_workspace_size(A(hidden=7)) == 0
    assert tp.attn_workspace_size(A(dtype="f32")) == 0            # fp32: no split, no partials
    # qkv wgrad with bias: missing or short workspace, misaligned workspace
    L, b = tp.lib, ctypes.byref(d)
    assert L.tpmlp_attn_qkv_bwd_wgrad(b, P, P, P, P, 0, None, 0, None) == E_WS
    assert L.tpmlp_attn_qkv_bwd_wgrad(b, P, P, P, P, 0, P, need - 1, None) == E_WS
    assert L.tpmlp_attn_qkv_bwd_wgrad(b, P, P, P, P, 0, MIS, n, None) == E_ALIGN


# ------------------------------------------------------------------ mixture of experts
def Mo(**kw):
    base = dict(tokens=1000, hidden=256, ffn_shard=128, experts=8, act="gelu", dtype="bf16",
                has_bias=True)
    base.update(kw)
    return tp.make_moe_desc(**base)


def moe_calls(d, p=P, acc=0, ws=None, nbytes=0, bias=P, counts=P):
    b = ctypes.byref(d) if d is not None else None
    L = tp.lib
    return [L.tpmlp_moe_fwd(b, counts, p, p, bias, p, p, p, p, None),
            L.tpmlp_moe_bwd_dgrad(b, counts, p, p, p, p, p, p, None),
            L.tpmlp_moe_bwd_wgrad(b, counts, p, p, p, p, p, bias, p, acc, ws, nbytes, None)]


def test_moe_desc_struct_layout():
    assert ctypes.sizeof(tp.MoeDesc) == 48


@pytest.mark.parametrize("kw,code", [
    (dict(tokens=-1), E_SHAPE), (dict(hidden=0), E_SHAPE), (dict(ffn_shard=24), E_SHAPE),
    (dict(experts=0), E_SHAPE), (dict(experts=1025), E_SHAPE), (dict(hidden=1 << 22), E_SHAPE),
    (dict(tokens=1 << 30, hidden=1 << 21, experts=1024), E_SHAPE),
    (dict(dtype=9), E_DTYPE), (dict(act=5), E_DTYPE),
    (dict(dtype="f32"), E_UNSUP), (dict(dtype="e4m3"), E_UNSUP),
    (dict(act="swiglu", has_bias=True), E_UNSUP),
])
def test_moe_desc_validation(kw, code):
    assert moe_calls(Mo(**kw)) == [code] * 3


def test_moe_null_reserved_pointers():
    assert moe_calls(None) == [E_NULL] * 3
    for f in ("reserved0", "reserved1", "has_bias"):
        d = Mo()
        setattr(d, f, 2)
        assert moe_calls(d) == [E_DTYPE] * 3, f
    assert moe_calls(Mo(), counts=None) == [E_NULL] * 3
    assert moe_calls(Mo(), p=None) == [E_NULL] * 3
    assert moe_calls(Mo(), p=MIS) == [E_ALIGN] * 3
    assert moe_calls(Mo(), counts=MIS) == [E_ALIGN] * 3


def test_moe_bias_accumulate_workspace():
    L, d = tp.lib, Mo()
    b = ctypes.byref(d)
    assert L.tpmlp_moe_fwd(b, P, P, P, None, P, P, P, P, None) == E_NULL
    n = tp.moe_workspace_size(d)
    tiles_n = (256 + 255) // 256
    assert n == ((8 * tiles_n * 128 * 4 + 255) // 256) * 256
    assert tp.moe_workspace_size(Mo(has_bias=False)) == 0
    assert tp.moe_workspace_size(Mo(act="swiglu", has_bias=False)) == 0
    assert tp.moe_workspace_size(Mo(dtype="f32")) == 0
    assert L.tpmlp_moe_bwd_wgrad(b, P, P, P, P, P, P, None, P, 0, P, n, None) == E_NULL
    assert L.tpmlp_moe_bwd_wgrad(b, P, P, P, P, P, P, P, P, 2, P, n, None) == E_DTYPE
    assert L.tpmlp_moe_bwd_wgrad(b, P, P, P, P, P, P, P, P, 0, None, 0, None) == E_WS
    assert L.tpmlp_moe_bwd_wgrad(b, P, P, P, P, P, P, P, P, 0, P, n - 1, None) == E_WS
    assert L.tpmlp_moe_bwd_wgrad(b, P, P, P, P, P, P, P, P, 0, MIS, n, None) == E_ALIGN
