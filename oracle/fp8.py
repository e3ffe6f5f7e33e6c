"""FP8 encodings (OCP E4M3 and E5M2) and per-tensor scaling, current and
delayed (test infrastructure).

The pages name FP8 training through Transformer Engine (code tour, "Honest
Limits"; concept note, "Key math / How it works"; the onegen.ai overview,
"Key Features") but fix neither the format nor the recipe. Readings used:

* Format: OCP E4M3 ("E4M3FN"), from the OCP 8-bit Floating Point
  Specification (OFP8), revision 1.0, section 5.1 / Table 1: 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
  subnormals m * 2^-9; S.1111.111 is NaN; there is no infinity; the largest
  finite magnitude is 448 (S.1111.110).
* Rounding: round to nearest, ties to even; values beyond 448 in magnitude
  saturate to +-448 (the specification's saturating conversion mode).
* Scaling: per-tensor current scaling. amax = max |v| over the tensor;
  scale = 448 / amax computed in float32 (amax = 0, or an amax so small
  that the quotient overflows float32, gives scale 1);
  scale_inv = 1 / scale in float32; code = E4M3(fl32(v * scale));
  the dequantised value is decode(code) * scale_inv.

* Gradients (the backward pass): OCP E5M2, OFP8 section 5.1 / Table 1:
  1 sign bit, 5 exponent bits with bias 15, 2 mantissa bits; exponent field
  0 encodes subnormals m * 2^-16; exponent field 31 encodes infinities
  (mantissa 0) and NaN; the largest finite magnitude is 57344
  (S.11110.11). Forward tensors in E4M3 and gradients in E5M2 is
  Transformer Engine's default "hybrid" format, the plainest reading of FP8
  "via Transformer Engine"; conversions saturate at the largest finite
  value, as for E4M3.
* Delayed scaling (Transformer Engine's default recipe, margin 0): a tensor
  produced inside the block is quantised with a scale derived from the
  amaxes of earlier calls, so no pass over the whole tensor has to finish
  before the first code is written. After the call the tensor's own amax
  enters a history (newest first, oldest dropped) and the next scale is
  fmax / max(history), kept unchanged while that maximum is 0 or not
  finite, or so small that the factor would overflow float32.

The float32 steps (division, reciprocal, product) are taken in float32 on
purpose: the quantised code is an integer decided by floating point, so both
the oracle and the device quantiser decide it in the same precision.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_E4M3_MIN_NORMAL_EXP = -6      # smallest normal exponent (field 1, bias 7)
_E4M3_MANT_BITS = 3
E5M2_MAX = 57344.0
_E5M2_MIN_NORMAL_EXP = -14     # field 1, bias 15
_E5M2_MANT_BITS = 2
FMAX = {"e4m3": E4M3_MAX, "e5m2": E5M2_MAX}


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 byte as float64 (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m.astype(np.float64) * 2.0 ** (_E4M3_MIN_NORMAL_EXP - _E4M3_MANT_BITS)
    nrm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    val = np.where(e == 0, sub, nrm)
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


def e4m3_encode(v) -> np.ndarray:
    """Round each value to the nearest E4M3 code (ties to even), saturating
    magnitudes above 448 to 448; NaN maps to S.1111.111."""
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    mag = np.abs(v)
    nan = np.isnan(v)
    mag = np.where(nan, 0.0, np.minimum(mag, E4M3_MAX))
    # binade exponent e = floor(log2 mag), clamped to the subnormal floor
    _, ex = np.frexp(mag)
    e = np.maximum(ex.astype(np.int64) - 1, _E4M3_MIN_NORMAL_EXP)
    quantum = np.exp2((e - _E4M3_MANT_BITS).astype(np.float64))
    n = np.rint(mag / quantum)                      # half to even; exact division
    r = n * quantum                                 # rounded magnitude (<= 448)
    # encode r
    _, exr = np.frexp(r)
    er = exr.astype(np.int64) - 1
    is_sub = (r < 2.0 ** _E4M3_MIN_NORMAL_EXP)
    field_e = np.where(is_sub, 0, er + 7)
    mant_sub = np.rint(r * 2.0 ** 9)
    mant_nrm = np.rint((r / np.exp2(er.astype(np.float64)) - 1.0) * 8.0)
    field_m = np.where(is_sub, mant_sub, mant_nrm).astype(np.int64)
    field_e = np.where(r == 0.0, 0, field_e)
    field_m = np.where(r == 0.0, 0, field_m)
    code = (field_e << 3) | field_m
    code = np.where(nan, 0x7F, code)
    code = code | (neg.astype(np.int64) << 7)
    return code.astype(np.uint8)


def current_scale(v, fmt: str = "e4m3"):
    """(amax, scale, scale_inv) of a tensor as float32 scalars.

    scale = fmax / amax in float32. An amax of 0 or a non-finite amax gives
    1, and so does an amax so small that fmax / amax overflows float32 (below
    about 1.3e-36 for E4M3): a factor of infinity would turn zeros into NaN
    (0 * inf) and make scale_inv 0."""
    v32 = np.asarray(v, dtype=np.float32)
    amax = np.float32(np.max(np.abs(v32))) if v32.size else np.float32(0.0)
    scale = np.float32(1.0)
    if amax > 0.0 and np.isfinite(amax):
        with np.errstate(over="ignore"):
            s = np.float32(np.float32(FMAX[fmt]) / amax)
        if np.isfinite(s):
            scale = s
    scale_inv = np.float32(np.float32(1.0) / scale)
    return amax, scale, scale_inv


def quantize_e4m3(v, scale=None):
    """Quantise float32 values with per-tensor current scaling.

    Returns (codes uint8, amax, scale, scale_inv). ``scale`` overrides the
    current-scaling factor (for testing a given scale)."""
    v32 = np.asarray(v, dtype=np.float32)
    amax, s, s_inv = current_scale(v32)
    if scale is not None:
        s = np.float32(scale)
        s_inv = np.float32(np.float32(1.0) / s)
    prod = (v32 * s).astype(np.float32)             # fl32(v * scale)
    return e4m3_encode(prod), amax, s, s_inv


def dequantize_e4m3(codes, scale_inv) -> np.ndarray:
    """decode(code) * scale_inv in float64 (exact: 4-bit by 24-bit product)."""
    return e4m3_decode(codes) * np.float64(np.float32(scale_inv))


def e5m2_decode(codes) -> np.ndarray:
    """Value of each E5M2 byte as float64 (+-inf for S.11111.00, NaN for
    S.11111.01 .. S.11111.11)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    m = c & 0x3
    sub = m.astype(np.float64) * 2.0 ** (_E5M2_MIN_NORMAL_EXP - _E5M2_MANT_BITS)
    nrm = (1.0 + m / 4.0) * np.exp2(e.astype(np.float64) - 15.0)
    val = np.where(e == 0, sub, nrm)
    val = np.where((e == 0x1F) & (m == 0), np.inf, val)
    val = np.where((e == 0x1F) & (m != 0), np.nan, val)
    return sign * val


def e5m2_encode(v) -> np.ndarray:
    """Round each value to the nearest E5M2 code (ties to even), saturating
    magnitudes above 57344 (infinities included) to 57344; NaN maps to
    S.11111.11."""
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    nan = np.isnan(v)
    mag = np.where(nan, 0.0, np.minimum(np.abs(v), E5M2_MAX))
    _, ex = np.frexp(mag)
    e = np.maximum(ex.astype(np.int64) - 1, _E5M2_MIN_NORMAL_EXP)
    quantum = np.exp2((e - _E5M2_MANT_BITS).astype(np.float64))
    r = np.rint(mag / quantum) * quantum            # half to even; <= 57344
    _, exr = np.frexp(r)
    er = exr.astype(np.int64) - 1
    is_sub = r < 2.0 ** _E5M2_MIN_NORMAL_EXP
    field_e = np.where(is_sub, 0, er + 15)
    mant_sub = np.rint(r * 2.0 ** 16)
    mant_nrm = np.rint((r / np.exp2(er.astype(np.float64)) - 1.0) * 4.0)
    field_m = np.where(is_sub, mant_sub, mant_nrm).astype(np.int64)
    field_e = np.where(r == 0.0, 0, field_e)
    field_m = np.where(r == 0.0, 0, field_m)
    code = (field_e << 2) | field_m
    code = np.where(nan, 0x7F, code)
    code = code | (neg.astype(np.int64) << 7)
    return code.astype(np.uint8)


_ENC = {"e4m3": e4m3_encode, "e5m2": e5m2_encode}
_DEC = {"e4m3": e4m3_decode, "e5m2": e5m2_decode}


def quantize(v, fmt: str, scale):
    """Codes of fl32(fl32(v) * scale) in format fmt ("e4m3" or "e5m2")."""
    s = np.float32(scale)
    prod = (np.asarray(v, dtype=np.float32) * s).astype(np.float32)
    return _ENC[fmt](prod)


def dequantize(codes, fmt: str, scale_inv) -> np.ndarray:
    """decode(code) * scale_inv in float64."""
    return _DEC[fmt](codes) * np.float64(np.float32(scale_inv))


def delayed_update(history, amax, scale, fmt: str):
    """One step of delayed scaling, all in float32.

    ``history`` holds earlier amaxes, newest first; ``scale`` is the factor
    this call quantised with. Returns (new_history, new_scale, scale_inv):
    the history with ``amax`` in front and its oldest entry dropped, the
    factor for the next call, and 1 / scale (the dequantisation factor of
    this call's codes)."""
    h = np.asarray(history, dtype=np.float32)
    new_h = np.concatenate([np.array([amax], dtype=np.float32), h[:-1]]) if h.size else h
    scale = np.float32(scale)
    m = np.float32(np.max(new_h)) if new_h.size else np.float32(0.0)
    new_scale = scale
    if m > 0.0 and np.isfinite(m):
        with np.errstate(over="ignore"):
            s = np.float32(np.float32(FMAX[fmt]) / m)
        if np.isfinite(s):   # a maximum so small that the factor overflows keeps it too
            new_scale = s
    return new_h, new_scale, np.float32(np.float32(1.0) / scale)
