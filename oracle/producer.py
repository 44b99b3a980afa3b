"""The fused producer store in float64: per-head RMS norm and rotary embedding of
the step's query / key / index-query / index-key rows, then the FP4 store of K, V
and index K, and the main query as bf16 (and, optionally, e4m3).

Test infrastructure (see the package docstring): only the tests, the smoke check
and bench.py's CPU baseline may import this module.

Pages: ATOM PR "[MiniMax-M3.1] FP4 index cache and NVFP4 sparse KV cache",
Follow-up: MXFP4 caches (the quantization moves into the fused qk-norm / RoPE /
cache kernel, so no bf16 staging buffer and no store launch remain); vLLM PR
"MXFP4 KV + indexer cache for MiniMax-M3.1", Claims (the fused kernel writes the
K, V and index-K pages and writes the main query as e4m3).

The pages name the norm and the rotary embedding but define neither. Readings:
  * norm: RMS norm of each 128-dim head row with a per-tensor weight w (bf16):
        y = x / sqrt(mean(x^2) + eps) * w,
    applied to the query heads, the key, the index query and the index key;
    the value is not normed;
  * rotary: rotate-half pairs over the first rd dims (rd even, a multiple of 16,
    at most 128): for d < rd/2, with h = rd/2, c = cos[pos][d], s = sin[pos][d],
        (y_d, y_{d+h}) -> (y_d c - y_{d+h} s,  y_{d+h} c + y_d s),
    i.e. (y_d + i y_{d+h}) times (c + i s); dims rd..127 pass through. The angle
    table is an input (float32), so neither side evaluates a sine;
  * every produced row is rounded to bf16 (round to nearest even): the rows the
    unfused path stages. K, V and index K are quantized from those bf16 rows by
    the store rule, so the fused store writes the bytes the unfused one would;
  * the e4m3 query is the OCP E4M3FN value nearest to the bf16 query (ties to
    even, saturating at 448, sign bit = (q < 0)), with no scale.

A kernel evaluates these formulas in float32, so its bf16 results may differ
from the exact ones where an exact value lies within the float32 evaluation
error of a bf16 rounding boundary. ``produce`` therefore returns, per element,
the two bf16 values at the ends of [exact - tol, exact + tol]; they coincide
except at such boundaries, where either is correct. ``tol`` bounds the error of
any float32 evaluation order of the formulas above (derivation at ``_tolerance``).
"""
from __future__ import annotations

import numpy as np

from . import formats as F

HEAD_DIM = 128
TENSORS = ("q", "k", "idx_q", "idx_k")   # the normed and rotated tensors, in weight order


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x [..., 128] and w [128] float64: x / sqrt(mean(x^2) + eps) * w."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def rotary(y: np.ndarray, cos: np.ndarray, sin: np.ndarray, rd: int) -> np.ndarray:
    """Rotate-half rotary embedding of y [..., 128] over dims [0, rd) with angle
    tables cos, sin [..., rd / 2] (broadcast against y's leading axes)."""
    h = rd // 2
    out = y.copy()
    if h == 0:
        return out
    a, b = y[..., :h], y[..., h:rd]
    out[..., :h] = a * cos - b * sin
    out[..., h:rd] = b * cos + a * sin
    return out


def _tolerance(y: np.ndarray, cos: np.ndarray, sin: np.ndarray, rd: int) -> np.ndarray:
    """Bound on |float32 evaluation - exact| of every element of rotary(y).

    Before the rotation: the squares of bf16 inputs are exact in float32; a sum of
    128 positive terms in any order is within 127 * 2^-24 < 2^-17 relative; the
    mean (a power of two), the eps addition, the square root, the reciprocal or
    division and the two products add at most 6 roundings of 2^-24 (and the square
    root halves the error it is given), so y is within 2^-17.5 relative, counted
    here as 2^-16 |y|. A rotated element a c - b s adds the rounding of each
    product and of the sum: |error| <= 2^-16 (|a c| + |b s|) + 2^-23 |a c - b s|.
    """
    h = rd // 2
    tol = np.ldexp(np.abs(y), -16)
    if h:
        a, b = y[..., :h], y[..., h:rd]
        ac, bs, bc, as_ = np.abs(a * cos), np.abs(b * sin), np.abs(b * cos), np.abs(a * sin)
        tol[..., :h] = np.ldexp(ac + bs, -16) + np.ldexp(np.abs(a * cos - b * sin), -23)
        tol[..., h:rd] = np.ldexp(bc + as_, -16) + np.ldexp(np.abs(b * cos + a * sin), -23)
    return tol


def bf16_round(x: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) of the bfloat16 value nearest to each float64 x, ties to
    the even significand. Values here are far inside bf16's range; a result past
    it is refused rather than turned into an infinity."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                              # x = m 2^e, |m| in [0.5, 1)
    e = np.maximum(e, -125)                         # below 2^-126: fixed step 2^-133
    v = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)  # 8 significant bits, ties to even
    if not np.all(np.abs(v) <= 3.3895313892515355e38):
        raise ValueError("value outside the bf16 range")
    bits = v.astype(np.float32).view(np.uint32) >> 16   # v is exact in float32
    return bits.astype(np.uint16)


def e4m3_of_bf16(bits: np.ndarray) -> np.ndarray:
    """OCP E4M3FN bytes nearest to bf16 values: ties to the even code, magnitudes
    past 448 saturate to 448 (0x7E), sign bit = (value < 0)."""
    x = F.bf16_to_f64(bits)
    mids = (F.E4M3_POS[:-1] + F.E4M3_POS[1:]) / 2   # exact: <= 5 significant bits
    mag = F._nearest_even_index(np.abs(x), mids)
    return (np.where(x < 0, 0x80, 0) | mag).astype(np.uint8)


def produce(q_bits, k_bits, v_bits, iq_bits, ik_bits, w_bits, eps: float, cos_sin, positions, rd: int):
    """The fused producer's outputs for T tokens.

    q_bits uint16 [T, G, 128]; k/v/iq/ik_bits uint16 [T, 128]; w_bits uint16
    [4, 128] (weights of q, k, idx_q, idx_k); cos_sin float32 [P, rd] (cos in
    [0, rd/2), sin in [rd/2, rd)); positions int [T], each in [0, P).

    Returns {name: (exact float64, lo bits, hi bits)} for q, k, idx_q, idx_k
    (lo == hi except at a bf16 rounding boundary), and "v": v_bits unchanged.
    """
    if rd % 16 or not 0 <= rd <= HEAD_DIM:
        raise ValueError("rotary_dim must be a multiple of 16 in [0, 128]")
    pos = np.asarray(positions, dtype=np.int64)
    cs = np.asarray(cos_sin, dtype=np.float32).astype(np.float64)
    if pos.size and (pos.min() < 0 or pos.max() >= cs.shape[0]):
        raise ValueError("position outside the angle table")
    h = rd // 2
    cos, sin = cs[pos, :h], cs[pos, h:rd]            # [T, h]
    w = F.bf16_to_f64(np.asarray(w_bits, dtype=np.uint16))
    out = {"v": np.asarray(v_bits, dtype=np.uint16)}
    for name, bits, wi in (("q", q_bits, 0), ("k", k_bits, 1), ("idx_q", iq_bits, 2), ("idx_k", ik_bits, 3)):
        x = F.bf16_to_f64(np.asarray(bits, dtype=np.uint16))
        c, s = (cos[:, None, :], sin[:, None, :]) if x.ndim == 3 else (cos, sin)
        y = rms_norm(x, w[wi], eps)
        z = rotary(y, c, s, rd)
        tol = _tolerance(y, c, s, rd) + np.ldexp(np.abs(z), -40)   # + float64 evaluation here
        out[name] = (z, bf16_round(z - tol), bf16_round(z + tol))
    return out


def _le(av, an, bv, bn):
    """(value, sign) order: a <= b, with -0 below +0 (an, bn: 1 for a negative sign)."""
    return (av < bv) | ((av == bv) & (an >= bn))


def _between(lo, x, hi):
    """lo <= x <= hi element-wise, each a (value, negative-sign) pair of arrays."""
    return _le(lo[0], lo[1], x[0], x[1]) & _le(x[0], x[1], hi[0], hi[1])


def _bf16_key(bits):
    bits = np.asarray(bits, np.uint16)
    return F.bf16_to_f64(bits), (bits >> 15).astype(np.int64)


def _code_key(codes):
    codes = np.asarray(codes, np.uint8)
    return np.where(codes & 8, -1.0, 1.0) * F.E2M1_POS[codes & 7], (codes >> 3).astype(np.int64)


def _e4m3_key(b):
    b = np.asarray(b, np.uint8)
    return np.where(b & 0x80, -1.0, 1.0) * F.E4M3_POS[b & 0x7F], (b >> 7).astype(np.int64)


def bf16_matches(lo, hi, got) -> np.ndarray:
    """Element-wise: got lies between the two candidate bf16 values."""
    return _between(_bf16_key(lo), _bf16_key(got), _bf16_key(hi))


def e4m3_matches(lo, hi, got) -> np.ndarray:
    """Element-wise: got lies between the e4m3 bytes of the two candidates (the
    rounding is monotone, so these are the bytes of the values between them)."""
    return _between(_e4m3_key(e4m3_of_bf16(lo)), _e4m3_key(got), _e4m3_key(e4m3_of_bf16(hi)))


def store_matches(fmt: str, lo, hi, payload, scales) -> np.ndarray:
    """Per row: whether (payload, scales) as a kernel wrote them is the store of
    bf16 rows whose elements lie between lo and hi (uint16 [N, 128]).

    Where lo == hi for a whole group this is byte equality with the store rule.
    Elsewhere both rounding steps are monotone, so the check is by intervals:
    the scale byte must lie between the scales of the smallest and the largest
    amax the intervals allow, and, at that scale, each code between the codes of
    its interval's ends (in signed order, -0 below +0). The check is made element
    by element, so it is a slight relaxation at boundary elements (it does not
    ask that one choice of values gives the scale and every code at once).
    """
    lo = np.asarray(lo, np.uint16)
    hi = np.asarray(hi, np.uint16)
    payload = np.asarray(payload, np.uint8)
    scales = np.asarray(scales, np.uint8)
    gsz = F.NVFP4_GROUP if fmt == "nvfp4" else F.MXFP4_GROUP
    ng = F.HEAD_DIM // gsz
    lo_v, hi_v = F.bf16_to_f64(lo), F.bf16_to_f64(hi)
    if np.any(lo_v > hi_v):
        raise ValueError("lo above hi")
    # amax range: each element's smallest and largest magnitude over its interval
    mag_min = np.where((lo_v <= 0) & (hi_v >= 0), 0.0, np.minimum(np.abs(lo_v), np.abs(hi_v)))
    mag_max = np.maximum(np.abs(lo_v), np.abs(hi_v))
    a_lo = mag_min.reshape(-1, ng, gsz).max(axis=-1)
    a_hi = mag_max.reshape(-1, ng, gsz).max(axis=-1)
    # the scale bytes of those two amax values, through the store rule on a row
    # holding just that value in each group (the rule depends on amax alone)
    def scale_of(a):
        row = np.repeat(a, gsz, axis=-1)
        return F.quantize(fmt, bf16_round(row))[1]
    s_lo, s_hi = scale_of(a_lo), scale_of(a_hi)
    ok_scale = (scales >= s_lo) & (scales <= s_hi)          # both rules are monotone in amax
    # codes at the kernel's scale: the store rule applied to lo and to hi with that scale
    sval = F.E4M3_POS[scales & 0x7F] if fmt == "nvfp4" else np.ldexp(1.0, scales.astype(np.int64) - 127)
    sval = np.where((fmt == "mxfp4") & (scales == 0) & (a_hi == 0), 0.0, sval)
    c_lo = F._codes_for_scale(lo_v, sval, gsz)
    c_hi = F._codes_for_scale(hi_v, sval, gsz)
    got = F._unpack(payload)
    ok_code = _between(_code_key(c_lo), _code_key(got), _code_key(c_hi))
    return ok_scale.all(axis=-1) & ok_code.all(axis=-1)
