"""NVFP4 and MXFP4 row formats: code books, quantization, dequantization.

Test infrastructure (see the package docstring): only the tests, the smoke
check and bench.py's CPU baseline may import this module.

Two statements of every rule live here:
  * scalar, exact-rational versions (``fractions.Fraction``) written straight
    from the format definitions: a value is rounded to the nearest member of
    the finite code book, ties to the even code, anything past the largest
    member clamps to it (saturation);
  * vectorized float64 versions of the same rules, used on real batches.
    They decide every rounding by comparing against exact midpoints (every
    product and midpoint involved has at most 8 significant bits, so float64
    holds it exactly) and are pinned to the scalar versions and to an
    independent integer computation by the tests.

Row format (ATOM PR "[MiniMax-M3.1] FP4 index cache and NVFP4 sparse KV
cache", Design / Write path; ATOM PR "NVFP4 sparse KV", Summary):
  NVFP4: 128 elements -> 8 groups of 16; per group scale = e4m3(amax / 6)
         (OCP E4M3FN, round to nearest even, saturating at 448); codes are
         e2m1, round half to even, saturating at 6. 64 B payload + 8 B scales.
  MXFP4 (same PR, Follow-up: MXFP4 caches; vLLM PR "MXFP4 KV + indexer cache
         for MiniMax-M3.1", Claims): 4 groups of 32, one E8M0 scale each,
         64 B payload + 4 B scales = 68 B. The pages give no scale rule; the
         OCP MX v1.0 rule is taken: X = 2^(floor(log2 amax) - 2), clamped to
         the E8M0 range, codes = RNE-saturating e2m1 of x / X.
Packing (reading of the kernels' loads of even and odd elements): byte j of the payload holds
element 2j in its low nibble and element 2j+1 in its high nibble; scale
byte g covers elements [16 g, 16 g + 16) (NVFP4) or [32 g, 32 g + 32) (MXFP4).
Sign bit of a code = (x < 0): -0.0 gives 0x0, a small negative that rounds to
magnitude 0 keeps its sign bit (0x8).
"""
from __future__ import annotations

import struct
from fractions import Fraction as Fr

import numpy as np

HEAD_DIM = 128
NVFP4_GROUP = 16
MXFP4_GROUP = 32
PAYLOAD_BYTES = HEAD_DIM // 2                 # 64
NVFP4_SCALE_BYTES = HEAD_DIM // NVFP4_GROUP   # 8
MXFP4_SCALE_BYTES = HEAD_DIM // MXFP4_GROUP   # 4


def scale_bytes(fmt: str) -> int:
    return {"nvfp4": NVFP4_SCALE_BYTES, "mxfp4": MXFP4_SCALE_BYTES}[fmt]


def row_bytes(fmt: str) -> int:
    """Bytes per token and head: 72 (NVFP4) or 68 (MXFP4)."""
    return PAYLOAD_BYTES + scale_bytes(fmt)


# ---------------------------------------------------------------------------
# code books, from the bit-level definitions
# ---------------------------------------------------------------------------

def e2m1_value(code: int) -> Fr:
    """FP4 E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.

    Exponent field 0 is subnormal (m * 2^-1); otherwise (1 + m/2) * 2^(e-1).
    """
    sign = -1 if code & 0x8 else 1
    e = (code >> 1) & 0x3
    m = code & 0x1
    mag = Fr(m, 2) if e == 0 else (1 + Fr(m, 2)) * Fr(2) ** (e - 1)
    return sign * mag


def e4m3fn_value(byte: int):
    """OCP FP8 E4M3FN: bit 7 sign, 4 exponent bits (bias 7), 3 mantissa bits.

    Exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN (returned as
    None); there is no infinity, so the largest finite magnitude is 448.
    """
    if byte & 0x7F == 0x7F:
        return None
    sign = -1 if byte & 0x80 else 1
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    mag = Fr(m, 8) * Fr(1, 2 ** 6) if e == 0 else (1 + Fr(m, 8)) * Fr(2) ** (e - 7)
    return sign * mag


def e8m0_value(byte: int):
    """OCP E8M0: 2^(byte - 127); 0xFF is NaN (None)."""
    if byte == 0xFF:
        return None
    return Fr(2) ** (byte - 127)


def bf16_value(bits: int):
    """Exact value of a bfloat16 bit pattern (None for Inf / NaN)."""
    f = struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]
    if f != f or f in (float("inf"), float("-inf")):
        return None
    return Fr(f)


E2M1_TABLE = [(e2m1_value(c), c) for c in range(8)]            # non-negative codes
E4M3_TABLE = [(e4m3fn_value(b), b) for b in range(0x7F)]        # 0x00 .. 0x7E


def round_nearest_even(v: Fr, table) -> int:
    """Code of the member of ``table`` nearest to ``v``; ties go to the even
    code; values past the largest member clamp to it."""
    best_d = None
    cands = []
    for val, code in table:
        d = abs(v - val)
        if best_d is None or d < best_d:
            best_d, cands = d, [code]
        elif d == best_d:
            cands.append(code)
    if len(cands) == 1:
        return cands[0]
    even = [c for c in cands if c % 2 == 0]
    return even[0]


def quantize_nvfp4_group_exact(values):
    """One 16-element NVFP4 group from exact values -> (scale byte, 16 codes)."""
    amax = max(abs(x) for x in values)
    sbyte = round_nearest_even(amax / 6, E4M3_TABLE)
    s = e4m3fn_value(sbyte)
    codes = []
    for x in values:
        mag = 0 if s == 0 else round_nearest_even(abs(x) / s, E2M1_TABLE)
        codes.append((0x8 if x < 0 else 0) | mag)
    return sbyte, codes


def floor_log2(x: Fr) -> int:
    """Exact floor(log2 x) of a positive rational."""
    e = x.numerator.bit_length() - x.denominator.bit_length()
    while Fr(2) ** e > x:
        e -= 1
    while Fr(2) ** (e + 1) <= x:
        e += 1
    return e


def quantize_mxfp4_group_exact(values):
    """One 32-element MXFP4 group from exact values -> (E8M0 byte, 32 codes)."""
    amax = max(abs(x) for x in values)
    if amax == 0:
        return 0, [0] * len(values)
    e = floor_log2(amax) - 2          # 2 = largest exponent of e2m1 (6 = 1.5 * 2^2)
    byte = min(max(e + 127, 0), 254)
    s = e8m0_value(byte)
    codes = [(0x8 if x < 0 else 0) | round_nearest_even(abs(x) / s, E2M1_TABLE) for x in values]
    return byte, codes


def pack_codes(codes):
    """Element 2j -> low nibble of byte j, element 2j+1 -> high nibble."""
    return bytes((codes[2 * j] & 0xF) | ((codes[2 * j + 1] & 0xF) << 4) for j in range(len(codes) // 2))


def quantize_row_exact(fmt: str, bits):
    """Scalar exact quantization of one 128-element bf16 row -> (payload bytes, scale bytes)."""
    vals = [bf16_value(int(b)) for b in bits]
    if any(v is None for v in vals):
        raise ValueError("NaN / Inf input is outside the format's domain")
    gsz = NVFP4_GROUP if fmt == "nvfp4" else MXFP4_GROUP
    qfn = quantize_nvfp4_group_exact if fmt == "nvfp4" else quantize_mxfp4_group_exact
    scales, codes = [], []
    for g in range(0, HEAD_DIM, gsz):
        sb, cs = qfn(vals[g: g + gsz])
        scales.append(sb)
        codes += cs
    return pack_codes(codes), bytes(scales)


# ---------------------------------------------------------------------------
# vectorized float64 versions
# ---------------------------------------------------------------------------

E2M1_POS = np.array([float(v) for v, _ in E2M1_TABLE])          # 0 .5 1 1.5 2 3 4 6
E4M3_POS = np.array([float(v) for v, _ in E4M3_TABLE])          # bytes 0x00 .. 0x7E
E2M1_MIDS = (E2M1_POS[:-1] + E2M1_POS[1:]) / 2                  # .25 .75 1.25 1.75 2.5 3.5 5


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16)
    f = u.view(np.float32).astype(np.float64)
    if not np.all(np.isfinite(f)):
        raise ValueError("NaN / Inf input is outside the format's domain")
    return f


def _nearest_even_index(x: np.ndarray, mids: np.ndarray) -> np.ndarray:
    """Index of the nearest table entry given the table's exact midpoints.

    ``x`` and ``mids`` broadcast on all but the last axis of ``mids``; the
    number of midpoints strictly below x is the nearest index; x equal to a
    midpoint is a tie and goes to the even index.
    """
    below = (mids < x[..., None]).sum(axis=-1)
    n = mids.shape[-1]
    at = np.take_along_axis(mids, np.minimum(below, n - 1)[..., None], axis=-1)[..., 0] \
        if mids.ndim == x.ndim + 1 else mids[np.minimum(below, n - 1)]
    tie = (below < n) & (x == at)
    return np.where(tie & (below % 2 == 1), below + 1, below)


def _codes_for_scale(xf: np.ndarray, s: np.ndarray, gsz: int) -> np.ndarray:
    """e2m1 codes of xf [..., 128] given per-group scales s [..., 128/gsz]."""
    sh = xf.shape[:-1] + (HEAD_DIM // gsz, gsz)
    xg = xf.reshape(sh)
    sg = s[..., None]
    mids = sg[..., None] * E2M1_MIDS             # [..., groups, 1, 7] exact products
    mids = np.broadcast_to(mids, sh + (7,))
    mag = _nearest_even_index(np.abs(xg), mids)
    mag = np.where(sg == 0, 0, mag)
    sign = np.where(xg < 0, 8, 0)
    return (sign | mag).astype(np.uint8).reshape(xf.shape)


def _pack(codes: np.ndarray) -> np.ndarray:
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def quantize_nvfp4(bits: np.ndarray):
    """bf16 bits [..., 128] -> (payload uint8 [..., 64], scales uint8 [..., 8])."""
    xf = bf16_to_f64(bits)
    amax = np.abs(xf.reshape(xf.shape[:-1] + (8, 16))).max(axis=-1)
    six_e = 6.0 * E4M3_POS                          # exact (<= 6 significant bits)
    sidx = _nearest_even_index(amax, (six_e[:-1] + six_e[1:]) / 2)
    s = E4M3_POS[sidx]
    codes = _codes_for_scale(xf, s, NVFP4_GROUP)
    return _pack(codes), sidx.astype(np.uint8)


def quantize_mxfp4(bits: np.ndarray):
    """bf16 bits [..., 128] -> (payload uint8 [..., 64], E8M0 scales uint8 [..., 4])."""
    xf = bf16_to_f64(bits)
    amax = np.abs(xf.reshape(xf.shape[:-1] + (4, 32))).max(axis=-1)
    _, ex = np.frexp(amax)                           # amax = m * 2^ex, m in [0.5, 1)
    e = ex.astype(np.int64) - 1 - 2                  # floor(log2 amax) - 2
    byte = np.clip(e + 127, 0, 254)
    byte = np.where(amax == 0, 0, byte)
    s = np.ldexp(1.0, (byte - 127).astype(np.int64))
    codes = _codes_for_scale(xf, s, MXFP4_GROUP)
    codes = np.where(np.repeat(amax == 0, 32, axis=-1), 0, codes).astype(np.uint8)
    return _pack(codes), byte.astype(np.uint8)


def quantize(fmt: str, bits: np.ndarray):
    return quantize_nvfp4(bits) if fmt == "nvfp4" else quantize_mxfp4(bits)


def _unpack(payload: np.ndarray) -> np.ndarray:
    p = np.asarray(payload, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def code_values(payload: np.ndarray) -> np.ndarray:
    c = _unpack(payload)
    return np.where(c & 8, -1.0, 1.0) * E2M1_POS[c & 7]


def dequantize_nvfp4(payload: np.ndarray, scales: np.ndarray) -> np.ndarray:
    sb = np.asarray(scales, dtype=np.uint8)
    if np.any((sb & 0x7F) == 0x7F):
        raise ValueError("NaN scale byte")
    s = np.where(sb & 0x80, -1.0, 1.0) * E4M3_POS[sb & 0x7F]
    return code_values(payload) * np.repeat(s, NVFP4_GROUP, axis=-1)


def dequantize_mxfp4(payload: np.ndarray, scales: np.ndarray) -> np.ndarray:
    sb = np.asarray(scales, dtype=np.uint8)
    if np.any(sb == 0xFF):
        raise ValueError("NaN scale byte")
    s = np.ldexp(1.0, sb.astype(np.int64) - 127)
    return code_values(payload) * np.repeat(s, MXFP4_GROUP, axis=-1)


def dequantize(fmt: str, payload, scales) -> np.ndarray:
    return dequantize_nvfp4(payload, scales) if fmt == "nvfp4" else dequantize_mxfp4(payload, scales)
