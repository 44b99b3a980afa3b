"""Pins of the oracle's fused producer store (per-head RMS norm, rotate-half
rotary, bf16 rounding, e4m3 query, and the boundary-aware store check) against
library routines, closed forms and simulated float32 evaluations.

Nothing here calls the HIP library. Each check is chosen so that a plausible
mistake in the oracle (the mean over the wrong axis, eps outside the root, a
swapped rotation sign, the angle table looked up by row instead of position, a
rounding tie going the wrong way, a tolerance too small for float32) fails it.
"""
import math

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import producer as P
import workloads as W


def _bits(t):
    return W.bf16_bits(t)


# --- RMS norm -----------------------------------------------------------------

def test_rms_norm_matches_torch_rms_norm():
    """torch.nn.functional.rms_norm in float64 is the library statement of
    x / sqrt(mean(x^2) + eps) * w over the last axis."""
    rng = np.random.default_rng(1)
    x = rng.normal(size=(5, 3, 128)) * rng.uniform(0.1, 10, size=(5, 3, 1))
    w = rng.normal(1.0, 0.2, size=128)
    for eps in (0.0, 1e-6, 0.5):
        want = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w), eps).numpy()
        np.testing.assert_allclose(P.rms_norm(x, w, eps), want, rtol=1e-14, atol=0)


def test_rms_norm_hand_example():
    x = np.zeros(128)
    x[0], x[1] = 3.0, 4.0            # mean(x^2) = 25 / 128
    y = P.rms_norm(x, np.ones(128), 0.0)
    assert y[0] == pytest.approx(3 * math.sqrt(128) / 5, rel=1e-15)
    assert y[1] == pytest.approx(4 * math.sqrt(128) / 5, rel=1e-15)
    assert np.all(y[2:] == 0)
    y = P.rms_norm(x, np.full(128, 2.0), 25 / 128)   # eps equal to the mean square halves it
    assert y[0] == pytest.approx(2 * 3 / math.sqrt(50 / 128), rel=1e-15)


def test_rms_norm_invariants():
    rng = np.random.default_rng(2)
    x = rng.normal(size=(7, 128))
    y = P.rms_norm(x, np.ones(128), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(P.rms_norm(37.5 * x, np.ones(128), 0.0), y, rtol=1e-13)


# --- rotary ---------------------------------------------------------------------

@pytest.mark.parametrize("rd", [16, 64, 128])
def test_rotary_is_complex_multiplication(rd):
    """(y_d + i y_{d+h}) (c + i s) in complex128: the rotate-half pairing."""
    rng = np.random.default_rng(rd)
    h = rd // 2
    y = rng.normal(size=(6, 128))
    th = rng.uniform(-4, 4, size=(6, h))
    c, s = np.cos(th), np.sin(th)
    z = (y[:, :h] + 1j * y[:, h:rd]) * (c + 1j * s)
    out = P.rotary(y, c, s, rd)
    np.testing.assert_allclose(out[:, :h], z.real, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(out[:, h:rd], z.imag, rtol=1e-14, atol=1e-15)
    assert np.array_equal(out[:, rd:], y[:, rd:])


def test_rotary_invariants():
    rng = np.random.default_rng(3)
    y = rng.normal(size=(4, 128))
    th = rng.uniform(-10, 10, size=(4, 32))
    out = P.rotary(y, np.cos(th), np.sin(th), 64)
    # a rotation keeps each pair's length and undoes with the opposite angle
    np.testing.assert_allclose(out[:, :32] ** 2 + out[:, 32:64] ** 2, y[:, :32] ** 2 + y[:, 32:64] ** 2, rtol=1e-13)
    back = P.rotary(out, np.cos(-th), np.sin(-th), 64)
    np.testing.assert_allclose(back, y, rtol=1e-12, atol=1e-13)
    # position 0 (angle 0) and rd = 0 change nothing
    assert np.array_equal(P.rotary(y, np.ones((4, 64)), np.zeros((4, 64)), 128), y)
    assert np.array_equal(P.rotary(y, np.zeros((4, 0)), np.zeros((4, 0)), 0), y)
    # a quarter turn maps (a, b) to (-b, a)
    q = P.rotary(y, np.zeros((4, 64)), np.ones((4, 64)), 128)
    assert np.array_equal(q[:, :64], -y[:, 64:]) and np.array_equal(q[:, 64:], y[:, :64])


# --- bf16 and e4m3 rounding -----------------------------------------------------

def test_bf16_round_hand_ties():
    one = 1.0
    cases = [
        (one, 0x3F80),
        (one + 2 ** -8, 0x3F80),            # tie between 1 and 1 + 2^-7: even significand
        (one + 3 * 2 ** -8, 0x3F82),        # tie between 1 + 2^-7 and 1 + 2^-6: even
        (one + 2 ** -8 + 2 ** -30, 0x3F81), # just past the tie
        (-(one + 2 ** -8), 0xBF80),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (2.0 ** -134, 0x0000),              # half the smallest subnormal: tie to 0
        (3 * 2.0 ** -134, 0x0002),          # 1.5 steps: tie to 2 steps
        (2.0 ** -133, 0x0001),
        (255.5, 0x4380),                    # tie between 255 (odd significand) and 256
    ]
    for v, bits in cases:
        got = int(P.bf16_round(np.array([v]))[0])
        assert got == bits, (v, hex(got), hex(bits))


def test_bf16_round_matches_torch_on_float32_values():
    """torch's float32 -> bfloat16 conversion rounds to nearest even; on values
    that float32 holds exactly it is the same rounding."""
    rng = np.random.default_rng(4)
    u = rng.integers(0, 2 ** 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.3e38)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(P.bf16_round(f.astype(np.float64)), want)


def test_e4m3_of_bf16_matches_torch_and_exact_rounding():
    """Every finite bf16 below the saturation point against torch's float8_e4m3fn
    conversion (round to nearest even), and a sample against the exact-rational
    nearest-even search over the code book."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(f) & (np.abs(f) < 464.0)
    bits, f = bits[keep], f[keep]
    want = torch.from_numpy(f.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = P.e4m3_of_bf16(bits)
    # the one difference is -0.0: torch keeps its sign bit, the rule (sign bit =
    # value < 0, as for the FP4 codes) gives +0; a negative value that rounds to
    # zero keeps its sign in both
    neg0 = bits == 0x8000
    assert got[neg0].tolist() == [0x00] and want[neg0].tolist() == [0x80]
    assert np.array_equal(got[~neg0], want[~neg0])
    tiny = np.array([0x8001, 0x3A00, 0xBA00], dtype=np.uint16)   # -tiny, 2^-11, -2^-11: round to 0
    assert P.e4m3_of_bf16(tiny).tolist() == [0x80, 0x00, 0x80]
    for b in bits[::997]:
        v = F.bf16_value(int(b))
        mag = F.round_nearest_even(abs(v), F.E4M3_TABLE)
        assert P.e4m3_of_bf16(np.array([b]))[0] == ((0x80 if v < 0 else 0) | mag)


def test_e4m3_saturates():
    vals = np.array([464.0, 500.0, 1e4, -448.0, -1e4], dtype=np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    assert P.e4m3_of_bf16(bits).tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


# --- produce() and its float32 tolerance ----------------------------------------

def _inputs(T=24, G=4, rd=64, seed=7):
    q = _bits(W.gen_prenorm_rows((T, G, 128), seed, W.PQ_FAMILY))
    k = _bits(W.gen_prenorm_rows((T, 128), seed, W.PK_FAMILY))
    v = _bits(W.gen_prenorm_rows((T, 128), seed, W.PV_FAMILY))
    iq = _bits(W.gen_prenorm_rows((T, 128), seed, W.PIQ_FAMILY))
    ik = _bits(W.gen_prenorm_rows((T, 128), seed, W.PIK_FAMILY))
    w = _bits(W.gen_norm_weights(seed))
    cs = W.rope_table(4096, rd)
    pos = np.random.default_rng(seed).integers(0, 4096, size=T)
    return q, k, v, iq, ik, w, cs, pos


def _fp32_eval(x_bits, w_bits, eps, cos, sin, rd, order):
    """One float32 evaluation of the producer formula in numpy; `order` picks the
    summation order of the squares and the association of the products."""
    x = F.bf16_to_f64(x_bits).astype(np.float32)
    w = F.bf16_to_f64(w_bits).astype(np.float32)
    sq = x * x
    if order == 0:                                  # left to right
        ss = np.zeros(x.shape[:-1], np.float32)
        for d in range(128):
            ss = (ss + sq[..., d]).astype(np.float32)
    elif order == 1:                                # pairwise tree
        t = sq
        while t.shape[-1] > 1:
            t = (t[..., 0::2] + t[..., 1::2]).astype(np.float32)
        ss = t[..., 0]
    else:                                           # right to left, in 16 lanes of 8
        lanes = np.zeros(x.shape[:-1] + (16,), np.float32)
        for e in range(7, -1, -1):
            lanes = (lanes + sq[..., e::8][..., :16]).astype(np.float32)
        ss = lanes.sum(axis=-1, dtype=np.float32)
    ms = (ss / np.float32(128)).astype(np.float32)
    r = (np.float32(1) / np.sqrt((ms + np.float32(eps)).astype(np.float32))).astype(np.float32)
    y = (x * r[..., None]).astype(np.float32) * w if order != 1 else x * (r[..., None] * w).astype(np.float32)
    y = y.astype(np.float32)
    h = rd // 2
    out = y.copy()
    c, s = cos.astype(np.float32), sin.astype(np.float32)
    if h:
        a, b = y[..., :h], y[..., h:rd]
        out[..., :h] = ((a * c).astype(np.float32) - (b * s).astype(np.float32)).astype(np.float32)
        out[..., h:rd] = ((b * c).astype(np.float32) + (a * s).astype(np.float32)).astype(np.float32)
    return P.bf16_round(out.astype(np.float64))


@pytest.mark.parametrize("rd", [0, 64, 128])
def test_tolerance_covers_float32_evaluations(rd):
    """Three float32 evaluation orders of the formula: every bf16 result lies in
    the oracle's [lo, hi], and the exact rounding is unique for nearly every element."""
    q, k, v, iq, ik, w, cs, pos = _inputs(T=64, G=4, rd=rd)
    eps = 1e-6
    out = P.produce(q, k, v, iq, ik, w, eps, cs, pos, rd)
    h = rd // 2
    cos, sin = cs[pos, :h].astype(np.float64), cs[pos, h:rd].astype(np.float64)
    n_amb = n_all = 0
    for name, x, wi in (("q", q, 0), ("k", k, 1), ("idx_q", iq, 2), ("idx_k", ik, 3)):
        z, lo, hi = out[name]
        c, s = (cos[:, None, :], sin[:, None, :]) if x.ndim == 3 else (cos, sin)
        for order in range(3):
            got = _fp32_eval(x, w[wi], eps, c, s, rd, order)
            assert P.bf16_matches(lo, hi, got).all(), (name, order)
        n_amb += int((lo != hi).sum())
        n_all += lo.size
        assert np.all(F.bf16_to_f64(lo) <= F.bf16_to_f64(hi))
    assert n_amb < 0.02 * n_all, (n_amb, n_all)


def test_produce_structure():
    """Query heads are normed and rotated like the key (same weight, same data, same
    token position gives the same row); the angle table is looked up by position;
    v passes through."""
    q, k, v, iq, ik, w, cs, pos = _inputs(T=10, G=3, rd=64)
    q2 = q.copy()
    q2[:, 1] = k
    w2 = w.copy()
    w2[0] = w[1]
    out = P.produce(q2, k, v, iq, ik, w2, 1e-6, cs, pos, 64)
    assert np.array_equal(out["q"][0][:, 1], out["k"][0])
    assert np.array_equal(out["v"], v)
    perm = np.random.default_rng(0).permutation(10)
    o2 = P.produce(q[perm], k[perm], v[perm], iq[perm], ik[perm], w, 1e-6, cs, pos[perm], 64)
    o1 = P.produce(q, k, v, iq, ik, w, 1e-6, cs, pos, 64)
    for name in P.TENSORS:
        assert np.array_equal(o2[name][0], o1[name][0][perm])
    with pytest.raises(ValueError):
        P.produce(q, k, v, iq, ik, w, 1e-6, cs, pos, 40)
    with pytest.raises(ValueError):
        P.produce(q, k, v, iq, ik, w, 1e-6, cs, pos + 4096, 64)


# --- the boundary-aware checks ------------------------------------------------------

@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_store_matches_accepts_float32_stores_and_rejects_mistakes(fmt):
    q, k, v, iq, ik, w, cs, pos = _inputs(T=64, G=2, rd=128)
    out = P.produce(q, k, v, iq, ik, w, 1e-6, cs, pos, 128)
    z, lo, hi = out["k"]
    h = 64
    cos, sin = cs[pos, :h].astype(np.float64), cs[pos, h:].astype(np.float64)
    for order in range(3):
        got_bits = _fp32_eval(k, w[1], 1e-6, cos, sin, 128, order)
        pay, sc = F.quantize(fmt, got_bits)
        assert P.store_matches(fmt, lo, hi, pay, sc).all()
    # where the rounding is unique the check is byte equality
    pay, sc = F.quantize(fmt, lo)
    same = (lo == hi).all(axis=-1)
    assert same.any() and P.store_matches(fmt, lo, hi, pay, sc)[same].all()
    # planted mistakes: a flipped sign of a non-zero code, a scale one step off,
    # two elements swapped, the rows of two tokens exchanged
    codes = F._unpack(pay)
    r = int(np.nonzero(same)[0][0])
    j = int(np.nonzero(codes[r] & 7)[0][0])
    bad = codes.copy()
    bad[r, j] ^= 8
    assert not P.store_matches(fmt, lo, hi, F._pack(bad), sc)[r]
    bad_s = sc.copy()
    bad_s[r, 0] += 1
    assert not P.store_matches(fmt, lo, hi, pay, bad_s)[r]
    j2 = int(np.nonzero((codes[r] & 7) != (codes[r, j] & 7))[0][0])
    bad = codes.copy()
    bad[r, [j, j2]] = bad[r, [j2, j]]
    assert not P.store_matches(fmt, lo, hi, F._pack(bad), sc)[r]
    sw = np.arange(lo.shape[0])
    sw[[0, 1]] = [1, 0]
    assert not P.store_matches(fmt, lo, hi, pay[sw], sc[sw])[:2].all()


def test_query_checks_accept_and_reject():
    q, k, v, iq, ik, w, cs, pos = _inputs(T=16, G=4, rd=64)
    z, lo, hi = P.produce(q, k, v, iq, ik, w, 1e-6, cs, pos, 64)["q"]
    assert P.bf16_matches(lo, hi, lo).all() and P.bf16_matches(lo, hi, hi).all()
    assert P.e4m3_matches(lo, hi, P.e4m3_of_bf16(hi)).all()
    nz = ((lo & 0x7FFF) != 0) & ((hi & 0x7FFF) != 0)
    below = (lo.astype(np.int32) + np.where(lo & 0x8000, 1, -1)).astype(np.uint16)   # one bf16 step under lo
    above = (hi.astype(np.int32) + np.where(hi & 0x8000, -1, 1)).astype(np.uint16)   # one step over hi
    assert not P.bf16_matches(lo, hi, below)[nz].any()
    assert not P.bf16_matches(lo, hi, above)[nz].any()
    flip = P.e4m3_of_bf16(lo) ^ 0x80
    nz = (P.e4m3_of_bf16(lo) & 0x7F) != 0
    assert not P.e4m3_matches(lo, hi, flip)[nz].any()
