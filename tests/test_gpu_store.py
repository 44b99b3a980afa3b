"""m3s_store parity: stored codes and scales bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from tests.goldens import read_groups
from tests.stepcase import say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _bits_to_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


def _store_rows(m3s, fmt, bits: np.ndarray, slots=None, pages=None, which=("k", "v", "idx")):
    T = bits.shape[0]
    pages = pages or (T + 127) // 128
    cache = m3s.Cache(fmt, pages, DEV)
    x = _bits_to_bf16(bits)
    s = torch.arange(T, dtype=torch.int32, device=DEV) if slots is None else torch.as_tensor(slots, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    m3s.m3s_store(cache, x if "k" in which else None, x if "v" in which else None,
                  x if "idx" in which else None, s.to(torch.int32), st)
    torch.cuda.synchronize()
    return cache, int(st.item())


def _planes(cache, name):
    p, s = cache.planes[name]
    return p.cpu().numpy().reshape(-1, 64), s.cpu().numpy().reshape(-1, s.shape[-1])


@pytest.mark.parametrize("fmt,fname,gsz", [("nvfp4", "nvfp4_groups.txt", 16), ("mxfp4", "mxfp4_groups.txt", 32)])
def test_store_hand_cases(gpu, fmt, fname, gsz):
    cases = read_groups(fname, gsz)
    rows = np.zeros((len(cases), 128), np.uint16)
    for i, (_, bits, _, _) in enumerate(cases):
        rows[i, gsz: 2 * gsz] = bits                     # second group of the row
    cache, st = _store_rows(gpu, fmt, rows)
    assert st == 0
    pay, sc = _planes(cache, "idx")
    for i, (name, _, scale, payload) in enumerate(cases):
        assert sc[i, 1] == scale, name
        assert np.array_equal(pay[i, gsz // 2: gsz], payload), name


def _groups_of_sorted_bf16(gsz):
    """Every finite bf16 value, sorted by magnitude and cut into groups, both signs."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    b = b[((b >> 7) & 0xFF) != 0xFF]
    mag = np.sort(b[b < 0x8000])
    out = []
    for sign in (0, 0x8000):
        v = mag | sign
        v = np.concatenate([v, np.zeros((-len(v)) % 128, np.uint16)])
        out.append(v.reshape(-1, 128))
        # same values with a neighbouring group's max spilled in (mixes ranges inside a group)
        r = np.roll(v, gsz // 2).reshape(-1, 128)
        out.append(r)
    return np.concatenate(out)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_store_exhaustive_bf16(gpu, fmt):
    """Every finite bf16 value inside groups of neighbouring magnitudes (all scales reached)."""
    rows = _groups_of_sorted_bf16(16 if fmt == "nvfp4" else 32)
    say(f"[store exhaustive] fmt={fmt} rows={rows.shape[0]}")
    cache, st = _store_rows(gpu, fmt, rows, which=("idx",))
    assert st == 0
    pay, sc = _planes(cache, "idx")
    wp, ws = F.quantize(fmt, rows)
    T = rows.shape[0]
    assert np.array_equal(sc[:T], ws)
    assert np.array_equal(pay[:T], wp)


def test_store_nvfp4_every_scale_against_every_code(gpu):
    """For every positive finite E4M3 scale s: a group [6 s, x...] fixes scale s; x runs over
    every finite bf16 with |x| <= 6 s (both signs)."""
    b = np.arange(1 << 15, dtype=np.uint32).astype(np.uint16)
    b = b[((b >> 7) & 0xFF) != 0xFF]
    xf = F.bf16_to_f64(b)
    groups = []
    for sb in range(1, 0x7F):
        amax = 6.0 * F.E4M3_POS[sb]
        anchor = np.array([amax], np.float32).view(np.uint32) >> 16
        assert F.bf16_to_f64(anchor.astype(np.uint16))[0] == amax
        vals = b[xf <= amax]
        vals = np.concatenate([vals, vals | 0x8000])
        vals = np.concatenate([vals, np.zeros((-len(vals)) % 15, np.uint16)]).reshape(-1, 15)
        g = np.concatenate([np.full((vals.shape[0], 1), anchor[0], np.uint16), vals], axis=1)
        groups.append(g)
    g = np.concatenate(groups)
    g = np.concatenate([g, np.zeros(((-g.shape[0]) % 8, 16), np.uint16)])
    rows = g.reshape(-1, 128)
    say(f"[store every scale] rows={rows.shape[0]}")
    cache, st = _store_rows(gpu, "nvfp4", rows, which=("k",))
    assert st == 0
    pay, sc = _planes(cache, "k")
    wp, ws = F.quantize("nvfp4", rows)
    T = rows.shape[0]
    assert np.array_equal(sc[:T], ws)
    assert np.array_equal(pay[:T], wp)
    # the anchor fixed the intended scale in every group
    assert set(np.unique(ws[ws != 0]).tolist()) == set(range(1, 0x7F))


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_store_random_rows_pad_rows_untouched(gpu, fmt):
    rng = np.random.default_rng(2)
    T = 3000
    x = W.bf16_bits(W.gen_rows(T, 9, 0))
    raw = rng.integers(0, 1 << 16, size=(T // 3, 128)).astype(np.uint16)
    raw = np.where(((raw >> 7) & 0xFF) == 0xFF, raw & 0x807F, raw)
    x[: T // 3] = raw
    pages = 40
    slots = rng.permutation(pages * 128)[:T].astype(np.int32)
    slots[::7] = -1                                     # pad rows
    cache = gpu.Cache(fmt, pages, DEV)
    for name in ("k", "v", "idx"):
        cache.planes[name][0].fill_(0xAB)
        cache.planes[name][1].fill_(0xCD)
    xt = _bits_to_bf16(x)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    gpu.m3s_store(cache, xt, xt, xt, torch.as_tensor(slots, device=DEV), st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    wp, ws = F.quantize(fmt, x)
    live = slots >= 0
    for name in ("k", "v", "idx"):
        pay, sc = _planes(cache, name)
        assert np.array_equal(pay[slots[live]], wp[live]), name
        assert np.array_equal(sc[slots[live]], ws[live]), name
        untouched = np.ones(pages * 128, bool)
        untouched[slots[live]] = False
        assert np.all(pay[untouched] == 0xAB) and np.all(sc[untouched] == 0xCD), name


def test_kv_store_equals_index_store(gpu):
    """The same rows stored as K, as V and as index K give identical planes (ATOM PR
    "NVFP4 sparse KV", Tests)."""
    x = W.bf16_bits(W.gen_rows(512, 4, 1))
    cache, st = _store_rows(gpu, "nvfp4", x)
    assert st == 0
    k = _planes(cache, "k")
    for name in ("v", "idx"):
        o = _planes(cache, name)
        assert np.array_equal(k[0], o[0]) and np.array_equal(k[1], o[1])


def test_store_strided_rows_and_partial_tensors(gpu):
    """Rows with a stride > 128 (e.g. a slice of a fused qkv buffer); only idx stored."""
    x = W.gen_rows(256, 5, 2, DEV)
    buf = torch.zeros((256, 384), dtype=torch.bfloat16, device=DEV)
    buf[:, 128:256] = x
    cache = gpu.Cache("nvfp4", 2, DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    gpu.m3s_store(cache, None, None, buf[:, 128:256], torch.arange(256, dtype=torch.int32, device=DEV), st)
    torch.cuda.synchronize()
    wp, ws = F.quantize("nvfp4", W.bf16_bits(x))
    pay, sc = _planes(cache, "idx")
    assert np.array_equal(pay, wp) and np.array_equal(sc, ws)
    assert int(cache.planes["k"][0].abs().sum().item()) == 0


def test_store_out_of_range_slot_sets_status_and_writes_nothing(gpu):
    x = _bits_to_bf16(W.bf16_bits(W.gen_rows(4, 1, 0)))
    cache = gpu.Cache("nvfp4", 1, DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    gpu.m3s_store(cache, x, x, x, torch.tensor([0, 128, 5000, -1], dtype=torch.int32, device=DEV), st)
    torch.cuda.synchronize()
    assert int(st.item()) & gpu.DEV_BITS["BAD_SLOT"]
    pay, _ = _planes(cache, "k")
    assert np.all(pay[1:] == 0)
