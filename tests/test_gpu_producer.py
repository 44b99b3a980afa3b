"""m3s_qknorm_rope_store (the fused producer store) against the oracle's producer:
query rows, e4m3 query and the stored K / V / index-K bytes, element by element.

The kernel computes the norm and the rotation in float32; a bf16 result may take
either neighbouring value only where the exact value lies within float32
evaluation error of a bf16 rounding boundary (the oracle's [lo, hi] interval).
Everywhere else the comparison is exact, and the value plane is compared byte
for byte with the oracle's store of the unchanged value rows."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import producer as P
from tests.stepcase import say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
SENT = 0xA5


def _dev_bits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _inputs(T, G, rd, seed, max_pos=4096):
    host = {
        "q": W.bf16_bits(W.gen_prenorm_rows((T, G, 128), seed, W.PQ_FAMILY)),
        "k": W.bf16_bits(W.gen_prenorm_rows((T, 128), seed, W.PK_FAMILY)),
        "v": W.bf16_bits(W.gen_prenorm_rows((T, 128), seed, W.PV_FAMILY)),
        "idx_q": W.bf16_bits(W.gen_prenorm_rows((T, 128), seed, W.PIQ_FAMILY)),
        "idx_k": W.bf16_bits(W.gen_prenorm_rows((T, 128), seed, W.PIK_FAMILY)),
        "w": W.bf16_bits(W.gen_norm_weights(seed)),
    }
    host["cs"] = W.rope_table(max_pos, rd)
    host["pos"] = np.random.default_rng(seed + 1).integers(0, max_pos, size=T).astype(np.int32)
    return host


def _run(m3s, fmt, host, slots, pages, eps=1e-6, e4m3=True, positions=None):
    T, G = host["q"].shape[:2]
    cache = m3s.Cache(fmt, pages, DEV)
    for p, s in cache.planes.values():
        p.fill_(SENT)
        s.fill_(SENT)
    q_out = torch.full((T, G, 128), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    iq_out = torch.full((T, 128), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    qe = torch.full((T, G, 128), SENT, dtype=torch.uint8, device=DEV) if e4m3 else None
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    pos = host["pos"] if positions is None else positions
    m3s.m3s_qknorm_rope_store(
        cache, _dev_bits(host["q"]), _dev_bits(host["k"]), _dev_bits(host["v"]), _dev_bits(host["idx_q"]),
        _dev_bits(host["idx_k"]), _dev_bits(host["w"]), eps,
        torch.as_tensor(pos, dtype=torch.int32, device=DEV),
        torch.as_tensor(host["cs"], device=DEV), torch.as_tensor(slots, dtype=torch.int32, device=DEV),
        q_out=q_out, idx_q_out=iq_out, q_out_e4m3=qe, dev_status=st)
    torch.cuda.synchronize()
    got = {
        "q": q_out.view(torch.int16).cpu().numpy().view(np.uint16),
        "idx_q": iq_out.view(torch.int16).cpu().numpy().view(np.uint16),
        "e4m3": None if qe is None else qe.cpu().numpy(),
        "status": int(st.item()),
    }
    for name, (p, s) in cache.planes.items():
        got[name] = (p.cpu().numpy().reshape(-1, 64), s.cpu().numpy().reshape(pages * 128, -1))
    return got


def _check(fmt, host, got, slots, eps=1e-6, tokens=None):
    """Every output of the given tokens (default: all) against the oracle."""
    T = host["q"].shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    rd = host["cs"].shape[1]
    want = P.produce(host["q"], host["k"], host["v"], host["idx_q"], host["idx_k"], host["w"], eps,
                     host["cs"], host["pos"], rd)
    amb = 0
    for name in ("q", "idx_q"):
        _, lo, hi = want[name]
        ok = P.bf16_matches(lo[tokens], hi[tokens], got[name][tokens])
        assert ok.all(), (name, np.argwhere(~ok)[:5])
        amb += int((lo != hi).sum())
    if got["e4m3"] is not None:
        _, lo, hi = want["q"]
        assert P.e4m3_matches(lo[tokens], hi[tokens], got["e4m3"][tokens]).all()
    live = tokens[np.asarray(slots)[tokens] >= 0]
    sl = np.asarray(slots)[live]
    for name, plane in (("k", "k"), ("idx_k", "idx")):
        _, lo, hi = want[name]
        pay, sc = got[plane]
        ok = P.store_matches(fmt, lo[live], hi[live], pay[sl], sc[sl])
        assert ok.all(), (name, live[~ok][:5])
    pay, sc = got["v"]
    wp, ws = F.quantize(fmt, host["v"][live])
    assert np.array_equal(pay[sl], wp) and np.array_equal(sc[sl], ws)
    return amb


def _untouched(got, pages, used):
    """Slots outside `used` still hold the fill pattern in every plane."""
    mask = np.ones(pages * 128, bool)
    mask[np.asarray(used, dtype=np.int64)] = False
    for name in ("k", "v", "idx"):
        pay, sc = got[name]
        assert (pay[mask] == SENT).all() and (sc[mask] == SENT).all(), name


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("T,G,rd,pad_every", [(64, 16, 128, 0), (37, 4, 64, 5), (5, 1, 0, 0), (130, 2, 16, 7)])
def test_producer_parity(gpu, fmt, T, G, rd, pad_every):
    """Query rows, e4m3 query, K / V / index-K bytes of every token; pad tokens
    (slot -1) write no cache bytes; slots nobody owns stay untouched."""
    seed = 11 + T + G + rd
    say(f"[producer] fmt={fmt} T={T} G={G} rd={rd} pad_every={pad_every}")
    host = _inputs(T, G, rd, seed)
    pages = (T + 127) // 128 + 2
    slots = np.random.default_rng(seed).permutation(pages * 128)[:T].astype(np.int32)
    if pad_every:
        slots[::pad_every] = -1
    got = _run(gpu, fmt, host, slots, pages)
    assert got["status"] == 0, hex(got["status"])
    amb = _check(fmt, host, got, slots)
    say(f"[producer]   boundary elements {amb}")
    _untouched(got, pages, slots[slots >= 0])


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_producer_equals_unfused_store(gpu, fmt):
    """The fused store writes the bytes that m3s_store writes for the kernel's own bf16
    rows: feed the key as the index query with the key's weight, so idx_q_out is the
    key row the kernel quantized, and store that row with m3s_store."""
    T, G, rd = 48, 2, 64
    host = _inputs(T, G, rd, 5)
    host["idx_q"] = host["k"].copy()
    host["w"] = host["w"].copy()
    host["w"][2] = host["w"][1]
    pages = 1
    slots = np.arange(T, dtype=np.int32)
    got = _run(gpu, fmt, host, slots, pages, e4m3=False)
    assert got["status"] == 0
    cache = gpu.Cache(fmt, pages, DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    row = _dev_bits(got["idx_q"])
    gpu.m3s_store(cache, row, None, None, torch.as_tensor(slots, device=DEV), st)
    torch.cuda.synchronize()
    p, s = cache.planes["k"]
    assert int(st.item()) == 0
    assert np.array_equal(p.cpu().numpy().reshape(-1, 64)[:T], got["k"][0][:T])
    assert np.array_equal(s.cpu().numpy().reshape(128, -1)[:T], got["k"][1][:T])


def test_producer_bad_position_and_slot(gpu):
    """A position outside the angle table sets BAD_POSITION and that token writes
    nothing; a slot past the cache sets BAD_SLOT, writes no cache bytes, and still
    writes the token's queries; every other token is exact."""
    fmt, T, G, rd = "nvfp4", 20, 4, 32
    host = _inputs(T, G, rd, 9, max_pos=64)
    pages = 1
    slots = np.arange(T, dtype=np.int32) + 3
    slots[7] = pages * 128 + 5                     # past the cache
    pos = host["pos"].copy()
    pos[4] = 64                                    # == max_pos: outside the table
    pos[11] = -1
    got = _run(gpu, fmt, host, slots, pages, positions=pos)
    bits = gpu.DEV_BITS
    assert got["status"] == bits["BAD_POSITION"] | bits["BAD_SLOT"], hex(got["status"])
    for t in (4, 11):
        assert (got["q"][t] == 0xFFFF).all() and (got["idx_q"][t] == 0xFFFF).all()
        assert (got["e4m3"][t] == SENT).all()
    good = np.array([t for t in range(T) if t not in (4, 11)])
    slots_ok = slots.copy()
    slots_ok[7] = -1                               # its queries are checked, its cache bytes are not written
    _check(fmt, host, got, slots_ok, tokens=good)
    _untouched(got, pages, slots_ok[good][slots_ok[good] >= 0])


def test_producer_no_tokens(gpu):
    fmt = "mxfp4"
    cache = gpu.Cache(fmt, 1, DEV)
    z = torch.zeros((0, 128), dtype=torch.bfloat16, device=DEV)
    q, iq, qe = gpu.m3s_qknorm_rope_store(
        cache, torch.zeros((0, 2, 128), dtype=torch.bfloat16, device=DEV), z, z, z, z,
        torch.ones((4, 128), dtype=torch.bfloat16, device=DEV), 1e-6,
        torch.zeros(0, dtype=torch.int32, device=DEV), torch.zeros((8, 64), dtype=torch.float32, device=DEV),
        torch.zeros(0, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert q.shape == (0, 2, 128) and iq.shape == (0, 128) and qe is None
