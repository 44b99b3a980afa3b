"""m3s_decode_rows parity: row map and block prefix bit-exact against the oracle."""
import numpy as np
import pytest
import torch

from oracle import path as P

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _run(m3s, cu_q, seq, R):
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    rows = m3s.m3s_decode_rows(torch.as_tensor(np.asarray(cu_q, np.int32), device=DEV),
                               torch.as_tensor(np.asarray(seq, np.int32), device=DEV), R, dev_status=st)
    torch.cuda.synchronize()
    return rows.row_req.cpu().numpy(), rows.row_len.cpu().numpy(), rows.grp_blk.cpu().numpy(), int(st.item())


def test_rows_random_batches(gpu):
    rng = np.random.default_rng(8)
    for B in (1, 3, 8, 48, 1023, 1024, 1025, 3000, 4096):
        ql = rng.integers(1, 17, size=B)
        seq = ql + rng.integers(0, 500_000, size=B)
        cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
        R = min(65536, int(cu[-1]) + int(rng.integers(0, 40)))
        if cu[-1] > R:
            continue
        rr, rl, rb, st = _run(gpu, cu, seq, R)
        wr, wl = P.decode_rows(cu, seq, R)
        assert st == 0
        assert np.array_equal(rr, wr) and np.array_equal(rl, wl), B
        nb = (seq + 127) // 128
        assert np.array_equal(rb, np.concatenate([[0], np.cumsum(nb)])), B


def test_rows_reject_bad_requests(gpu):
    # request 1 has q_len 0, request 2 has q_len 17, request 3 has seq_len < q_len
    cu = [0, 2, 2, 19, 23, 24]
    seq = [100, 50, 4000, 3, 10]
    rr, rl, rb, st = _run(gpu, cu, seq, 30)
    assert st & gpu.DEV_BITS["BAD_ROWS"]
    assert rr[:2].tolist() == [0, 0] and rl[:2].tolist() == [99, 100]
    assert np.all(rr[2:23] == -1) and np.all(rl[2:23] == 0)       # rejected requests -> pad rows
    assert rr[23] == 4 and rl[23] == 10
    assert np.all(rr[24:] == -1)
    assert rb.tolist() == [0, 1, 1, 1, 1, 2]                       # rejected requests own no blocks


def test_rows_empty_batch(gpu):
    rr, rl, rb, st = _run(gpu, [0], np.zeros(0, np.int32), 5)
    assert st == 0 and np.all(rr == -1) and np.all(rl == 0) and rb.tolist() == [0]


def _prefill(m3s, cu_q, seq, R, max_groups=None):
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    rows = m3s.m3s_prefill_rows(torch.as_tensor(np.asarray(cu_q, np.int32), device=DEV),
                                torch.as_tensor(np.asarray(seq, np.int32), device=DEV), R, max_groups, dev_status=st)
    torch.cuda.synchronize()
    g = lambda t: t.cpu().numpy()
    return g(rows.row_req), g(rows.row_len), g(rows.grp_row), g(rows.grp_req), g(rows.grp_blk), int(st.item())


def _check_groups(cu, seq, rl, gr, gq, gb, group_rows=64):
    """Work groups: consecutive runs of at most 64 rows of one request, in row order,
    covering every live row once; block prefix = causal blocks of each group's last row."""
    G = len(gq)
    live = [g for g in range(G) if gq[g] >= 0]
    want_rows, nb = [], []
    for b in range(len(seq)):
        for s0 in range(int(cu[b]), int(cu[b + 1]), group_rows):
            want_rows.append((s0, b))
    assert [(int(gr[g]), int(gq[g])) for g in live] == want_rows
    assert live == list(range(len(live)))                  # real groups first
    for g in range(G):
        n = int(gr[g + 1] - gr[g])
        if gq[g] >= 0:
            b = int(gq[g])
            assert 1 <= n <= group_rows and gr[g] >= cu[b] and gr[g + 1] <= cu[b + 1]
            nb.append((int(rl[gr[g + 1] - 1]) + 127) // 128 if seq[b] >= cu[b + 1] - cu[b] else 0)
        else:
            assert n == 0
            nb.append(0)
    assert np.array_equal(gb, np.concatenate([[0], np.cumsum(nb)]))


def test_prefill_rows_random_batches(gpu):
    rng = np.random.default_rng(9)
    for B, qmax in ((1, 3000), (3, 700), (8, 40), (50, 300), (200, 20)):
        ql = rng.integers(1, qmax + 1, size=B)
        seq = ql + rng.integers(0, 200_000, size=B)
        cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
        R = int(cu[-1]) + int(rng.integers(0, 40))
        if R > 65536:
            continue
        rr, rl, gr, gq, gb, st = _prefill(gpu, cu, seq, R)
        wr, wl = P.prefill_rows(cu, seq, R)
        assert st == 0
        assert np.array_equal(rr, wr) and np.array_equal(rl, wl), B
        _check_groups(cu, seq, rl, gr, gq, gb)


def test_prefill_rows_reject(gpu):
    bad_bit = gpu.DEV_BITS["BAD_ROWS"]
    # a request with seq_len < q_len: its rows are pad rows, the others are mapped
    cu, seq = [0, 40, 45, 80], [100, 3, 35]
    rr, rl, gr, gq, gb, st = _prefill(gpu, cu, seq, 80)
    assert st & bad_bit
    assert np.all(rr[40:45] == -1) and np.all(rl[40:45] == 0)
    assert rr[:40].tolist() == [0] * 40 and rl[79] == 35
    _check_groups(cu, seq, rl, gr, gq, gb)
    # a decreasing cu_q, or too few groups: every row becomes a pad row
    for cu, seq, R, G in (([0, 30, 20, 50], [30, 40, 50], 50, None), ([0, 70, 80], [70, 80], 80, 2)):
        rr, rl, gr, gq, gb, st = _prefill(gpu, cu, seq, R, G)
        assert st & bad_bit
        assert np.all(rr == -1) and np.all(rl == 0) and gb[-1] == 0 and np.all(gq == -1)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_store_and_rows_equals_separate_calls(gpu, fmt):
    """One launch for store + row map writes what the two separate calls write, status
    bits included (a slot past the cache and a rejected request)."""
    rng = np.random.default_rng(12)
    T, P = 300, 8
    g = torch.Generator(device="cpu").manual_seed(3)
    x = (torch.randn((3, T, 128), generator=g) * 3).to(torch.bfloat16).to(DEV)
    slots = torch.as_tensor(rng.permutation(P * 128)[:T].astype(np.int32), device=DEV)
    slots[7] = P * 128 + 5   # bad slot
    slots[9] = -1            # pad row
    ql = rng.integers(1, 17, size=40)
    ql[3] = 20               # rejected request
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(ql)]).astype(np.int32), device=DEV)
    seq = torch.as_tensor((ql + rng.integers(0, 9000, size=40)).astype(np.int32), device=DEV)
    R = int(cu[-1].item()) + 5
    outs = []
    for fused in (False, True):
        c = gpu.Cache(fmt, P, DEV)
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        rr = torch.full((R,), 77, dtype=torch.int32, device=DEV)
        rl = torch.full((R,), 77, dtype=torch.int32, device=DEV)
        rb = torch.full((41,), 77, dtype=torch.int32, device=DEV)
        if fused:
            gpu.m3s_store_and_rows(c, x[0], x[1], x[2], slots, cu, seq, R, rr, rl, rb, st)
        else:
            gpu.m3s_store(c, x[0], x[1], x[2], slots, st)
            gpu.m3s_decode_rows(cu, seq, R, rr, rl, rb, st)
        torch.cuda.synchronize()
        outs.append(([t.cpu() for pl in c.planes.values() for t in pl], rr.cpu(), rl.cpu(), rb.cpu(), int(st.item())))
    (pa, ra, la, ba, sa), (pb, rb_, lb, bb, sb) = outs
    assert all(torch.equal(u, w) for u, w in zip(pa, pb))
    assert torch.equal(ra, rb_) and torch.equal(la, lb) and torch.equal(ba, bb)
    assert sa == sb and sa & gpu.DEV_BITS["BAD_SLOT"] and sa & gpu.DEV_BITS["BAD_ROWS"]


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_store_and_prefill_rows_equals_separate_calls(gpu, fmt):
    """One launch for store + prefill row map writes what m3s_store and m3s_prefill_rows
    write, status bits included (a slot past the cache; chunks of 300, 1, 64, 65 and 700
    rows, one request with fewer tokens than rows)."""
    rng = np.random.default_rng(21)
    ql = np.array([300, 1, 64, 65, 700], dtype=np.int64)
    seq_np = ql + rng.integers(0, 9000, size=len(ql))
    seq_np[1] = 0            # fewer tokens than rows: rejected
    T, P = int(ql.sum()), 16
    g = torch.Generator(device="cpu").manual_seed(4)
    x = (torch.randn((3, T, 128), generator=g) * 3).to(torch.bfloat16).to(DEV)
    slots = torch.as_tensor(rng.permutation(P * 128)[:T].astype(np.int32), device=DEV)
    slots[11] = P * 128 + 3  # bad slot
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(ql)]).astype(np.int32), device=DEV)
    seq = torch.as_tensor(seq_np.astype(np.int32), device=DEV)
    R = T + 7
    outs = []
    for fused in (False, True):
        c = gpu.Cache(fmt, P, DEV)
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        if fused:
            rows = gpu.m3s_store_and_prefill_rows(c, x[0], x[1], x[2], slots, cu, seq, R, dev_status=st)
        else:
            gpu.m3s_store(c, x[0], x[1], x[2], slots, st)
            rows = gpu.m3s_prefill_rows(cu, seq, R, dev_status=st)
        torch.cuda.synchronize()
        outs.append(([t.cpu() for pl in c.planes.values() for t in pl],
                     [t.cpu() for t in (rows.row_req, rows.row_len, rows.grp_row, rows.grp_req, rows.grp_blk)],
                     int(st.item())))
    (pa, ra, sa), (pb, rb_, sb) = outs
    assert all(torch.equal(u, w) for u, w in zip(pa, pb))
    assert all(torch.equal(u, w) for u, w in zip(ra, rb_))
    assert sa == sb and sa & gpu.DEV_BITS["BAD_SLOT"] and sa & gpu.DEV_BITS["BAD_ROWS"]

