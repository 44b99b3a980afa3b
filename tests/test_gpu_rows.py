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
    return rows.row_req.cpu().numpy(), rows.row_len.cpu().numpy(), rows.req_blk.cpu().numpy(), int(st.item())


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
