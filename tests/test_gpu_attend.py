"""m3s_sparse_attend parity: outputs within 5e-3 max relative error of the oracle (fed
the oracle's own top-k ids, so attention is checked independently of the index)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import path as P
from tests.stepcase import max_rel_err, oracle_requests, run_gpu_step

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
CFG0 = W.config(0)
TOL = 5e-3


def _attend(gpu, step, ids_np, sm_scale, q=None):
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    lay = step.case.layout
    q = step.case.q if q is None else q
    R = step.rows.num_rows
    if R > q.shape[0]:
        q = torch.cat([q, torch.zeros((R - q.shape[0],) + tuple(q.shape[1:]), dtype=q.dtype, device=DEV)])
    ids = torch.as_tensor(np.ascontiguousarray(ids_np, dtype=np.int32), device=DEV)
    out = gpu.m3s_sparse_attend(step.cache, q, step.bt, lay.max_blocks, step.rows, ids, sm_scale, dev_status=st)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), int(st.item())


def _oracle_ids_matrix(want_ids, R, k):
    m = np.full((R, k), -1, np.int32)
    for r, v in want_ids.items():
        m[r] = v
    return m


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("G,topk", [(1, 1), (4, 4), (16, 5), (16, 16), (2, 64)])
def test_attend_small_ragged(gpu, fmt, G, topk):
    seq = [2048, 5000, 300, 129, 128, 127, 17, 9000]
    step = run_gpu_step(gpu, CFG0, DEV, seq_lens=seq, q_len=3, G=G, topk=topk, fmt=fmt, sm_scale=0.37)
    assert step.status == 0
    ids, outs, _, _ = oracle_requests(step, fmt, topk, 0.37, range(len(seq)))
    got, st = _attend(gpu, step, _oracle_ids_matrix(ids, step.rows.num_rows, topk), 0.37)
    assert st == 0
    for r, want in outs.items():
        e = max_rel_err(got[r], want)
        assert e <= TOL, (r, e)


def test_attend_pad_rows_are_zero_and_id_order_does_not_matter(gpu):
    seq = [3000, 700]
    step = run_gpu_step(gpu, CFG0, DEV, seq_lens=seq, q_len=2, G=16, topk=16, num_rows=7)
    ids, outs, _, _ = oracle_requests(step, "nvfp4", 16, 1.0, range(2))
    m = _oracle_ids_matrix(ids, 7, 16)
    a, st = _attend(gpu, step, m, 1.0)
    assert st == 0
    assert np.all(a[4:] == 0)
    rng = np.random.default_rng(1)
    m2 = m.copy()
    for r in range(4):
        m2[r] = m2[r][rng.permutation(16)]
    b, _ = _attend(gpu, step, m2, 1.0)
    for r in range(4):
        assert max_rel_err(a[r], outs[r]) <= TOL
        assert max_rel_err(b[r], a[r]) <= 1e-5


def test_attend_single_token_row_and_zero_query(gpu):
    case = W.make_case(CFG0, DEV, seq_lens=[1, 600], q_len=1, G=4)
    case.q[1] = 0
    step = run_gpu_step(gpu, CFG0, DEV, topk=4, case=case)
    ids, outs, _, rl = oracle_requests(step, "nvfp4", 4, 1.0, range(2))
    got, st = _attend(gpu, step, _oracle_ids_matrix(ids, 2, 4), 1.0)
    assert st == 0
    vh0 = F.dequantize("nvfp4", *F.quantize("nvfp4", W.bf16_bits(case.v[:1])))[0]
    assert np.allclose(got[0], vh0[None], rtol=1e-6, atol=1e-6)      # one token: out = v0
    lay = case.layout
    toks = P.selected_tokens(ids[1], int(rl[1]))
    vh = F.dequantize("nvfp4", *F.quantize("nvfp4", W.bf16_bits(case.v[int(lay.tok_off[1]):int(lay.tok_off[2])])))
    assert max_rel_err(got[1], np.broadcast_to(vh[toks].mean(0), got[1].shape)) <= TOL


def test_attend_invalid_ids_are_skipped_and_flagged(gpu):
    step = run_gpu_step(gpu, CFG0, DEV, seq_lens=[3000], q_len=1, G=8, topk=8)
    nb = (3000 + 127) // 128
    good = np.array([[0, 3, 7, 11, -1, -1, -1, -1]], np.int32)
    bad = np.array([[0, 3, 7, 11, nb, 5000, -1, -1]], np.int32)
    a, st_a = _attend(gpu, step, good, 1.0)
    b, st_b = _attend(gpu, step, bad, 1.0)
    assert st_a == 0
    assert st_b & gpu.DEV_BITS["BAD_BLOCK_ID"]
    assert np.array_equal(a, b)


def test_attend_large_scale_and_wide_query_range(gpu):
    """Queries spanning a wide dynamic range and a sharp softmax."""
    case = W.make_case(CFG0, DEV, seq_lens=[2500, 900], q_len=2, G=16)
    case.q[0, :8] *= 64
    case.q[1, 8:] *= 2.0 ** -20
    step = run_gpu_step(gpu, CFG0, DEV, topk=8, case=case, sm_scale=2.0)
    ids, outs, _, _ = oracle_requests(step, "nvfp4", 8, 2.0, range(2))
    got, st = _attend(gpu, step, _oracle_ids_matrix(ids, 4, 8), 2.0)
    assert st == 0
    for r, want in outs.items():
        assert max_rel_err(got[r], want) <= TOL, r


@pytest.mark.parametrize("topk", [16, 64])
def test_attend_workspace_reuse(gpu, topk):
    """One workspace across repeated calls, first filled with junk: every call's output
    equals the call on a fresh workspace bit for bit."""
    seq = [4000, 1500, 9000]
    step = run_gpu_step(gpu, CFG0, DEV, seq_lens=seq, q_len=4, G=16, topk=topk)
    lay = step.case.layout
    ws = gpu.attend_workspace(step.rows, lay.max_blocks, topk, 16, DEV)
    ws.fill_(0x7F)
    for rep in range(3):
        out = gpu.m3s_sparse_attend(step.cache, step.case.q, step.bt, lay.max_blocks, step.rows, step.ids,
                                    step.case.cfg.sm_scale, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, step.out), rep
