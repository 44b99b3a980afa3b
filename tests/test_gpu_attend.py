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
@pytest.mark.parametrize("G,topk", [(1, 1), (4, 4), (16, 5), (16, 16), (2, 64), (3, 16), (12, 7)])
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


def _many_row_case(topk, G, seed_shift=0):
    """Enough short requests of 8 rows that rows x splits exceed four times the CU count:
    the attention's split kernel then takes four blocks per wave (k >= 13), or two (k <= 12),
    with an online softmax across them, and a quarter or half of the splits."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nsplit = (topk + 3) // 4
    rows_needed = 4 * cus // nsplit + 1
    lens = [300, 2048, 5000, 129, 9000, 700, 3333, 1280]
    nreq = (rows_needed + 7) // 8 + 1
    seq = [lens[(i + seed_shift) % len(lens)] + 17 * i for i in range(nreq)]
    return W.make_case(CFG0, DEV, seq_lens=seq, q_len=8, G=G), nsplit, cus


@pytest.mark.parametrize("fmt,topk", [("nvfp4", 5), ("nvfp4", 12), ("mxfp4", 12), ("nvfp4", 16), ("nvfp4", 20),
                                      ("nvfp4", 64), ("mxfp4", 16)])
def test_attend_two_blocks_per_wave(gpu, fmt, topk):
    """Many rows (two blocks per attention wave for k = 5 and 12, four for 16, 20 and 64)
    against the oracle, including top-k values whose last split leaves block slots empty
    (5, 12, 20), a top-k of 16 in one split (no combine), and a 64 in four splits with their
    combine."""
    case, nsplit, cus = _many_row_case(topk, 16)
    step = run_gpu_step(gpu, CFG0, DEV, topk=topk, fmt=fmt, case=case, sm_scale=0.37)
    R = step.rows.num_rows
    assert R * nsplit > 4 * cus
    assert step.status == 0
    ids, outs, _, _ = oracle_requests(step, fmt, topk, 0.37, range(len(case.layout.seq_lens)))
    got, st = _attend(gpu, step, _oracle_ids_matrix(ids, R, topk), 0.37)
    assert st == 0
    worst = max(max_rel_err(got[r], want) for r, want in outs.items())
    assert worst <= TOL, worst


@pytest.mark.parametrize("topk", [12, 16])
def test_attend_two_blocks_per_wave_flags_and_wide_queries(gpu, topk):
    """Two (k = 12) or four (k = 16) blocks per wave with invalid ids (past the row's blocks,
    past max_blocks), a block-table entry outside the cache, and queries spanning a wide range
    with a sharp softmax: invalid blocks are skipped and flagged, and the rest matches the
    oracle over the valid blocks."""
    case, nsplit, cus = _many_row_case(topk, 16, seed_shift=3)
    case.q[0::5, :8] *= 64
    case.q[1::7, 8:] *= 2.0 ** -20
    step = run_gpu_step(gpu, CFG0, DEV, topk=topk, case=case, sm_scale=2.0)
    R = step.rows.num_rows
    assert R * nsplit > 4 * cus and step.status == 0
    lay = case.layout
    ids, outs, _, rl = oracle_requests(step, "nvfp4", topk, 2.0, range(len(lay.seq_lens)))
    m = _oracle_ids_matrix(ids, R, topk)
    # row 3: one slot replaced by an id past its causal blocks; row 10: an id past max_blocks
    nb3 = (int(rl[3]) + 127) // 128
    m_bad = m.copy()
    slot3 = int(np.argmax(m[3] < 0)) if (m[3] < 0).any() else topk - 1
    m_bad[3, slot3] = nb3
    m_bad[10, topk - 1] = lay.max_blocks + 5
    # row 20's first selected block on a page outside the cache
    b20 = int(step.rows.row_req[20].item())
    blk = int(m[20, 0])
    bt = step.bt.clone()
    bt[b20, blk] = lay.num_pages + 11
    step.bt = bt
    got, st = _attend(gpu, step, m_bad, 2.0)
    assert st & gpu.DEV_BITS["BAD_BLOCK_ID"] and st & gpu.DEV_BITS["BAD_PAGE"]
    from oracle import path as Pth
    wc_q = F.bf16_to_f64(W.bf16_bits(case.q))
    row_req = step.rows.row_req.cpu().numpy()
    planes = {}
    affected = set()
    for r, want in outs.items():
        b = int(row_req[r])
        nb = (int(rl[r]) + 127) // 128
        kept = [int(j) for j in m_bad[r] if 0 <= j < nb and not (b == b20 and j == blk)]
        if len(kept) != int((m[r] >= 0).sum()):    # a skipped block: the oracle over the rest
            affected.add(r)
            if b not in planes:
                lo, hi = int(lay.tok_off[b]), int(lay.tok_off[b + 1])
                planes[b] = (F.dequantize("nvfp4", *F.quantize("nvfp4", W.bf16_bits(case.k[lo:hi]))),
                             F.dequantize("nvfp4", *F.quantize("nvfp4", W.bf16_bits(case.v[lo:hi]))))
            want = Pth.attend_row(wc_q[r], planes[b][0], planes[b][1], kept, int(rl[r]), 2.0)
        assert max_rel_err(got[r], want) <= TOL, r
    assert {10, 20} <= affected   # row 3 put its bad id in an empty slot


def test_attend_mxfp4_extreme_scales(gpu):
    """MXFP4 K / V groups whose E8M0 scales lie far outside fp16's range (amax about 2^18,
    scale byte 143; amax about 2^-28, byte 97): the attention decodes to bf16, exact for
    every byte a store writes, and matches the oracle within 5e-3."""
    case = W.make_case(CFG0, DEV, seq_lens=[3000, 900], q_len=2, G=16)
    tok = torch.arange(case.k.shape[0], device=DEV)
    big_k = ((tok // 128) % 3 == 0).to(torch.float32) * (2.0 ** 14 - 1) + 1
    small_k = torch.where((tok // 128) % 3 == 1, 2.0 ** -30, 1.0)
    big_v = ((tok // 64) % 4 == 1).to(torch.float32) * (2.0 ** 14 - 1) + 1
    small_v = torch.where((tok // 64) % 4 == 2, 2.0 ** -30, 1.0)
    case.k = (case.k.float() * (big_k * small_k)[:, None]).to(torch.bfloat16)
    case.v = (case.v.float() * (big_v * small_v)[:, None]).to(torch.bfloat16)
    sm = 2.0 ** -12   # keeps the logits of the 2^14-scaled keys of order one
    step = run_gpu_step(gpu, CFG0, DEV, topk=8, fmt="mxfp4", case=case, sm_scale=sm)
    assert step.status == 0, hex(step.status)
    sc = step.cache.planes["k"][1].cpu().numpy()
    assert sc.max() >= 142 and sc[sc > 0].min() <= 102      # outside fp16's exact range
    ids, outs, _, _ = oracle_requests(step, "mxfp4", 8, sm, range(2))
    got, st = _attend(gpu, step, _oracle_ids_matrix(ids, 4, 8), sm)
    assert st == 0
    worst = max(max_rel_err(got[r], want) for r, want in outs.items())
    assert worst <= TOL, worst


def test_attend_nvfp4_scale_range(gpu):
    """NVFP4 K / V groups over the E4M3 scale range: request 0 scaled by 2^-7 (most groups
    take subnormal scales, below 2^-6), request 1 by 2^6 (the outlier groups' scales near
    the 448 top), request 2 by 2^e per 128-token block (K) and per 64 tokens (V), e cycling
    over -8 .. 6. The attention decodes code x scale exactly in fp16 for every E4M3 byte and
    matches the oracle within 5e-3, through the split kernel (the oracle's ids) and through
    the one-call top-k + attention (its own ids, bit-exact)."""
    case = W.make_case(CFG0, DEV, seq_lens=[3000, 2500, 2600], q_len=2, G=16)
    lay = case.layout
    n = case.k.shape[0]
    tok = torch.arange(n, device=DEV)
    req = torch.bucketize(tok, torch.as_tensor(lay.tok_off[1:], device=DEV), right=True)
    loc = tok - torch.as_tensor(lay.tok_off, device=DEV)[req]
    e_k = torch.where(req == 0, -7, torch.where(req == 1, 6, (loc // 128) % 15 - 8)).to(torch.float32)
    e_v = torch.where(req == 0, -7, torch.where(req == 1, 6, (loc // 64) % 15 - 8)).to(torch.float32)
    case.k = (case.k.float() * torch.exp2(e_k)[:, None]).to(torch.bfloat16)
    case.v = (case.v.float() * torch.exp2(e_v)[:, None]).to(torch.bfloat16)
    sm = 2.0 ** -6   # logits of order one for the 2^6-scaled keys
    step = run_gpu_step(gpu, CFG0, DEV, topk=8, fmt="nvfp4", case=case, sm_scale=sm)
    assert step.status == 0, hex(step.status)
    sc = step.cache.planes["k"][1].cpu().numpy().ravel()
    sv = step.cache.planes["v"][1].cpu().numpy().ravel()
    for p in (sc, sv):
        mag = p & 0x7F
        assert ((mag >= 1) & (mag <= 7)).any() and (mag >= 0x76).any()   # subnormal and near 448
    R = step.rows.num_rows
    ids, outs, _, _ = oracle_requests(step, "nvfp4", 8, sm, range(3))
    got, st = _attend(gpu, step, _oracle_ids_matrix(ids, R, 8), sm)
    assert st == 0
    worst = max(max_rel_err(got[r], want) for r, want in outs.items())
    assert worst <= TOL, worst
    ws = gpu.index_attend_workspace(step.rows, lay.max_blocks, 8, 16, DEV)
    fid = torch.full((R, 8), -9, dtype=torch.int32, device=DEV)
    fout = torch.full((R, 16, 128), float("nan"), dtype=torch.float32, device=DEV)
    st2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    gpu.m3s_index_topk_attend(step.cache, case.q_idx, case.q, step.bt, lay.max_blocks, step.rows, 8, sm,
                              topk_ids=fid, out=fout, workspace=ws, dev_status=st2)
    torch.cuda.synchronize()
    assert int(st2.item()) == 0
    fid, fout = fid.cpu().numpy(), fout.cpu().double().numpy()
    for r, want in outs.items():
        assert (fid[r] == np.asarray(ids[r])).all(), r
        assert max_rel_err(fout[r], want) <= TOL, r


def test_attend_mxfp4_unstorable_scale_flagged(gpu):
    """An E8M0 scale byte above 252 (no store writes one) decodes to infinity: the
    affected outputs are written as 0 and the range bit is set; nothing is NaN."""
    step = run_gpu_step(gpu, CFG0, DEV, seq_lens=[2000], q_len=1, G=16, topk=4, fmt="mxfp4")
    assert step.status == 0
    blk = int(step.ids[0, 0].item())
    page = int(step.bt[0, blk].item())
    step.cache.planes["k"][1][page, 3, :] = 254
    ids = step.ids.cpu().numpy()
    got, st = _attend(gpu, step, ids, 1.0)
    assert st & gpu.DEV_BITS["RANGE"]
    assert np.isfinite(got).all()
