"""m3s_index_topk parity: top-k ids bit-exact against the oracle (small sizes, every row)."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.stepcase import oracle_requests, run_gpu_step, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
CFG0 = W.config(0)


def _check_all(gpu, step, fmt, topk, tie_high=False, q_idx_bits=None, init_blocks=0, local_blocks=0):
    lay = step.case.layout
    B = len(lay.seq_lens)
    ids, _, rr, _ = oracle_requests(step, fmt, topk, 1.0, range(B), tie_high, q_idx_bits, init_blocks,
                                    local_blocks)
    got = step.ids.cpu().numpy()
    for r, want in ids.items():
        assert got[r].tolist() == want.tolist(), (r, got[r].tolist(), want.tolist())
    for r in range(len(rr)):
        if rr[r] < 0:
            assert np.all(got[r] == -1)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("topk", [1, 4, 16, 64])
def test_index_small_ragged(gpu, fmt, topk):
    seq = [2048, 5000, 300, 129, 128, 127, 17, 9000]
    step = run_gpu_step(gpu, CFG0, DEV, seq_lens=seq, q_len=3, G=4, topk=topk, fmt=fmt)
    assert step.status == 0, hex(step.status)
    _check_all(gpu, step, fmt, topk)


@pytest.mark.parametrize("q_len", [1, 8, 16])
def test_index_q_len_and_pad_rows(gpu, q_len):
    seq = [4000, 1500, 260]
    R = len(seq) * q_len + 5
    step = run_gpu_step(gpu, CFG0, DEV, seq_lens=seq, q_len=q_len, G=2, topk=8, num_rows=R)
    assert step.status == 0, hex(step.status)
    _check_all(gpu, step, "nvfp4", 8)
    assert np.all(step.ids.cpu().numpy()[len(seq) * q_len:] == -1)


@pytest.mark.parametrize("tie_high", [False, True])
def test_index_zero_query_ties(gpu, tie_high):
    """Zero queries: every score is 0; ties go to the lower (or higher) ids. Three and four
    requests, as in the ATOM tie test."""
    for nreq in (3, 4):
        seq = [3000] * nreq
        case = W.make_case(CFG0, DEV, seq_lens=seq, q_len=2, G=2)
        case.q_idx = torch.zeros_like(case.q_idx)
        step = run_gpu_step(gpu, CFG0, DEV, topk=16, case=case, flags=1 if tie_high else 0)
        assert step.status == 0
        nb = (3000 + 127) // 128
        want = list(range(nb - 16, nb)) if tie_high else list(range(16))
        assert all(row == want for row in step.ids.cpu().numpy().tolist())


@pytest.mark.parametrize("fmt,q_len", [("nvfp4", 2), ("nvfp4", 70), ("mxfp4", 70)])
def test_index_equal_blocks_need_exact_rescore(gpu, fmt, q_len):
    """Every page holds the same tokens, so every block ties exactly but the fp32 error
    bound is non-zero: the band covers all blocks and the exact rescore must order them
    by id. With 70 rows per request the rows go through the prefill row map and the wide
    scan (two 64-row work groups per request, the second partly filled)."""
    case = W.make_case(CFG0, DEV, seq_lens=[128 * 40, 128 * 33 + 5], q_len=q_len, G=2)
    lay = case.layout
    for b in range(2):
        lo, hi = int(lay.tok_off[b]), int(lay.tok_off[b + 1])
        n = hi - lo
        base = case.idx[lo: lo + 128].clone()
        reps = (n + 127) // 128
        case.idx[lo:hi] = base.repeat(reps, 1)[:n]
    step = run_gpu_step(gpu, CFG0, DEV, topk=16, case=case, fmt=fmt, prefill=q_len > 16)
    assert step.status == 0, hex(step.status)
    _check_all(gpu, step, fmt, 16)


def test_index_band_overflow_selects_by_key(gpu):
    """More than 1024 blocks tie exactly (every page holds the same tokens) and the fp32
    error bound is non-zero, so the band exceeds the rescore's capacity. The select then
    takes the k best fp32 keys (identical pages give identical fp32 scores, so ties go to
    the lower ids) and reports M3S_DEV_BAND_OVERFLOW. The ids still equal the exact
    selection, through m3s_index_topk and through the fused m3s_index_topk_attend."""
    nblk = 1100
    case = W.make_case(CFG0, DEV, seq_lens=[128 * nblk], q_len=2, G=2)
    lay = case.layout
    n = int(lay.seq_lens[0])
    base = case.idx[:128].clone()
    case.idx[:n] = base.repeat(nblk, 1)[:n]
    step = run_gpu_step(gpu, CFG0, DEV, topk=16, case=case)
    assert step.status == gpu.DEV_BITS["BAND_OVERFLOW"], hex(step.status)
    _check_all(gpu, step, "nvfp4", 16)
    assert step.ids.cpu().numpy().tolist() == [list(range(16))] * 2
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    ids_f, _ = gpu.m3s_index_topk_attend(step.cache, case.q_idx, case.q, step.bt, lay.max_blocks, step.rows, 16,
                                         1.0, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == gpu.DEV_BITS["BAND_OVERFLOW"], hex(int(st.item()))
    assert torch.equal(ids_f, step.ids)


@pytest.mark.parametrize("fmt,q_len", [("nvfp4", 4), ("nvfp4", 70), ("mxfp4", 70)])
def test_index_near_ties_are_decided_exactly(gpu, fmt, q_len):
    """Blocks that differ from block 0 by a single tiny element: exact scores differ far
    below the fp32 error bound, so the selection is decided by the float64 rescore (70
    rows: the prefill row map and the wide scan, whose bounds are reduced across the
    wave's rows for four query tiles at once)."""
    case = W.make_case(CFG0, DEV, seq_lens=[128 * 64], q_len=q_len, G=2)
    n = 128 * 64
    base = case.idx[:128].clone()
    idx = base.repeat(64, 1)
    g = torch.Generator(device="cpu").manual_seed(5)
    # perturb one element of one token per block by a tiny bf16 amount
    for j in range(64):
        t = j * 128 + int(torch.randint(0, 128, (1,), generator=g))
        d = int(torch.randint(0, 128, (1,), generator=g))
        idx[t, d] = (idx[t, d].float() * (1 + 2.0 ** -7 * int(torch.randint(-2, 3, (1,), generator=g)))).to(torch.bfloat16)
    case.idx[:n] = idx
    step = run_gpu_step(gpu, CFG0, DEV, topk=16, case=case, fmt=fmt, prefill=q_len > 16)
    assert step.status == 0, hex(step.status)
    _check_all(gpu, step, fmt, 16)


def test_index_fewer_blocks_than_k(gpu):
    step = run_gpu_step(gpu, CFG0, DEV, seq_lens=[100, 300, 1000], q_len=2, G=2, topk=16)
    got = step.ids.cpu().numpy()
    assert got[0].tolist() == [0] + [-1] * 15
    assert got[2].tolist() == [0, 1, 2] + [-1] * 13
    assert got[4].tolist() == list(range(8)) + [-1] * 8


def test_index_bad_page_is_flagged(gpu):
    """A block-table entry outside [0, num_pages) is never read: the block scores -inf and
    the device status says why."""
    step = run_gpu_step(gpu, CFG0, DEV, seq_lens=[3000], q_len=1, G=2, topk=4)
    assert step.status == 0
    lay = step.case.layout
    bad = lay.block_table.copy()
    bad[0, 5] = lay.num_pages + 7
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    ids = gpu.m3s_index_topk(step.cache, step.case.q_idx, torch.as_tensor(bad, device=DEV), lay.max_blocks,
                             step.rows, 4, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & gpu.DEV_BITS["BAD_PAGE"]
    assert 5 not in ids.cpu().numpy()[0].tolist()


@pytest.mark.parametrize("topk", [16, 63, 64])
def test_index_wave_boundaries(gpu, topk):
    # block counts around the select's 64-per-wave and 256-per-pass boundaries
    seq = [64 * 128 * 3 + 1, 195 * 128, 256 * 128, 257 * 128 + 7, 40000]
    step = run_gpu_step(gpu, CFG0, DEV, seq_lens=seq, q_len=2, G=2, topk=topk)
    assert step.status == 0, hex(step.status)
    _check_all(gpu, step, "nvfp4", topk)



@pytest.mark.parametrize("fill", [0x7F, 0xFF])
def test_index_dirty_workspace(gpu, fill):
    """Workspace entries of blocks past a row's causal range are never written by the
    scan; the select must not read them (a stale huge or NaN bound would widen the
    certification band). The workspace is filled with junk bytes before the call."""
    step = run_gpu_step(gpu, CFG0, DEV, seq_lens=[9000, 700, 30000], q_len=3, G=2, topk=16)
    lay = step.case.layout
    ws = gpu.index_workspace(step.rows, lay.max_blocks, 16, DEV)
    ws.fill_(fill)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    ids = gpu.m3s_index_topk(step.cache, step.case.q_idx, torch.as_tensor(lay.block_table, device=DEV),
                             lay.max_blocks, step.rows, 16, workspace=ws, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0, hex(int(st.item()))
    assert torch.equal(ids, step.ids)
    _check_all(gpu, step, "nvfp4", 16)


def _adversarial_queries(R, seed):
    """Index queries whose 32-dim blocks stress the scorers' query handling: an all-zero
    block, blocks spanning 24 binades, one dominant element over tiny ones, values whose
    quotient by the block's leading power rounds to 16, and exact powers of two."""
    g = np.random.default_rng(seed)
    q = g.standard_normal((R, 128)) / np.sqrt(128.0)
    for r in range(R):
        kind = r % 4
        if kind == 0:
            q[r, 0:32] = 0.0
            e = -(np.arange(32) % 25)
            q[r, 32:64] = np.where(np.arange(32) % 2, -1.0, 1.0) * np.ldexp(1.0 + (np.arange(32) % 7) / 8.0, e)
        elif kind == 1:
            q[r, 64:96] = np.ldexp(1.0, -18) * g.standard_normal(32)
            q[r, 64] = 8.0
            q[r, 96:128] = np.ldexp(1.0 + 127.0 / 128.0, -3) * np.sign(g.standard_normal(32))
        elif kind == 2:
            q[r, :] = np.ldexp(1.0, g.integers(-12, 2, 128)) * np.sign(g.standard_normal(128))
        else:
            q[r, 0:32] = np.ldexp(1.0 + 1.0 / 2 + 1.0 / 16 + 1.0 / 128, -4) * np.sign(g.standard_normal(32))
            q[r, 32:64] *= 2.0 ** 20
    return torch.as_tensor(q, dtype=torch.float32).to(torch.bfloat16)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_index_adversarial_queries(gpu, fmt):
    seq = [6000, 128 * 20 + 3, 2500]
    case = W.make_case(CFG0, DEV, seq_lens=seq, q_len=4, G=2)
    qi = _adversarial_queries(case.q_idx.shape[0], 11).to(DEV)
    step = run_gpu_step(gpu, CFG0, DEV, topk=8, case=case, fmt=fmt, q_idx=qi)
    assert step.status == 0, hex(step.status)
    _check_all(gpu, step, fmt, 8)


@pytest.mark.parametrize("init,local,topk", [(1, 2, 8), (4, 16, 16), (0, 3, 4), (20, 0, 16), (3, 3, 4),
                                             (2, 1, 64)])
@pytest.mark.parametrize("tie_high", [False, True])
def test_index_forced_blocks(gpu, init, local, topk, tie_high):
    """Forced initial / local blocks: ids bit-exact against the oracle on ragged rows, among
    them the review's case (top-k 16, init 4, local 16) and forced sets larger than k."""
    seq = [9000, 2048, 700, 129, 40000]
    step = run_gpu_step(gpu, CFG0, DEV, seq_lens=seq, q_len=3, G=2, topk=topk, flags=1 if tie_high else 0,
                        init_blocks=init, local_blocks=local)
    assert step.status == 0, hex(step.status)
    _check_all(gpu, step, "nvfp4", topk, tie_high, init_blocks=init, local_blocks=local)
    if (init, local, topk) == (4, 16, 16):
        ids = step.ids.cpu().numpy()
        r = int(step.case.layout.cu_q[4]) + 2   # last row of the 40000-token request
        nb = (40000 + 127) // 128
        assert ids[r].tolist() == [0, 1, 2, 3] + list(range(nb - 12, nb))



@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_prefill_step(gpu, fmt):
    """Prefill rows (chunks of 300, 40 and 133 tokens after prefixes, and a 700-token
    request with no prefix) through the same scan, top-k and attention: ids bit-exact,
    attention within 5e-3 on every row."""
    from tests.stepcase import max_rel_err
    seq = [3300, 700, 1500, 173]
    ql = [300, 700, 40, 133]
    case = W.make_case(CFG0, DEV, seq_lens=seq, q_len=ql, G=4)
    step = run_gpu_step(gpu, CFG0, DEV, topk=8, case=case, fmt=fmt, prefill=True, sm_scale=0.3)
    assert step.status == 0, hex(step.status)
    ids, outs, rr, rl = oracle_requests(step, fmt, 8, 0.3, range(len(seq)))
    got = step.ids.cpu().numpy()
    o = step.out.cpu().double().numpy()
    assert np.array_equal(step.rows.row_req.cpu().numpy(), rr)
    worst = 0.0
    for r, want in ids.items():
        assert got[r].tolist() == want.tolist(), (r, got[r].tolist(), want.tolist())
        worst = max(worst, max_rel_err(o[r], outs[r]))
    assert worst <= 5e-3, worst


@pytest.mark.parametrize("topk", [16, 64])
def test_index_max_blocks(gpu, topk):
    """The largest rows: one request of 1,000,000 tokens (7813 blocks, the select's widest
    variant), two rows; ids bit-exact against the oracle."""
    step = run_gpu_step(gpu, CFG0, DEV, seq_lens=[1_000_000], q_len=2, G=2, topk=topk)
    assert step.status == 0, hex(step.status)
    _check_all(gpu, step, "nvfp4", topk)
