"""m3s_index_topk_attend (select and attention split in one kernel) against the two
separate calls on the same inputs: ids and outputs bit for bit, status included, over
decode and prefill rows, both formats, forced blocks, the tie rule, pad rows, one and
many splits, and the select's three register widths; one case also against the oracle.
Launches of more than two workgroups per CU take the separate kernels inside the call,
the select then writing each selected id's page for the attention (the 340-row prefill
cases and the 163-row decode case); every other case runs the fused kernel."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.stepcase import run_gpu_step, oracle_requests, max_rel_err, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
CFG0 = W.config(0)


def _pad(t, R):
    if R <= t.shape[0]:
        return t
    return torch.cat([t, torch.zeros((R - t.shape[0],) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)])


def _fused(gpu, step, topk, sm_scale, flags=0, init_blocks=0, local_blocks=0, workspace_junk=True):
    R = step.ids.shape[0]
    qi, q = _pad(step.case.q_idx, R), _pad(step.case.q, R)
    G = q.shape[1]
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = gpu.index_attend_workspace(step.rows, step.case.layout.max_blocks, topk, G, DEV)
    if workspace_junk:
        ws.fill_(0x7F)
    ids = torch.full((R, topk), -9, dtype=torch.int32, device=DEV)
    out = torch.full((R, G, 128), float("nan"), dtype=torch.float32, device=DEV)
    gpu.m3s_index_topk_attend(step.cache, qi, q, step.bt, step.case.layout.max_blocks, step.rows, topk, sm_scale,
                              flags=flags, topk_ids=ids, out=out, workspace=ws, dev_status=st,
                              init_blocks=init_blocks, local_blocks=local_blocks)
    torch.cuda.synchronize()
    return ids, out, int(st.item())


CASES = [
    # fmt, seq_lens, q_len, G, topk, flags, init, local, prefill, extra pad rows
    ("nvfp4", [150_000, 3000, 40_000], 8, 16, 16, 0, 0, 0, False, 3),
    ("mxfp4", [150_000, 3000, 40_000], 8, 16, 16, 0, 0, 0, False, 0),
    ("nvfp4", [20_000, 700, 9000], [4, 1, 8], 4, 4, 0, 0, 0, False, 2),      # one split
    ("nvfp4", [20_000, 9000], 3, 8, 64, 1, 0, 0, False, 0),                  # 16 splits, higher-id ties
    ("mxfp4", [30_000, 12_000, 800], 2, 2, 16, 0, 4, 16, False, 1),         # forced blocks
    ("nvfp4", [30_000, 5000], [300, 40], 4, 8, 0, 0, 0, True, 0),           # prefill rows (separate kernels)
    ("mxfp4", [30_000, 5000], [100, 20], 4, 8, 0, 0, 0, True, 0),           # prefill rows (fused kernel)
    ("mxfp4", [30_000, 600], [300, 40], 4, 8, 0, 0, 0, True, 0),            # separate kernels; 5-block rows
    ("nvfp4", [4000, 900, 150_000, 20_000] * 5, 8, 16, 16, 0, 0, 0, False, 3),  # 163 decode rows: separate
    ("nvfp4", [500_000], 2, 2, 16, 0, 0, 0, False, 0),                      # 3907 blocks: 16 per thread
    ("mxfp4", [1_000_000], 2, 2, 16, 0, 0, 0, False, 0),                    # 7813 blocks: 32 per thread
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-k{c[4]}-{i}" for i, c in enumerate(CASES)])
def test_fused_equals_separate_calls(gpu, case):
    fmt, seq, ql, G, topk, flags, init, local, prefill, npad = case
    say(f"[fused] {case}")
    wc = W.make_case(CFG0, DEV, seq_lens=seq, q_len=ql, G=G)
    R = int(wc.layout.cu_q[-1]) + npad
    step = run_gpu_step(gpu, CFG0, DEV, topk=topk, fmt=fmt, flags=flags, sm_scale=0.3, num_rows=R, case=wc,
                        init_blocks=init, local_blocks=local, prefill=prefill)
    assert step.status == 0, hex(step.status)
    ids, out, st = _fused(gpu, step, topk, 0.3, flags, init, local)
    assert st == step.status
    assert torch.equal(ids, step.ids)
    assert torch.equal(out, step.out)


ORACLE_CASES = [
    # fmt, seq_lens, q_len, G, topk
    ("nvfp4", [40_000, 2000, 9000], 8, 8, 16),
    ("nvfp4", [40_000, 2000, 9000], 8, 12, 16),         # G not a power of two
    ("mxfp4", [30_000, 700], 4, 3, 16),                 # G not a power of two
    ("nvfp4", [500_000], 2, 2, 16),                     # 3907 blocks: 16 per thread
    ("mxfp4", [1_000_000], 2, 2, 16),                   # 7813 blocks: 32 per thread
    ("mxfp4", [400_000, 3000], 2, 4, 16),               # 3125 blocks: 14 per thread
    ("nvfp4", [300_000], 3, 4, 16),                     # 2344 blocks: 14 per thread
    ("mxfp4", [150_000, 900], 2, 4, 16),                # 1172 blocks: 5 per thread
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", ORACLE_CASES, ids=[f"{c[0]}-G{c[3]}-{max(c[1])}" for c in ORACLE_CASES])
def test_fused_against_oracle(gpu, case):
    """Ids exact and attention within 5e-3 of the oracle, directly, on every row."""
    fmt, seq, ql, G, topk = case
    say(f"[fused vs oracle] {case}")
    wc = W.make_case(CFG0, DEV, seq_lens=seq, q_len=ql, G=G)
    step = run_gpu_step(gpu, CFG0, DEV, topk=topk, fmt=fmt, sm_scale=0.3, case=wc)
    assert step.status == 0, hex(step.status)
    ids, out, st = _fused(gpu, step, topk, 0.3)
    assert st == 0
    want_ids, want_out, _, _ = oracle_requests(step, fmt, topk, 0.3, range(len(seq)))
    assert len(want_ids) == ids.shape[0]
    got = ids.cpu().numpy()
    o = out.cpu().double().numpy()
    worst = 0.0
    for r, w in want_ids.items():
        assert got[r].tolist() == w.tolist(), r
        worst = max(worst, max_rel_err(o[r], want_out[r]))
    say(f"[fused vs oracle] max rel err {worst:.2e}")
    assert worst <= 5e-3, worst


@pytest.mark.parametrize("ql,prefill", [(4, False), ([300, 40], True)], ids=["fused-kernel", "separate-kernels"])
def test_fused_invalid_pages_flagged(gpu, ql, prefill):
    """A selected block whose page is outside the cache is skipped and flagged, as in
    the separate attention; ids are unchanged. With 340 rows the call runs the
    separate kernels and the page comes from the select's page list."""
    seq, G, topk = [20_000, 6000], 4, 8
    say(f"[fused invalid page] q_len {ql}")
    wc = W.make_case(CFG0, DEV, seq_lens=seq, q_len=ql, G=G)
    step = run_gpu_step(gpu, CFG0, DEV, topk=topk, sm_scale=0.3, case=wc, prefill=prefill)
    bad_blk = int(step.ids[0, 0].item())
    bt = step.bt.clone()
    bt[0, bad_blk] = step.case.layout.num_pages + 3
    step.bt = bt
    R = step.ids.shape[0]
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    ids_s = gpu.m3s_index_topk(step.cache, step.case.q_idx, bt, step.case.layout.max_blocks, step.rows, topk,
                               dev_status=st)
    out_s = gpu.m3s_sparse_attend(step.cache, step.case.q, bt, step.case.layout.max_blocks, step.rows, ids_s, 0.3,
                                  dev_status=st)
    torch.cuda.synchronize()
    ids, out, st_f = _fused(gpu, step, topk, 0.3)
    assert st_f == int(st.item()) and st_f & gpu.DEV_BITS["BAD_PAGE"]
    assert torch.equal(ids, ids_s) and torch.equal(out, out_s)


def test_many_rows_three_wave_select(gpu):
    """More rows than two select workgroups per CU (520 prefill rows of one 300,000-token
    request: 2344 blocks, 16 per thread) take the NVFP4 select built for three waves per
    SIMD, in m3s_index_topk and, with the page list, in the fused call: ids of sampled
    rows bit-exact against the oracle, and the fused call's ids and outputs bit for bit
    those of the separate calls."""
    from oracle import formats as F
    from oracle import path as P
    seq, ql, topk = [300_000], [520], 16
    say("[many rows] 520 prefill rows, 300000 tokens")
    wc = W.make_case(CFG0, DEV, seq_lens=seq, q_len=ql, G=2)
    step = run_gpu_step(gpu, CFG0, DEV, topk=topk, sm_scale=0.3, case=wc, prefill=True)
    assert step.status == 0, hex(step.status)
    ids, out, st = _fused(gpu, step, topk, 0.3)
    assert st == 0
    assert torch.equal(ids, step.ids) and torch.equal(out, step.out)
    _, row_len = P.decode_rows(wc.layout.cu_q, wc.layout.seq_lens, 520)
    qi = F.bf16_to_f64(W.bf16_bits(wc.q_idx))
    kidx = F.dequantize("nvfp4", *F.quantize("nvfp4", W.bf16_bits(wc.idx[:seq[0]])))
    got = step.ids.cpu().numpy()
    for r in (0, 261, 519):
        want = P.topk_blocks(P.block_scores(qi[r], kidx, int(row_len[r])), topk, False, 0, 0)
        assert got[r].tolist() == want.tolist(), r


def test_many_rows_page_list_in_workspace(gpu):
    """With many rows the fused call runs the select and the attention as separate kernels,
    and the select leaves each selected id's page in the workspace's last part (num_rows x
    topk int32 after the index and attention parts, each 256-byte aligned): the block-table
    entry of the row's request for a valid id, -1 for an empty slot (5-block rows)."""
    seq, ql, G, topk = [30_000, 600], [300, 40], 4, 8
    say("[page list] 340 prefill rows")
    wc = W.make_case(CFG0, DEV, seq_lens=seq, q_len=ql, G=G)
    step = run_gpu_step(gpu, CFG0, DEV, topk=topk, sm_scale=0.3, case=wc, prefill=True)
    R = step.ids.shape[0]
    mb = wc.layout.max_blocks
    ws = gpu.index_attend_workspace(step.rows, mb, topk, G, DEV)
    ws.fill_(0x7F)
    ids = torch.full((R, topk), -9, dtype=torch.int32, device=DEV)
    out = torch.empty((R, G, 128), dtype=torch.float32, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    gpu.m3s_index_topk_attend(step.cache, wc.q_idx, wc.q, step.bt, mb, step.rows, topk, 0.3, topk_ids=ids,
                              out=out, workspace=ws, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and torch.equal(ids, step.ids)
    a256 = lambda n: (n + 255) // 256 * 256
    off = a256(gpu.m3s_workspace_bytes(gpu.OP_INDEX_TOPK, R, 2, mb, topk, G)) + \
        a256(gpu.m3s_workspace_bytes(gpu.OP_SPARSE_ATTEND, R, 2, mb, topk, G))
    assert ws.numel() == off + a256(R * topk * 4)
    pages = ws[off: off + R * topk * 4].cpu().view(torch.int32).reshape(R, topk).numpy()
    got = ids.cpu().numpy()
    bt = step.bt.cpu().numpy()
    req = step.rows.row_req.cpu().numpy()
    want = np.where(got >= 0, bt[req[:, None], np.maximum(got, 0)], -1)
    assert (got == -1).any() and (got >= 0).any()
    assert np.array_equal(pages, want)
