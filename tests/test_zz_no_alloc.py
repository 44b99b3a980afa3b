"""m3s_index_topk_attend_noalloc (the library's static scratch as the workspace) against
m3s_index_topk_attend on a caller workspace: ids, outputs and status bit for bit, on two
calls in a row, the second with a smaller input (fewer rows, shorter contexts), so the
scratch holds the first call's contents when the second runs. Then a call whose
workspace would exceed the scratch is refused before launching anything."""
import pytest
import torch

import workloads as W
from tests.stepcase import run_gpu_step, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
CFG0 = W.config(0)


def _both(gpu, step, topk, sm_scale, fmt):
    lay = step.case.layout
    R = step.ids.shape[0]
    G = step.case.q.shape[1]
    st_a = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = gpu.index_attend_workspace(step.rows, lay.max_blocks, topk, G, DEV)
    ids_a, out_a = gpu.m3s_index_topk_attend(step.cache, step.case.q_idx, step.case.q, step.bt, lay.max_blocks,
                                             step.rows, topk, sm_scale, workspace=ws, dev_status=st_a)
    st_b = torch.zeros(1, dtype=torch.int32, device=DEV)
    ids_b = torch.full((R, topk), -9, dtype=torch.int32, device=DEV)
    out_b = torch.full((R, G, 128), float("nan"), dtype=torch.float32, device=DEV)
    gpu.m3s_index_topk_attend_noalloc(step.cache, step.case.q_idx, step.case.q, step.bt, lay.max_blocks, step.rows,
                                      topk, sm_scale, topk_ids=ids_b, out=out_b, dev_status=st_b)
    torch.cuda.synchronize()
    return (ids_a, out_a, int(st_a.item())), (ids_b, out_b, int(st_b.item()))


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_noalloc_equals_workspace_call_twice(gpu, fmt):
    cases = [([150_000, 40_000, 9000, 150_000], 8, 16, 16),   # first call: 32 rows, 4 splits per row
             ([20_000, 3000], 4, 8, 8)]                        # second: 8 rows, shorter, 2 splits
    for i, (seq, ql, G, topk) in enumerate(cases):
        say(f"[noalloc] call {i}: {fmt} seq {seq} q_len {ql} G {G} topk {topk}")
        wc = W.make_case(CFG0, DEV, seq_lens=seq, q_len=ql, G=G)
        step = run_gpu_step(gpu, CFG0, DEV, topk=topk, fmt=fmt, sm_scale=0.3, case=wc)
        assert step.status == 0
        (ia, oa, sa), (ib, ob, sb) = _both(gpu, step, topk, 0.3, fmt)
        assert sa == sb == 0
        assert torch.equal(ia, ib) and torch.equal(oa, ob)
        assert torch.equal(ib, step.ids)


def test_noalloc_refuses_sizes_past_the_scratch(gpu):
    """A row count whose workspace exceeds the scratch returns M3S_ERR_WORKSPACE before any
    launch: the outputs keep their fill."""
    seq, ql = [1_000_000], [4096]
    wc = W.make_case(CFG0, DEV, seq_lens=seq, q_len=ql, G=16)
    lay = wc.layout
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    rows = gpu.m3s_prefill_rows(torch.as_tensor(lay.cu_q, device=DEV), torch.as_tensor(lay.seq_lens, device=DEV),
                                4096, dev_status=status)
    need = gpu.m3s_workspace_bytes(gpu.OP_INDEX_TOPK_ATTEND, 4096, rows.num_reqs, lay.max_blocks, 16, 16)
    assert need > gpu.NOALLOC_SCRATCH_BYTES
    cache = gpu.Cache("nvfp4", lay.num_pages, DEV)
    bt = torch.as_tensor(lay.block_table, device=DEV)
    ids = torch.full((4096, 16), -9, dtype=torch.int32, device=DEV)
    with pytest.raises(gpu.M3SError) as e:
        gpu.m3s_index_topk_attend_noalloc(cache, wc.q_idx, wc.q, bt, lay.max_blocks, rows, 16, 1.0, topk_ids=ids,
                                          dev_status=status)
    assert e.value.status == gpu.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((ids == -9).all())
