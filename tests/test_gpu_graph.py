"""The calls are safe to capture in a HIP graph: a captured step (store + row map +
index top-k + sparse attend, decode or prefill, as separate calls, with the fused index
call, or as one m3s_decode_step call) and a captured fused producer store,
replayed several times with eager work in between that overwrites every output,
workspace and the step's cache slots with junk, give the eager results bit for bit on
every replay."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.stepcase import say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
CFG0 = W.config(0)


def _fill_history(m3s, fmt, lay, case):
    cache = m3s.Cache(fmt, lay.num_pages, DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    slots = torch.as_tensor(W.all_slots(lay), device=DEV)
    hist = torch.ones(lay.total_tokens, dtype=torch.bool, device=DEV)
    new_idx = torch.as_tensor(lay.new_tokens, device=DEV)
    hist[new_idx] = False
    h = torch.nonzero(hist).flatten()
    m3s.m3s_store(cache, case.k[h], case.v[h], case.idx[h], slots[h].contiguous(), status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return cache, slots[new_idx].contiguous(), new_idx


@pytest.mark.parametrize("fmt,prefill,fused", [("nvfp4", False, False), ("mxfp4", False, False),
                                               ("nvfp4", True, False), ("mxfp4", True, False),
                                               ("nvfp4", False, True), ("mxfp4", True, True),
                                               ("nvfp4", False, "step"), ("mxfp4", False, "step")])
def test_step_graph_replays_match_eager(gpu, fmt, prefill, fused):
    """fused: False, the four calls; True, store + row map then m3s_index_topk_attend;
    "step": one m3s_decode_step call."""
    seq = [3000, 9000, 20000]
    ql = [200, 70, 1] if prefill else [4, 8, 1]
    G, topk = 8, 8
    say(f"[graph] step fmt={fmt} prefill={prefill} fused={fused}")
    case = W.make_case(CFG0, DEV, seq_lens=seq, q_len=ql, G=G)
    lay = case.layout
    R = int(lay.cu_q[-1]) + 3                       # three pad rows
    cache, s_new, new_idx = _fill_history(gpu, fmt, lay, case)
    k_new, v_new, i_new = (t[new_idx].contiguous() for t in (case.k, case.v, case.idx))
    pad = lambda t: torch.cat([t, torch.zeros((3,) + tuple(t.shape[1:]), dtype=t.dtype, device=DEV)])
    if fused == "step":  # one token per row: the pad rows' tokens are zero rows with slot -1
        k_new, v_new, i_new = pad(k_new), pad(v_new), pad(i_new)
    s_new_rows = torch.cat([s_new, torch.full((3,), -1, dtype=torch.int32, device=DEV)])
    q, q_idx = pad(case.q), pad(case.q_idx)
    cu_q = torch.as_tensor(lay.cu_q, device=DEV)
    seq_t = torch.as_tensor(lay.seq_lens, device=DEV)
    bt = torch.as_tensor(lay.block_table, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    row_req = torch.empty(R, dtype=torch.int32, device=DEV)
    row_len = torch.empty(R, dtype=torch.int32, device=DEV)
    req_blk = torch.empty(len(seq) + 1, dtype=torch.int32, device=DEV)
    if prefill:
        rows = gpu.m3s_prefill_rows(cu_q, seq_t, R, dev_status=status)
    else:
        rows = gpu.m3s_decode_rows(cu_q, seq_t, R, row_req, row_len, req_blk, status)
    ids = torch.empty((R, topk), dtype=torch.int32, device=DEV)
    out = torch.empty((R, G, 128), dtype=torch.float32, device=DEV)
    ws_i = gpu.index_workspace(rows, lay.max_blocks, topk, DEV)
    ws_a = gpu.attend_workspace(rows, lay.max_blocks, topk, G, DEV)
    ws_f = gpu.index_attend_workspace(rows, lay.max_blocks, topk, G, DEV)

    def step():
        if fused == "step":
            gpu.m3s_decode_step(cache, k_new, v_new, i_new, s_new_rows, cu_q, seq_t, R, row_req, row_len, req_blk,
                                q_idx, q, bt, lay.max_blocks, topk, 0.3, 0, ids, out, ws_f, status)
            return
        if prefill:
            gpu.m3s_store(cache, k_new, v_new, i_new, s_new, status)
            gpu.m3s_prefill_rows(cu_q, seq_t, R, rows.num_groups, status, out=rows)
        else:
            gpu.m3s_store_and_rows(cache, k_new, v_new, i_new, s_new, cu_q, seq_t, R, row_req, row_len, req_blk,
                                   status)
        if fused:
            gpu.m3s_index_topk_attend(cache, q_idx, q, bt, lay.max_blocks, rows, topk, 0.3, 0, ids, out, ws_f, status)
        else:
            gpu.m3s_index_topk(cache, q_idx, bt, lay.max_blocks, rows, topk, 0, ids, ws_i, status)
            gpu.m3s_sparse_attend(cache, q, bt, lay.max_blocks, rows, ids, 0.3, out, ws_a, status)

    step()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ids_e, out_e = ids.clone(), out.clone()
    assert torch.isfinite(out_e).all()

    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step()
    torch.cuda.synchronize()
    junk = [ids, out, ws_i, ws_a, ws_f, rows.row_req, rows.row_len, rows.grp_blk]
    if prefill:
        junk += [rows.grp_row, rows.grp_req]
    else:
        junk += [row_req, row_len, req_blk]
    sl = s_new.long()
    for rep in range(3):
        # eager work between replays: junk everywhere the step writes
        for t in junk:
            if t.dtype.is_floating_point:
                t.fill_(float("nan"))
            else:
                t.fill_(-7 if t.dtype != torch.uint8 else 0x7E)
        for p, s in cache.planes.values():
            p.view(-1, p.shape[-1])[sl] = 0x77
            s.view(-1, s.shape[-1])[sl] = 0x3F
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0, rep
        assert torch.equal(ids, ids_e), rep
        assert torch.equal(out, out_e), rep


def test_producer_graph_replays_match_eager(gpu):
    T, G, rd, fmt = 40, 4, 64, "nvfp4"
    say(f"[graph] producer T={T} G={G} rd={rd}")
    mk = lambda shape, f: W.gen_prenorm_rows(shape, 3, f, DEV)
    q = mk((T, G, 128), W.PQ_FAMILY)
    k, v, iq, ik = (mk((T, 128), f) for f in (W.PK_FAMILY, W.PV_FAMILY, W.PIQ_FAMILY, W.PIK_FAMILY))
    w = W.gen_norm_weights(3, DEV)
    cs = torch.as_tensor(W.rope_table(512, rd), device=DEV)
    pos = torch.as_tensor(np.random.default_rng(2).integers(0, 512, size=T).astype(np.int32), device=DEV)
    slots = torch.as_tensor(np.random.default_rng(5).permutation(256)[:T].astype(np.int32), device=DEV)
    cache = gpu.Cache(fmt, 2, DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    q_out = torch.empty((T, G, 128), dtype=torch.bfloat16, device=DEV)
    iq_out = torch.empty((T, 128), dtype=torch.bfloat16, device=DEV)
    qe = torch.empty((T, G, 128), dtype=torch.uint8, device=DEV)

    def run():
        gpu.m3s_qknorm_rope_store(cache, q, k, v, iq, ik, w, 1e-6, pos, cs, slots, q_out=q_out, idx_q_out=iq_out,
                                  q_out_e4m3=qe, dev_status=status)

    run()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    want = [t.clone() for t in (q_out, iq_out, qe)] + [t.clone() for pl in cache.planes.values() for t in pl]
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        q_out.view(torch.int16).fill_(-1)
        iq_out.view(torch.int16).fill_(-1)
        qe.fill_(0x55)
        for p, s in cache.planes.values():
            p.view(-1, 64)[slots.long()] = 0x77
            s.view(-1, s.shape[-1])[slots.long()] = 0x3F
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [q_out, iq_out, qe] + [t for pl in cache.planes.values() for t in pl]
        for a, b in zip(got, want):
            assert torch.equal(a, b), rep
        assert int(status.item()) == 0
