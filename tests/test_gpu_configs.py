"""The full step on every workload configuration: ids bit-exact and attention within 5e-3
of the oracle on every row of every request, stored planes bit-exact on sampled requests'
pages; and the one-call forms (m3s_index_topk_attend, and m3s_decode_step, the call the
bench times) equal to the separate calls bit for bit on every row."""
import time

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from tests.stepcase import max_rel_err, oracle_requests, run_gpu_step, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 5e-3

# requests whose stored planes are compared byte for byte with the oracle's store (the
# 48-request batch: its longest (450,000 tokens) and shortest (38,904 tokens) requests)
PLANE_SAMPLES = {0: [0], 1: [0, 5], 2: [0, 3], 3: [9, 36], 4: [2, 7]}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ci", [0, 1, 2, 3, 4])
def test_config_full_step(gpu, ci):
    cfg = W.config(ci)
    step = run_gpu_step(gpu, cfg, DEV)
    assert step.status == 0, hex(step.status)
    lay = step.case.layout
    reqs = list(range(len(lay.seq_lens)))
    say(f"[config {cfg.name}] oracle on all {len(reqs)} requests")
    t0 = time.perf_counter()
    ids, outs, rr, rl = oracle_requests(step, cfg.fmt, cfg.topk, cfg.sm_scale, reqs)
    say(f"[config {cfg.name}] oracle {time.perf_counter() - t0:.1f} s")
    got_ids = step.ids.cpu().numpy()
    got = step.out.cpu().double().numpy()
    assert np.array_equal(step.rows.row_req.cpu().numpy(), rr)
    assert np.array_equal(step.rows.row_len.cpu().numpy(), rl)
    worst = 0.0
    for r in ids:
        assert got_ids[r].tolist() == ids[r].tolist(), (r, got_ids[r].tolist(), ids[r].tolist())
        worst = max(worst, max_rel_err(got[r], outs[r]))
    say(f"[config {cfg.name}] ids equal on {len(ids)} rows, max rel err {worst:.2e}")
    assert len(ids) == int(lay.cu_q[-1])
    assert worst <= TOL
    # the bench's call: select and attention fused, on the same inputs, bit for bit
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    ids_f, out_f = gpu.m3s_index_topk_attend(step.cache, step.case.q_idx, step.case.q, step.bt, lay.max_blocks,
                                             step.rows, cfg.topk, cfg.sm_scale, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(ids_f, step.ids) and torch.equal(out_f, step.out)
    # the call the bench times: the whole step in m3s_decode_step (store of the new rows,
    # which are already in the cache: the same bytes again; row map; index; attention)
    newt = torch.as_tensor(lay.new_tokens, device=DEV)
    R = int(lay.cu_q[-1])
    rq, rl, rb = (torch.full((n,), -7, dtype=torch.int32, device=DEV) for n in (R, R, len(lay.seq_lens) + 1))
    _, ids_d, out_d = gpu.m3s_decode_step(
        step.cache, step.case.k[newt], step.case.v[newt], step.case.idx[newt],
        torch.as_tensor(lay.new_slots, device=DEV), torch.as_tensor(lay.cu_q, device=DEV),
        torch.as_tensor(lay.seq_lens, device=DEV), R, rq, rl, rb, step.case.q_idx, step.case.q, step.bt,
        lay.max_blocks, cfg.topk, cfg.sm_scale, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(ids_d, step.ids) and torch.equal(out_d, step.out)
    assert torch.equal(rq, step.rows.row_req) and torch.equal(rl, step.rows.row_len)
    assert torch.equal(rb, step.rows.grp_blk)
    # stored planes of the sampled requests (index plane: every page; K/V: the new rows' pages)
    sb = 8 if cfg.fmt == "nvfp4" else 4
    for b in PLANE_SAMPLES[ci]:
        lo, hi = int(lay.tok_off[b]), int(lay.tok_off[b + 1])
        slots = W.all_slots(lay)[lo:hi].astype(np.int64)
        wp, ws = F.quantize(cfg.fmt, W.bf16_bits(step.case.idx[lo:hi]))
        p, s = step.cache.planes["idx"]
        p = p.view(-1, 64)[torch.as_tensor(slots, device=DEV)].cpu().numpy()
        s = s.view(-1, sb)[torch.as_tensor(slots, device=DEV)].cpu().numpy()
        assert np.array_equal(p, wp) and np.array_equal(s, ws), b
    new = lay.new_tokens
    for name in ("k", "v"):
        wp, ws = F.quantize(cfg.fmt, W.bf16_bits(getattr(step.case, name)[torch.as_tensor(new, device=DEV)]))
        p, s = step.cache.planes[name]
        sl = torch.as_tensor(lay.new_slots.astype(np.int64), device=DEV)
        assert np.array_equal(p.view(-1, 64)[sl].cpu().numpy(), wp)
        assert np.array_equal(s.view(-1, sb)[sl].cpu().numpy(), ws)
