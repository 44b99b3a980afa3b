"""m3s_decode_step (store, row map and index scan in one launch, then the fused select and
attention) against m3s_store_and_rows followed by m3s_index_topk_attend on a copy of the
same cache: planes, row map, ids, outputs and status, bit for bit. The separate calls are
checked against the oracle elsewhere; here the one-launch step must change nothing.

Cases cover the decode workloads' shapes (8 x 8 rows at 150K, 48 lognormal requests),
tails that cross a page boundary, steps whose rows are the whole context, single-block
requests, many requests (many tail workgroups), slices spanning many requests (query rows staged
in LDS or not), pad rows, a rejected request, a bad page
in a tail block, and a slot mapping that breaks the decode convention inside one page
(flagged, results still equal since the page has one writer). The new tokens' slots start
out holding random bytes, so a read of a page before the step's store has landed shows."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.stepcase import say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
CFG0 = W.config(0)


def _history_cache(gpu, wc, fmt):
    """A cache holding every token of the case except the step's new ones."""
    lay = wc.layout
    cache = gpu.Cache(fmt, lay.num_pages, DEV)
    slots = torch.as_tensor(W.all_slots(lay), device=DEV)
    hist = torch.ones(lay.total_tokens, dtype=torch.bool, device=DEV)
    hist[torch.as_tensor(lay.new_tokens, device=DEV)] = False
    h = torch.nonzero(hist).flatten()
    for s in range(0, h.numel(), 1 << 20):
        hh = h[s: s + (1 << 20)]
        gpu.m3s_store(cache, wc.k[hh], wc.v[hh], wc.idx[hh], slots[hh].contiguous())
    return cache


def _clone(gpu, cache):
    c = gpu.Cache(cache.fmt, cache.num_pages, DEV)
    for name in ("k", "v", "idx"):
        for i in range(2):
            c.planes[name][i].copy_(cache.planes[name][i])
    return c


def _run_both(gpu, wc, fmt, topk, sm_scale, pad_rows=0, reject=(), slot_swap=None, bad_tail_page=None, flags=0,
              init_blocks=0, local_blocks=0):
    lay = wc.layout
    R = int(lay.cu_q[-1])
    NR = R + pad_rows
    G = wc.q.shape[1]
    say(f"[step] {fmt} reqs={len(lay.seq_lens)} rows={NR} G={G} topk={topk} max_seq={int(lay.seq_lens.max())} "
        f"pad={pad_rows} reject={list(reject)} swap={slot_swap} bad_tail_page={bad_tail_page}")
    cache_a = _history_cache(gpu, wc, fmt)
    # the new tokens' slots hold stale bytes (as a recycled page does): a step that read
    # a page before its own store landed would see them
    g = torch.Generator(device="cpu").manual_seed(5)
    rows_of = torch.as_tensor(lay.new_slots.astype(np.int64), device=DEV)
    for name in ("k", "v", "idx"):
        for i in range(2):
            pl = cache_a.planes[name][i].view(-1, cache_a.planes[name][i].shape[-1])
            junk = torch.randint(0, 256, (rows_of.numel(), pl.shape[1]), generator=g, dtype=torch.uint8)
            pl[rows_of] = junk.to(DEV)
    cache_b = _clone(gpu, cache_a)
    new = torch.as_tensor(lay.new_tokens, device=DEV)
    rows_in = []
    for src in (wc.k, wc.v, wc.idx):
        t = torch.zeros((NR, 128), dtype=torch.bfloat16, device=DEV)
        t[:R] = src[new]
        rows_in.append(t)
    slots_np = np.full(NR, -1, dtype=np.int32)
    slots_np[:R] = lay.new_slots
    seq_np = lay.seq_lens.copy()
    for b in reject:  # seq_len < q_len: the row map rejects the request, its rows get slot -1
        seq_np[b] = int(lay.q_lens[b]) - 1
        slots_np[lay.cu_q[b]: lay.cu_q[b + 1]] = -1
    if slot_swap is not None:
        i, j = slot_swap
        slots_np[i], slots_np[j] = slots_np[j], slots_np[i]
    bt_np = lay.block_table.copy()
    if bad_tail_page is not None:  # request b's last block: an entry outside the planes
        b = bad_tail_page
        bt_np[b, int(lay.nblk[b]) - 1] = lay.num_pages + 5
        slots_np[lay.cu_q[b]: lay.cu_q[b + 1]] = -1
    slots = torch.as_tensor(slots_np, device=DEV)
    seq = torch.as_tensor(seq_np, device=DEV)
    cu_q = torch.as_tensor(lay.cu_q, device=DEV)
    bt = torch.as_tensor(bt_np, device=DEV)
    qi = torch.zeros((NR, 128), dtype=torch.bfloat16, device=DEV)
    qi[:R] = wc.q_idx
    q = torch.zeros((NR, G, 128), dtype=torch.bfloat16, device=DEV)
    q[:R] = wc.q
    B = len(seq_np)

    def outs():
        return (torch.full((NR,), -7, dtype=torch.int32, device=DEV),
                torch.full((NR,), -7, dtype=torch.int32, device=DEV),
                torch.full((B + 1,), -7, dtype=torch.int32, device=DEV))

    st_a = torch.zeros(1, dtype=torch.int32, device=DEV)
    rq_a, rl_a, rb_a = outs()
    rows_a = gpu.m3s_store_and_rows(cache_a, *rows_in, slots, cu_q, seq, NR, rq_a, rl_a, rb_a, st_a)
    ids_a, out_a = gpu.m3s_index_topk_attend(cache_a, qi, q, bt, lay.max_blocks, rows_a, topk, sm_scale, flags=flags,
                                             dev_status=st_a, init_blocks=init_blocks, local_blocks=local_blocks)
    st_b = torch.zeros(1, dtype=torch.int32, device=DEV)
    rq_b, rl_b, rb_b = outs()
    ids_b = torch.full((NR, topk), -9, dtype=torch.int32, device=DEV)
    out_b = torch.full((NR, G, 128), float("nan"), dtype=torch.float32, device=DEV)
    _, ids_b, out_b = gpu.m3s_decode_step(cache_b, *rows_in, slots, cu_q, seq, NR, rq_b, rl_b, rb_b, qi, q, bt,
                                          lay.max_blocks, topk, sm_scale, flags=flags, topk_ids=ids_b, out=out_b,
                                          dev_status=st_b, init_blocks=init_blocks, local_blocks=local_blocks)
    torch.cuda.synchronize()
    for name in ("k", "v", "idx"):
        for i in range(2):
            assert torch.equal(cache_a.planes[name][i], cache_b.planes[name][i]), f"plane {name}[{i}]"
    assert torch.equal(rq_a, rq_b) and torch.equal(rl_a, rl_b) and torch.equal(rb_a, rb_b)
    assert torch.equal(ids_a, ids_b)
    assert torch.equal(out_a.view(torch.int32), out_b.view(torch.int32))
    return int(st_a.item()), int(st_b.item())


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_step_equals_separate_calls_150k(gpu, fmt):
    cfg = W.config(1)
    wc = W.make_case(cfg, DEV)
    sa, sb = _run_both(gpu, wc, fmt, cfg.topk, cfg.sm_scale)
    assert sa == sb == 0


def test_step_equals_separate_calls_lognormal(gpu):
    cfg = W.config(3)
    wc = W.make_case(cfg, DEV)
    sa, sb = _run_both(gpu, wc, "nvfp4", cfg.topk, cfg.sm_scale)
    assert sa == sb == 0


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_step_page_edges(gpu, fmt):
    """Tails inside one page, across a page boundary, equal to the whole context, and
    single-block requests, with q_len from 1 to 16."""
    seq = [1, 8, 16, 127, 128, 129, 130, 135, 255, 256, 300, 5000, 16, 20_000, 2048, 131]
    ql = [1, 8, 16, 4, 16, 1, 8, 16, 2, 16, 12, 16, 9, 16, 3, 16]
    wc = W.make_case(CFG0, DEV, seq_lens=seq, q_len=ql, G=8)
    sa, sb = _run_both(gpu, wc, fmt, 8, 0.5)
    assert sa == sb == 0


def test_step_many_requests(gpu):
    """200 requests: 25 tail workgroups of eight requests, each storing a share of the step."""
    rng = np.random.default_rng(11)
    seq = [int(x) for x in rng.integers(40, 30_000, size=200)]
    wc = W.make_case(CFG0, DEV, seq_lens=seq, q_len=2, G=4)
    sa, sb = _run_both(gpu, wc, "nvfp4", 8, 1.0, flags=gpu.TOPK_TIE_HIGH_ID, init_blocks=1, local_blocks=2)
    assert sa == sb == 0


def test_step_max_requests(gpu):
    """4096 requests (the most a call takes) of one row each: 512 tail workgroups, more
    than the CUs, beside a single scan workgroup."""
    rng = np.random.default_rng(13)
    seq = [int(x) for x in rng.integers(1, 1500, size=4096)]
    wc = W.make_case(CFG0, DEV, seq_lens=seq, q_len=1, G=2)
    sa, sb = _run_both(gpu, wc, "nvfp4", 4, 1.0)
    assert sa == sb == 0


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_step_wide_slices(gpu, fmt):
    """1024 requests of 16 rows with 1 to 5 blocks before their new tokens: a scan
    workgroup's slice spans several requests, so some slices' rows fit the 64 rows a
    workgroup stages in LDS and others exceed them (their waves then read the query rows
    from HBM)."""
    rng = np.random.default_rng(17)
    seq = [int(x) for x in rng.integers(150, 700, size=1024)]
    wc = W.make_case(CFG0, DEV, seq_lens=seq, q_len=16, G=2)
    sa, sb = _run_both(gpu, wc, fmt, 4, 1.0)
    assert sa == sb == 0


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_step_pad_rows_and_rejected_request(gpu, fmt):
    wc = W.make_case(CFG0, DEV, seq_lens=[9000, 300, 40_000, 129], q_len=[8, 4, 16, 2], G=4)
    sa, sb = _run_both(gpu, wc, fmt, 4, 1.0, pad_rows=7, reject=(1,))
    assert sa == sb == gpu.DEV_BITS["BAD_ROWS"]


def test_step_bad_tail_page(gpu):
    wc = W.make_case(CFG0, DEV, seq_lens=[9000, 3000, 40_000], q_len=[8, 4, 16], G=4)
    sa, sb = _run_both(gpu, wc, "nvfp4", 4, 1.0, bad_tail_page=2)
    assert sa == sb and sa & gpu.DEV_BITS["BAD_PAGE"]


def test_step_slot_convention_flag(gpu):
    """Two new tokens of one request in one page trade slots: the step flags it; the page
    has a single writer, so results still equal the separate calls'."""
    wc = W.make_case(CFG0, DEV, seq_lens=[9000, 3000], q_len=[8, 4], G=4)
    sa, sb = _run_both(gpu, wc, "nvfp4", 4, 1.0, slot_swap=(1, 2))
    assert sa == 0
    assert sb == gpu.DEV_BITS["STEP_SLOT"]
