"""Shared driver of GPU parity tests: one decode step through the C ABI and the
same step through the oracle, on the same seeded inputs (workloads)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import sys
from dataclasses import dataclass

import numpy as np
import torch

import workloads as W
from oracle import formats as F
from oracle import path as P


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@dataclass
class GpuStep:
    case: W.Case
    cache: object
    rows: object
    ids: torch.Tensor
    out: torch.Tensor
    status: int
    bt: torch.Tensor


def run_gpu_step(m3s, cfg, dev, seq_lens=None, q_len=None, G=None, topk=None, fmt=None, flags=0,
                 sm_scale=None, num_rows=None, case=None, q_idx=None, init_blocks=0, local_blocks=0,
                 prefill=False):
    """Fill the history with m3s_store, then run store / rows / top-k / attend for the step rows."""
    if case is None:
        case = W.make_case(cfg, dev, seq_lens=seq_lens, q_len=q_len, G=G)
    if q_idx is not None:
        case.q_idx = q_idx
    lay = case.layout
    fmt = fmt or cfg.fmt
    topk = topk or cfg.topk
    sm_scale = cfg.sm_scale if sm_scale is None else sm_scale
    R = int(lay.cu_q[-1]) if num_rows is None else num_rows
    say(f"[gpu step] cfg={cfg.name} fmt={fmt} reqs={len(lay.seq_lens)} rows={R} topk={topk} "
        f"G={case.q.shape[1]} tokens={lay.total_tokens}")
    cache = _m3s_cache(m3s, fmt, lay.num_pages, dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    slots = torch.as_tensor(W.all_slots(lay), device=dev)
    hist = torch.ones(lay.total_tokens, dtype=torch.bool, device=dev)
    new_idx = torch.as_tensor(lay.new_tokens, device=dev)
    hist[new_idx] = False
    hidx = torch.nonzero(hist).flatten()
    chunk = 1 << 20
    for s in range(0, hidx.numel(), chunk):
        h = hidx[s: s + chunk]
        m3s.m3s_store(cache, case.k[h], case.v[h], case.idx[h], slots[h].contiguous(), status)
    m3s.m3s_store(cache, case.k[new_idx], case.v[new_idx], case.idx[new_idx], slots[new_idx].contiguous(), status)
    cu_q = torch.as_tensor(lay.cu_q, device=dev)
    seq = torch.as_tensor(lay.seq_lens, device=dev)
    if prefill:
        rows = m3s.m3s_prefill_rows(cu_q, seq, R, dev_status=status)
    else:
        rows = m3s.m3s_decode_rows(cu_q, seq, R, dev_status=status)
    bt = torch.as_tensor(lay.block_table, device=dev)
    qi = case.q_idx
    q = case.q
    if R > qi.shape[0]:   # pad rows: any values
        qi = torch.cat([qi, torch.zeros((R - qi.shape[0], qi.shape[1]), dtype=qi.dtype, device=dev)])
        q = torch.cat([q, torch.zeros((R - q.shape[0],) + tuple(q.shape[1:]), dtype=q.dtype, device=dev)])
    ids = m3s.m3s_index_topk(cache, qi, bt, lay.max_blocks, rows, topk, flags=flags, dev_status=status,
                             init_blocks=init_blocks, local_blocks=local_blocks)
    out = m3s.m3s_sparse_attend(cache, q, bt, lay.max_blocks, rows, ids, sm_scale, dev_status=status)
    torch.cuda.synchronize()
    return GpuStep(case, cache, rows, ids, out, int(status.item()), bt)


def _m3s_cache(m3s, fmt, num_pages, dev):
    return m3s.Cache(fmt, num_pages, dev)


def oracle_requests(step: GpuStep, fmt, topk, sm_scale, requests, tie_high=False, q_idx_bits=None,
                    init_blocks=0, local_blocks=0, threads=None):
    """Oracle ids / outputs for the rows of `requests` (planes quantized by the oracle itself).

    The oracle's functions run unchanged; independent requests (and rows) run in a thread
    pool, since the numpy work releases the GIL."""
    case = step.case
    lay = case.layout
    R = step.ids.shape[0]
    qi_bits = W.bf16_bits(case.q_idx) if q_idx_bits is None else q_idx_bits
    q_bits = W.bf16_bits(case.q)
    row_req, row_len = P.decode_rows(lay.cu_q, lay.seq_lens, R)
    qi = F.bf16_to_f64(qi_bits)
    qm = F.bf16_to_f64(q_bits)
    requests = list(requests)
    workers = threads or min(16, max(1, len(os.sched_getaffinity(0))))
    host = {}
    kidx = {}
    want_ids = {}
    want_out = {}

    def quant(b):
        kidx[b] = F.dequantize(fmt, *F.quantize(fmt, host[b]["idx"]))

    def select(r):
        b = int(row_req[r])
        s = P.block_scores(qi[r], kidx[b], int(row_len[r]))
        want_ids[r] = P.topk_blocks(s, topk, tie_high, init_blocks, local_blocks)

    def attend(b):
        n = int(lay.seq_lens[b])
        rows = range(int(lay.cu_q[b]), int(lay.cu_q[b + 1]))
        need = sorted({int(j) for r in rows for j in want_ids[r] if j >= 0})
        kh = np.zeros((n, 128))
        vh = np.zeros((n, 128))
        for j in need:
            t = slice(j * 128, min(n, (j + 1) * 128))
            kh[t] = F.dequantize(fmt, *F.quantize(fmt, host[b]["k"][t]))
            vh[t] = F.dequantize(fmt, *F.quantize(fmt, host[b]["v"][t]))
        for r in rows:
            want_out[r] = P.attend_row(qm[r], kh, vh, want_ids[r], int(row_len[r]), sm_scale)

    with cf.ThreadPoolExecutor(workers) as ex:
        # batches of requests bound the host rows and dequantized planes held at once
        for i in range(0, len(requests), workers):
            batch = requests[i: i + workers]
            for b in batch:   # host copies of the request's rows (device tensors), serially
                lo, hi = int(lay.tok_off[b]), int(lay.tok_off[b + 1])
                host[b] = {n: W.bf16_bits(getattr(case, n)[lo:hi]) for n in ("idx", "k", "v")}
            list(ex.map(quant, batch))
            list(ex.map(select, [r for b in batch for r in range(int(lay.cu_q[b]), int(lay.cu_q[b + 1]))]))
            kidx.clear()
            list(ex.map(attend, batch))
            host.clear()
    return want_ids, want_out, row_req, row_len


def max_rel_err(got: np.ndarray, want: np.ndarray) -> float:
    """max over heads of ||got - want||_inf / ||want||_inf (rows of [G, 128])."""
    num = np.abs(got - want).max(axis=-1)
    den = np.abs(want).max(axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())
