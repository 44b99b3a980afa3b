"""The decode step in float64: store, row map, block scores, top-k, sparse attention.

Test infrastructure (see the package docstring): only the tests, the smoke
check and bench.py's CPU baseline may import this module.

Each function follows the pages:
  * store: quantize the step's rows and write them at their slots; a
    negative slot is a pad row and is left unwritten (ATOM PR "[MiniMax-M3.1]
    FP4 index cache and NVFP4 sparse KV cache", Write path and Tests).
  * decode_rows: each decode / verify row maps to (request, causal length)
    (ATOM PR "NVFP4 sparse KV", Summary, Attention).
  * block_scores: the index query of a row is scored against every causal
    128-token block of its request's index cache reached through the block
    table; a block's score is the max over its causal tokens of q_idx . k_idx
    (reading of the index score; the pages print no formula).
  * topk_blocks: the k best blocks; equal scores go to the lower block id by
    default (or to the higher id, the rule of the ATOM review notes on
    ``_pack_score_key``); ids are emitted ascending, padded with -1 (the review
    notes state that the fused top-k writes its ids in ascending order). Forced initial / local blocks (vLLM PR
    "MXFP4 KV + indexer cache for MiniMax-M3.1", Design; ATOM review notes on
    init_blocks + local_blocks > topk) rank above every scored block.
  * attend_row: softmax attention of the row's G query heads over the tokens
    of the selected blocks that are causal for the row, with the dequantized
    K/V (ATOM PR "NVFP4 sparse KV", Tests: the kernel is checked against
    attention computed on the dequantized cache).

Exactness of the scores: every dequantized NVFP4 key element has at most 6
significant bits and a bf16 query element 8, so each product is exact in
float64; the float64 sum of 128 products is exact whenever the sum of their
magnitudes stays below 2^53 times the smallest unit in the last place among
them. ``token_dots`` checks that condition for every token and recomputes any
token that fails it with ``math.fsum`` over the exact products, so the
scores, and therefore the top-k, are the exact-arithmetic ones.
"""
from __future__ import annotations

import math

import numpy as np

from . import formats as F

PAGE = 128


def decode_rows(cu_q, seq_lens, num_rows):
    """Row r in [cu_q[b], cu_q[b+1]) -> (b, seq_len[b] - q_len[b] + 1 + (r - cu_q[b])).

    Rows at or past cu_q[B] are padding: (-1, 0).
    """
    cu_q = [int(x) for x in cu_q]
    seq_lens = [int(x) for x in seq_lens]
    row_req = np.full(num_rows, -1, dtype=np.int32)
    row_len = np.zeros(num_rows, dtype=np.int32)
    for b in range(len(seq_lens)):
        q_len = cu_q[b + 1] - cu_q[b]
        for i in range(q_len):
            r = cu_q[b] + i
            n = seq_lens[b] - q_len + 1 + i
            if n < 1:
                raise ValueError("a row must see at least one token")
            row_req[r] = b
            row_len[r] = n
    return row_req, row_len


def prefill_rows(cu_q, seq_lens, num_rows):
    """Prefill rows: every query token of a request's chunk is a row and sees the request's
    prefix plus the chunk up to itself, the same map as ``decode_rows`` with no bound on a
    request's row count (the pages' prefill_rows, ATOM PR "[MiniMax-M3.1] FP4 index cache
    and NVFP4 sparse KV cache", Design: Row maps, which reports both device row maps agreeing
    with the torch mapping they replace)."""
    return decode_rows(cu_q, seq_lens, num_rows)


def new_planes(fmt: str, num_pages: int):
    """Zeroed plane set {name: (payload [P,128,64], scales [P,128,SB])}."""
    sb = F.scale_bytes(fmt)
    return {name: (np.zeros((num_pages, PAGE, F.PAYLOAD_BYTES), np.uint8),
                   np.zeros((num_pages, PAGE, sb), np.uint8)) for name in ("k", "v", "idx")}


def store(planes, fmt: str, rows: dict, slots):
    """Quantize rows[name] (bf16 bits [T,128]) and write each at slots[t] (skip slots < 0)."""
    slots = np.asarray(slots, dtype=np.int64)
    live = slots >= 0
    for name, bits in rows.items():
        if bits is None:
            continue
        pay, sc = F.quantize(fmt, np.asarray(bits)[live])
        s = slots[live]
        planes[name][0][s // PAGE, s % PAGE] = pay
        planes[name][1][s // PAGE, s % PAGE] = sc
    return planes


def gather_tokens(plane, fmt: str, bt_row, n: int):
    """Dequantized float64 [n, 128] of tokens 0..n-1 of one request (through its block table row)."""
    t = np.arange(n, dtype=np.int64)
    pages = np.asarray(bt_row, dtype=np.int64)[t // PAGE]
    if np.any(pages < 0):
        raise ValueError("block table entry < 0 inside the causal range")
    pay = plane[0][pages, t % PAGE]
    sc = plane[1][pages, t % PAGE]
    return F.dequantize(fmt, pay, sc)


def _lsb(x: np.ndarray) -> np.ndarray:
    """Unit in the last significant place of each non-zero float64 (inf for zeros)."""
    m, e = np.frexp(np.abs(x))
    mi = (m * 2.0 ** 53).astype(np.int64)
    low = mi & -mi
    out = np.ldexp(low.astype(np.float64), e.astype(np.int64) - 53)
    return np.where(x == 0, np.inf, out)


def token_dots(q: np.ndarray, khat: np.ndarray) -> np.ndarray:
    """Exact q . khat[t] for every token t (q [128] float64, khat [n,128] float64)."""
    dots = khat @ q
    mag = np.abs(khat) @ np.abs(q)
    lq = _lsb(q).min()
    lk = _lsb(khat).min(axis=-1)
    ok = mag < (2.0 ** 53) * lq * lk
    ok |= mag == 0
    for t in np.nonzero(~ok)[0]:
        dots[t] = math.fsum(float(a) * float(b) for a, b in zip(q, khat[t]))
    return dots


def block_scores(q: np.ndarray, khat: np.ndarray, row_len: int) -> np.ndarray:
    """Score of every causal block j < ceil(row_len / 128): max over its tokens t < row_len."""
    nb = (row_len + PAGE - 1) // PAGE
    d = token_dots(q, khat[:row_len])
    pad = np.full(nb * PAGE, -np.inf)
    pad[:row_len] = d
    s = pad.reshape(nb, PAGE).max(axis=1)
    return s + 0.0          # -0.0 -> +0.0: equal scores compare equal


def forced_class(nb: int, init_blocks: int = 0, local_blocks: int = 0) -> np.ndarray:
    """Per causal block: 2 for a forced initial block (id < init_blocks), 1 for a forced
    local block (one of the row's newest local_blocks blocks), else 0.

    Reading of the vLLM PR "MXFP4 KV + indexer cache for MiniMax-M3.1" (Design: the
    init / local sentinels 1e30 / 1e29 written on a row's causal blocks before its
    top-k) and of the ATOM review notes on init_blocks + local_blocks > topk: an
    initial block outranks a local one (its sentinel is the larger), both outrank every
    scored block, and a block that is both counts as initial.
    """
    j = np.arange(nb)
    cls = np.zeros(nb, dtype=np.int64)
    cls[j >= nb - local_blocks] = 1
    cls[j < init_blocks] = 2
    return cls


def topk_blocks(scores: np.ndarray, k: int, tie_high: bool = False, init_blocks: int = 0,
                local_blocks: int = 0) -> np.ndarray:
    """The k best blocks, emitted ascending, -1 padded.

    Order: forced class descending (``forced_class``); inside a forced class the higher
    id first (the ATOM review: with init + local > topk the newest local blocks, the
    row's own block among them, must be kept); among scored blocks score descending,
    then id ascending (descending with ``tie_high``).
    """
    nb = len(scores)
    ids = np.arange(nb)
    cls = forced_class(nb, init_blocks, local_blocks)
    s = np.asarray(scores, dtype=np.float64)
    tie = np.where(cls > 0, -ids, -ids if tie_high else ids)
    score_key = np.where(cls > 0, 0.0, -s)
    order = np.lexsort((tie, score_key, -cls))
    sel = np.sort(order[: min(k, nb)])
    out = np.full(k, -1, dtype=np.int32)
    out[: len(sel)] = sel
    return out


def selected_tokens(ids, row_len: int) -> np.ndarray:
    toks = []
    for j in ids:
        j = int(j)
        if j < 0:
            continue
        toks.append(np.arange(j * PAGE, min((j + 1) * PAGE, row_len)))
    return np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)


def attend_row(q: np.ndarray, khat: np.ndarray, vhat: np.ndarray, ids, row_len: int, sm_scale: float):
    """softmax(sm_scale * q khat^T) vhat over the causal tokens of the selected blocks.

    q [G,128] float64; khat / vhat: float64 rows indexed by token position.
    """
    t = selected_tokens(ids, row_len)
    if len(t) == 0:
        return np.zeros((q.shape[0], q.shape[1]))
    logits = sm_scale * (q @ khat[t].T)
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    return (p @ vhat[t]) / p.sum(axis=1, keepdims=True)


def request_rows(cu_q, b):
    return range(int(cu_q[b]), int(cu_q[b + 1]))


def step(planes, fmt, new_rows, new_slots, cu_q, seq_lens, block_table, q_idx_bits, q_bits,
         topk, sm_scale, num_rows=None, tie_high=False, requests=None, init_blocks=0, local_blocks=0):
    """One decode step: store -> decode_rows -> per row scores, top-k, attention.

    ``requests`` restricts the score / top-k / attention work to a subset of
    requests (rows of other requests are returned as -1 ids and zero output).
    Returns (row_req, row_len, topk_ids [R,k], out [R,G,128]).
    """
    store(planes, fmt, new_rows, new_slots)
    R = int(cu_q[-1]) if num_rows is None else num_rows
    row_req, row_len = decode_rows(cu_q, seq_lens, R)
    qi = F.bf16_to_f64(q_idx_bits)
    qm = F.bf16_to_f64(q_bits)
    G = qm.shape[1]
    ids = np.full((R, topk), -1, dtype=np.int32)
    out = np.zeros((R, G, F.HEAD_DIM))
    reqs = range(len(seq_lens)) if requests is None else requests
    for b in reqs:
        n = int(seq_lens[b])
        kidx = gather_tokens(planes["idx"], fmt, block_table[b], n)
        rows = list(request_rows(cu_q, b))
        sel = {}
        for r in rows:
            ids[r] = topk_blocks(block_scores(qi[r], kidx, int(row_len[r])), topk, tie_high, init_blocks,
                                 local_blocks)
            sel[r] = ids[r]
        need = sorted({int(j) for r in rows for j in sel[r] if j >= 0})
        kh = np.zeros((n, F.HEAD_DIM))
        vh = np.zeros((n, F.HEAD_DIM))
        if need:
            toks = np.concatenate([np.arange(j * PAGE, min((j + 1) * PAGE, n)) for j in need])
            pages = np.asarray(block_table[b], dtype=np.int64)[toks // PAGE]
            for name, dst in (("k", kh), ("v", vh)):
                pay = planes[name][0][pages, toks % PAGE]
                sc = planes[name][1][pages, toks % PAGE]
                dst[toks] = F.dequantize(fmt, pay, sc)
        for r in rows:
            out[r] = attend_row(qm[r], kh, vh, ids[r], int(row_len[r]), sm_scale)
    return row_req, row_len, ids, out
