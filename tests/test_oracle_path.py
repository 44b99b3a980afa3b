"""Pins of the oracle's step (row map, scores, top-k, attention) against closed forms,
brute force and library special cases. CPU only; nothing here calls the HIP library."""
import itertools
import math
from fractions import Fraction as Fr

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import path as P
from workloads import bf16_bits, make_case, config
from tests.goldens import to_bf16_bits


# --- decode_rows ---------------------------------------------------------------

def test_decode_rows_hand_example():
    cu_q = [0, 3, 4, 8]
    seq = [10, 5, 128]
    rr, rl = P.decode_rows(cu_q, seq, 10)
    assert rr.tolist() == [0, 0, 0, 1, 2, 2, 2, 2, -1, -1]
    assert rl.tolist() == [8, 9, 10, 5, 125, 126, 127, 128, 0, 0]


def test_decode_rows_matches_torch_mapping():
    rng = np.random.default_rng(3)
    for _ in range(20):
        B = int(rng.integers(1, 30))
        ql = rng.integers(1, 17, size=B)
        seq = ql + rng.integers(0, 5000, size=B)
        cu = np.concatenate([[0], np.cumsum(ql)])
        R = int(cu[-1] + rng.integers(0, 9))
        rr, rl = P.decode_rows(cu, seq, R)
        # torch formulation: request id by repeat_interleave, position by subtraction
        qlt = torch.as_tensor(ql)
        req = torch.repeat_interleave(torch.arange(B), qlt)
        pos = torch.arange(int(cu[-1])) - torch.as_tensor(cu[:-1])[req]
        ln = torch.as_tensor(seq)[req] - qlt[req] + 1 + pos
        assert rr[: cu[-1]].tolist() == req.tolist()
        assert rl[: cu[-1]].tolist() == ln.tolist()
        assert np.all(rr[cu[-1]:] == -1) and np.all(rl[cu[-1]:] == 0)


def test_decode_rows_rejects_short_context():
    with pytest.raises(ValueError):
        P.decode_rows([0, 4], [3], 4)


# --- scores --------------------------------------------------------------------

def _exact_scores(qbits, pay, sc, fmt, row_len):
    """Brute force with Fractions: max over causal tokens of the exact dot product."""
    q = [F.bf16_value(int(b)) for b in qbits]
    gsz = 16 if fmt == "nvfp4" else 32
    dec = F.e4m3fn_value if fmt == "nvfp4" else F.e8m0_value
    nb = (row_len + 127) // 128
    out = []
    for j in range(nb):
        best = None
        for t in range(j * 128, min((j + 1) * 128, row_len)):
            acc = Fr(0)
            for d in range(128):
                c = (int(pay[t, d // 2]) >> (4 * (d % 2))) & 0xF
                acc += q[d] * F.e2m1_value(c) * dec(int(sc[t, d // gsz]))
            best = acc if best is None or acc > best else best
        out.append(best)
    return out


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_block_scores_equal_exact_rationals(fmt):
    rng = np.random.default_rng(1)
    n = 300
    x = rng.standard_normal((n, 128))
    x[:, [5, 6, 90]] *= 8
    kb = to_bf16_bits(x.ravel()).reshape(n, 128)
    pay, sc = F.quantize(fmt, kb)
    khat = F.dequantize(fmt, pay, sc)
    qb = to_bf16_bits(rng.standard_normal(128) / math.sqrt(128))
    for row_len in (1, 127, 128, 129, 300):
        got = P.block_scores(F.bf16_to_f64(qb), khat, row_len)
        want = _exact_scores(qb, pay, sc, fmt, row_len)
        assert len(got) == len(want) == (row_len + 127) // 128
        assert [Fr(float(g)) for g in got] == want


def test_token_dots_exact_when_sum_needs_more_than_53_bits():
    """A query with a huge dynamic range makes the plain float64 sum round;
    the oracle must detect it and still return the exact value."""
    q = np.zeros(128)
    q[0] = 2.0 ** 60
    q[1] = 1.0
    q[2] = -(2.0 ** 60)
    k = np.zeros((1, 128))
    k[0, 0] = 1.0
    k[0, 1] = 1.0
    k[0, 2] = 1.0
    # exact: 2^60 + 1 - 2^60 = 1 ; a naive left-to-right float64 sum gives 0
    assert P.token_dots(q, k)[0] == 1.0


def test_scores_ignore_non_causal_tokens():
    khat = np.zeros((256, 128))
    khat[200, 0] = 100.0                     # would dominate block 1 if it were causal
    khat[150, 0] = 1.0
    q = np.zeros(128)
    q[0] = 1.0
    s = P.block_scores(q, khat, 180)
    assert s.tolist() == [0.0, 1.0]


# --- top-k ---------------------------------------------------------------------

def _brute_topk(scores, k, tie_high):
    """The unique subset whose members all beat all non-members under (score, id rule)."""
    n = len(scores)
    if n <= k:
        return list(range(n))

    def beats(a, b):
        if scores[a] != scores[b]:
            return scores[a] > scores[b]
        return a > b if tie_high else a < b

    found = []
    for S in itertools.combinations(range(n), k):
        rest = set(range(n)) - set(S)
        if all(beats(a, b) for a in S for b in rest):
            found.append(list(S))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("tie_high", [False, True])
def test_topk_brute_force_small(tie_high):
    rng = np.random.default_rng(4)
    for trial in range(60):
        n = int(rng.integers(1, 11))
        k = int(rng.integers(1, 6))
        scores = rng.integers(-3, 4, size=n).astype(np.float64)   # many exact ties
        if trial % 5 == 0:
            scores[:] = 0.0
        got = P.topk_blocks(scores, k, tie_high)
        want = sorted(_brute_topk(list(scores), k, tie_high))
        assert got.tolist() == want + [-1] * (k - len(want))


def test_topk_zero_query_selects_lowest_ids():
    # zero query: every score is 0, the lower-id rule selects 0..k-1
    assert P.topk_blocks(np.zeros(1172), 16).tolist() == list(range(16))
    assert P.topk_blocks(np.zeros(1172), 16, tie_high=True).tolist() == list(range(1156, 1172))


def test_topk_signed_zero_is_a_tie():
    s = np.array([-0.0, 0.0, -0.0, -1.0])
    assert P.topk_blocks(s + 0.0, 2).tolist() == [0, 1]


def test_topk_fewer_blocks_than_k():
    assert P.topk_blocks(np.array([3.0, 1.0, 2.0]), 5).tolist() == [0, 1, 2, -1, -1]


def test_topk_output_is_ascending_not_score_order():
    s = np.array([1.0, 9.0, 5.0, 7.0])
    assert P.topk_blocks(s, 3).tolist() == [1, 2, 3]


# --- attention -----------------------------------------------------------------

def _planes_for(seq_len, seed=0, fmt="nvfp4"):
    lay_case = make_case(config(0), "cpu", seq_lens=[seq_len], q_len=1)
    lay = lay_case.layout
    planes = P.new_planes(fmt, lay.num_pages)
    from workloads import all_slots
    slots = all_slots(lay)
    P.store(planes, fmt, {"k": bf16_bits(lay_case.k), "v": bf16_bits(lay_case.v),
                          "idx": bf16_bits(lay_case.idx)}, slots)
    return lay_case, planes


@pytest.mark.parametrize("seq_len", [1, 200, 640])
def test_attend_all_blocks_equals_dense_sdpa(seq_len):
    """top-k covering every causal block reproduces dense softmax attention over the
    dequantized cache (torch scaled_dot_product_attention in float64)."""
    case, planes = _planes_for(seq_len)
    lay = case.layout
    kh = P.gather_tokens(planes["k"], "nvfp4", lay.block_table[0], seq_len)
    vh = P.gather_tokens(planes["v"], "nvfp4", lay.block_table[0], seq_len)
    q = F.bf16_to_f64(bf16_bits(case.q[0]))           # [G,128]
    nb = (seq_len + 127) // 128
    ids = np.arange(nb)
    out = P.attend_row(q, kh, vh, ids, seq_len, 0.37)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(q)[None, :, None, :],
        torch.as_tensor(kh)[None, None].expand(1, q.shape[0], -1, -1),
        torch.as_tensor(vh)[None, None].expand(1, q.shape[0], -1, -1),
        scale=0.37)[0, :, 0, :].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_attend_single_token_returns_v0():
    case, planes = _planes_for(300)
    lay = case.layout
    kh = P.gather_tokens(planes["k"], "nvfp4", lay.block_table[0], 300)
    vh = P.gather_tokens(planes["v"], "nvfp4", lay.block_table[0], 300)
    q = F.bf16_to_f64(bf16_bits(case.q[0]))
    out = P.attend_row(q, kh, vh, [0, -1, -1], 1, 1.0)
    assert np.array_equal(out, np.broadcast_to(vh[0], out.shape))


def test_attend_zero_query_is_mean_of_selected_causal_tokens():
    case, planes = _planes_for(600)
    lay = case.layout
    kh = P.gather_tokens(planes["k"], "nvfp4", lay.block_table[0], 600)
    vh = P.gather_tokens(planes["v"], "nvfp4", lay.block_table[0], 600)
    out = P.attend_row(np.zeros((4, 128)), kh, vh, [1, 4], 590, 1.0)
    toks = list(range(128, 256)) + list(range(512, 590))
    assert np.allclose(out, vh[toks].mean(axis=0)[None], rtol=1e-13, atol=1e-15)


def test_step_invariant_under_page_permutation_and_id_order():
    cfg = config(0)
    case = make_case(cfg, "cpu", seq_lens=[700, 300], q_len=3, G=4)
    lay = case.layout
    from workloads import all_slots
    bits = {n: bf16_bits(getattr(case, n)) for n in ("k", "v", "idx")}
    hist = np.ones(lay.total_tokens, bool)
    hist[lay.new_tokens] = False

    def run(bt):
        slots = np.empty(lay.total_tokens, np.int32)
        for b in range(2):
            t = np.arange(int(lay.seq_lens[b]))
            slots[lay.tok_off[b]: lay.tok_off[b + 1]] = bt[b, t // 128] * 128 + t % 128
        planes = P.new_planes("nvfp4", lay.num_pages)
        P.store(planes, "nvfp4", {n: b[hist] for n, b in bits.items()}, slots[hist])
        new = {n: b[lay.new_tokens] for n, b in bits.items()}
        return P.step(planes, "nvfp4", new, slots[lay.new_tokens], lay.cu_q, lay.seq_lens, bt,
                      bf16_bits(case.q_idx), bf16_bits(case.q), 3, 0.5)

    a = run(lay.block_table)
    perm = np.random.default_rng(9).permutation(lay.num_pages).astype(np.int32)
    bt2 = np.where(lay.block_table >= 0, perm[np.maximum(lay.block_table, 0)], -1)
    b = run(bt2)
    assert np.array_equal(a[2], b[2])
    assert np.allclose(a[3], b[3], rtol=0, atol=1e-14)
    # id order inside a row does not change attention
    case_planes = _planes_for(700)
    kh = P.gather_tokens(case_planes[1]["k"], "nvfp4", case_planes[0].layout.block_table[0], 700)
    vh = P.gather_tokens(case_planes[1]["v"], "nvfp4", case_planes[0].layout.block_table[0], 700)
    q = F.bf16_to_f64(bf16_bits(case_planes[0].q[0]))
    o1 = P.attend_row(q, kh, vh, [0, 2, 5], 700, 1.0)
    o2 = P.attend_row(q, kh, vh, [5, 0, 2], 700, 1.0)
    assert np.allclose(o1, o2, rtol=0, atol=1e-14)


def test_step_matches_brute_force_tiny():
    """The whole step on a tiny batch against a from-scratch computation: Fraction
    block scores, brute-force subset top-k and a dense softmax over the chosen tokens."""
    case = make_case(config(0), "cpu", seq_lens=[300, 260], q_len=2, G=2)
    lay = case.layout
    from workloads import all_slots
    slots = all_slots(lay)
    bits = {n: bf16_bits(getattr(case, n)) for n in ("k", "v", "idx")}
    hist = np.ones(lay.total_tokens, bool)
    hist[lay.new_tokens] = False
    planes = P.new_planes("nvfp4", lay.num_pages)
    P.store(planes, "nvfp4", {n: b[hist] for n, b in bits.items()}, slots[hist])
    new = {n: b[lay.new_tokens] for n, b in bits.items()}
    rr, rl, ids, out = P.step(planes, "nvfp4", new, slots[lay.new_tokens], lay.cu_q, lay.seq_lens,
                              lay.block_table, bf16_bits(case.q_idx), bf16_bits(case.q), 2, 1.0)
    qi = bf16_bits(case.q_idx)
    qm = F.bf16_to_f64(bf16_bits(case.q))
    for r in range(4):
        b = int(rr[r])
        toks = slice(lay.tok_off[b], lay.tok_off[b + 1])
        pay, sc = F.quantize("nvfp4", bits["idx"][toks])
        ex = _exact_scores(qi[r], pay, sc, "nvfp4", int(rl[r]))
        want = sorted(_brute_topk(ex, 2, False))
        assert ids[r].tolist() == want
        kp, ks = F.quantize("nvfp4", bits["k"][toks])
        vp, vs = F.quantize("nvfp4", bits["v"][toks])
        kh, vh = F.dequantize("nvfp4", kp, ks), F.dequantize("nvfp4", vp, vs)
        t = [x for j in want for x in range(j * 128, min(j * 128 + 128, int(rl[r])))]
        lg = qm[r] @ kh[t].T
        p = np.exp(lg - lg.max(1, keepdims=True))
        ref = (p / p.sum(1, keepdims=True)) @ vh[t]
        assert np.allclose(out[r], ref, rtol=1e-12, atol=1e-14)


# ---- forced initial / local blocks (vLLM PR "MXFP4 KV + indexer cache for MiniMax-M3.1",
# Design; ATOM PR "[MiniMax-M3.1] FP4 index cache and NVFP4 sparse KV cache", review
# notes on init_blocks + local_blocks > topk). Expected selections worked by hand.

def test_forced_review_example_keeps_newest_local_blocks():
    """topk 16, init 4, local 16 on a long row: the review's failing kernel picked 0-3 and
    n-16..n-5; the kept set must be the 4 initial blocks and the 12 newest local ones,
    the row's own block n-1 among them."""
    n = 100
    scores = np.arange(n, dtype=np.float64)[::-1].copy()  # real scores favour low ids
    got = P.topk_blocks(scores, 16, init_blocks=4, local_blocks=16).tolist()
    assert got == [0, 1, 2, 3] + list(range(88, 100))
    assert n - 1 in got


def test_forced_blocks_fit_then_best_scores_fill():
    """init 2 + local 3 <= k 8 on 20 blocks with score = id: forced {0, 1, 17, 18, 19},
    then the best scored blocks 16, 15, 14."""
    scores = np.arange(20, dtype=np.float64)
    assert P.topk_blocks(scores, 8, init_blocks=2, local_blocks=3).tolist() == [0, 1, 14, 15, 16, 17, 18, 19]


def test_forced_overlap_counts_as_initial():
    """5 blocks, init 4, local 3, k 4: blocks 2, 3 are both; as initial blocks they rank
    with 0, 1 above the local block 4."""
    scores = np.array([0.0, 0.0, 0.0, 0.0, 9.0])
    assert P.topk_blocks(scores, 4, init_blocks=4, local_blocks=3).tolist() == [0, 1, 2, 3]
    assert P.forced_class(5, 4, 3).tolist() == [2, 2, 2, 2, 1]


def test_forced_ties_go_to_higher_ids_even_with_low_id_rule():
    """init 10 > k 4: the 4 highest initial ids are kept, whatever the scored tie rule."""
    scores = np.zeros(30)
    for tie_high in (False, True):
        assert P.topk_blocks(scores, 4, tie_high, init_blocks=10).tolist() == [6, 7, 8, 9]
    assert P.topk_blocks(scores, 4, local_blocks=10).tolist() == [26, 27, 28, 29]


def test_forced_blocks_outrank_any_score():
    scores = np.full(12, -1.0)
    scores[5] = 1e300
    assert P.topk_blocks(scores, 3, init_blocks=1, local_blocks=1).tolist() == [0, 5, 11]
    assert P.topk_blocks(scores, 2, init_blocks=1, local_blocks=1).tolist() == [0, 11]


def test_forced_zero_is_plain_topk_and_short_rows_take_all():
    rng = np.random.default_rng(3)
    s = rng.standard_normal(50)
    assert P.topk_blocks(s, 7).tolist() == P.topk_blocks(s, 7, init_blocks=0, local_blocks=0).tolist()
    assert P.topk_blocks(s[:5], 8, init_blocks=3, local_blocks=3).tolist() == [0, 1, 2, 3, 4, -1, -1, -1]


def test_prefill_rows_hand_example():
    """Request 0: prefix 5, chunk 3 (seq 8) -> rows 0-2 see 6, 7, 8 tokens; request 1: no
    prefix, chunk 40 -> rows 3-42 see 1..40; rows 43, 44 are padding."""
    rr, rl = P.prefill_rows([0, 3, 43], [8, 40], 45)
    assert rr.tolist() == [0] * 3 + [1] * 40 + [-1, -1]
    assert rl.tolist() == [6, 7, 8] + list(range(1, 41)) + [0, 0]


def test_prefill_rows_match_searchsorted():
    """The pages compute prefill rows with searchsorted over the chunk offsets."""
    rng = np.random.default_rng(4)
    q = rng.integers(1, 300, 7)
    cu = np.concatenate([[0], np.cumsum(q)])
    seq = q + rng.integers(0, 5000, 7)
    R = int(cu[-1]) + 3
    rr, rl = P.prefill_rows(cu, seq, R)
    r = np.arange(int(cu[-1]))
    b = np.searchsorted(cu, r, side="right") - 1
    assert np.array_equal(rr[: len(r)], b)
    assert np.array_equal(rl[: len(r)], seq[b] - (cu[b + 1] - cu[b]) + 1 + (r - cu[b]))
