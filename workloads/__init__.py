"""Seeded synthetic workloads for the NVFP4 / MXFP4 block-sparse decode step.

This module only draws inputs. It holds none of the method's arithmetic (no
quantization, scoring, selection or attention), so that both the HIP path and
the CPU oracle can be fed the same tensors from it without sharing any code.

Shapes follow the decode workloads of the MiniMax-M3 sparse layers described
in the ATOM pull request "[MiniMax-M3.1] FP4 index cache and NVFP4 sparse KV
cache" (Design and Results sections): one KV head and one index head per GPU,
head_dim 128, 128-token pages, 8 rows per request (one target row plus seven
draft rows, causal within the rows), G = 16 query heads per KV head, top-k 16
blocks, and 150K / 450K-token contexts.

Recipe (the same for every tensor family):
  * K, V and index-K rows: float32 N(0, 1); 2% of the 128 channels
    (round(0.02 * 128) = 3, chosen per tensor by the seeded numpy generator)
    are scaled by 8 for every token; then rounded to bfloat16 (RNE).
  * q (main query, [R, G, 128]) and q_idx (index query, [R, 128]):
    N(0, 1) / sqrt(128), rounded to bfloat16.
  * Block tables: the physical pages of all requests are a seeded random
    permutation of [0, num_pages); request b owns ceil(seq_len_b / 128)
    consecutive entries of that permutation. Unused table entries are -1.
  * Row layout: request b owns q_len rows; its tokens are 0 .. seq_len_b - 1,
    the last q_len of which are the step's new rows (stored during the step).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

PAGE = 128
HEAD_DIM = 128


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    seq_lens: tuple
    q_len: int
    G: int
    topk: int
    fmt: str  # "nvfp4" | "mxfp4"
    sm_scale: float = 1.0
    description: str = ""

    @property
    def num_reqs(self) -> int:
        return len(self.seq_lens)

    @property
    def num_rows(self) -> int:
        return self.num_reqs * self.q_len

    @property
    def seed(self) -> int:
        return self.index


def _lognormal_lens(seed: int, n: int) -> tuple:
    rng = np.random.default_rng(seed)
    x = np.exp(rng.normal(math.log(160_000.0), 0.5, size=n))
    x = np.clip(np.rint(x), 16_000, 450_000).astype(np.int64)
    return tuple(int(v) for v in x)


CONFIGS = (
    Config(0, "tiny_1x1_2k", (2048,), 1, 4, 4, "nvfp4",
           description="1 request x 1 row, 2048-token context in 16 pages, G=4, top-k 4"),
    Config(1, "b8x8_150k", (150_000,) * 8, 8, 16, 16, "nvfp4",
           description="8 requests x 8 rows, 150K context each, G=16, top-k 16, NVFP4"),
    Config(2, "b8x8_skew_450k", (450_000,) + (150_000,) * 7, 8, 16, 16, "nvfp4",
           description="8 requests x 8 rows, one 450K and seven 150K contexts"),
    Config(3, "b48x8_lognormal", _lognormal_lens(3, 48), 8, 16, 16, "nvfp4",
           description="48 requests x 8 rows, lognormal contexts (median 160K, sigma 0.5, clip 16K..450K)"),
    Config(4, "b8x8_150k_mxfp4", (150_000,) * 8, 8, 16, 16, "mxfp4",
           description="config b8x8_150k with MXFP4 planes (E8M0 scale per 32)"),
    Config(5, "prefill_1x4096_150k", (150_000,), 4096, 16, 16, "nvfp4",
           description="prefill: one request, a 4096-token chunk after a 145,904-token prefix, G=16, "
                       "top-k 16, NVFP4"),
)


def config(key) -> Config:
    if isinstance(key, int):
        return CONFIGS[key]
    for c in CONFIGS:
        if c.name == key:
            return c
    raise KeyError(key)


@dataclass
class Layout:
    """Host-side integer layout of one batch (numpy)."""
    seq_lens: np.ndarray      # int32 [B]
    q_lens: np.ndarray        # int32 [B]
    cu_q: np.ndarray          # int32 [B+1]
    nblk: np.ndarray          # int32 [B]   ceil(seq_len / 128)
    block_table: np.ndarray   # int32 [B, max_blocks], -1 where unused
    num_pages: int
    tok_off: np.ndarray       # int64 [B+1] offset of request b's tokens in the token-major arrays
    new_tokens: np.ndarray    # int64 [T_new] global token index of each step row
    new_slots: np.ndarray     # int32 [T_new]
    extra: dict = field(default_factory=dict)

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def total_tokens(self) -> int:
        return int(self.tok_off[-1])


def make_layout(seq_lens, q_len, seed: int, spare_pages: int = 0) -> Layout:
    """q_len: rows per request, one value for all or one per request (prefill chunks)."""
    seq = np.asarray(seq_lens, dtype=np.int64)
    B = len(seq)
    ql = np.broadcast_to(np.asarray(q_len, dtype=np.int32), (B,)).copy()
    if np.any(seq < ql):
        raise ValueError("seq_len must be >= q_len")
    nblk = (seq + PAGE - 1) // PAGE
    max_blocks = int(nblk.max())
    num_pages = int(nblk.sum()) + spare_pages
    rng = np.random.default_rng(seed + 1000)
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, : nblk[b]] = perm[off: off + nblk[b]]
        off += int(nblk[b])
    cu_q = np.zeros(B + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(ql)
    tok_off = np.zeros(B + 1, dtype=np.int64)
    tok_off[1:] = np.cumsum(seq)
    new_tok, new_slot = [], []
    for b in range(B):
        for i in range(int(ql[b])):
            t = int(seq[b]) - int(ql[b]) + i
            new_tok.append(int(tok_off[b]) + t)
            new_slot.append(int(bt[b, t // PAGE]) * PAGE + t % PAGE)
    return Layout(seq.astype(np.int32), ql, cu_q, nblk.astype(np.int32), bt, num_pages,
                  tok_off, np.asarray(new_tok, dtype=np.int64), np.asarray(new_slot, dtype=np.int32))


def all_slots(layout: Layout) -> np.ndarray:
    """int32 slot of every token (token-major order of the generated arrays)."""
    out = np.empty(layout.total_tokens, dtype=np.int32)
    for b in range(len(layout.seq_lens)):
        n = int(layout.seq_lens[b])
        t = np.arange(n, dtype=np.int64)
        pages = layout.block_table[b, t // PAGE].astype(np.int64)
        out[layout.tok_off[b]: layout.tok_off[b] + n] = (pages * PAGE + t % PAGE).astype(np.int32)
    return out


def outlier_channels(seed: int, which: int, n: int = 3) -> np.ndarray:
    rng = np.random.default_rng([seed, 7, which])
    return np.sort(rng.choice(HEAD_DIM, size=n, replace=False))


def _torch():
    import torch
    return torch


def gen_rows(num_tokens: int, seed: int, which: int, device="cpu", chunk: int = 1 << 20):
    """bf16 [num_tokens, 128] rows ~ N(0,1) with 3 outlier channels x8 (tensor family `which`)."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 100 + int(which))
    ch = torch.as_tensor(outlier_channels(seed, which), device=device)
    out = torch.empty((num_tokens, HEAD_DIM), dtype=torch.bfloat16, device=device)
    for s in range(0, num_tokens, chunk):
        e = min(num_tokens, s + chunk)
        x = torch.randn((e - s, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
        x[:, ch] *= 8.0
        out[s:e] = x.to(torch.bfloat16)
    return out


def gen_queries(shape, seed: int, which: int, device="cpu"):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 100 + 50 + int(which))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return (x / math.sqrt(HEAD_DIM)).to(torch.bfloat16)


K_FAMILY, V_FAMILY, IDX_FAMILY = 0, 1, 2
Q_FAMILY, QIDX_FAMILY = 0, 1


@dataclass
class Case:
    cfg: Config
    layout: Layout
    k: object      # torch bf16 [total_tokens, 128] (all tokens, token-major per request)
    v: object
    idx: object
    q: object      # torch bf16 [R, G, 128]
    q_idx: object  # torch bf16 [R, 128]


def make_case(cfg: Config, device="cpu", seq_lens=None, q_len=None, G=None) -> Case:
    seq = cfg.seq_lens if seq_lens is None else tuple(seq_lens)
    ql = cfg.q_len if q_len is None else q_len
    g = cfg.G if G is None else G
    lay = make_layout(seq, ql, cfg.seed)
    n = lay.total_tokens
    R = int(lay.cu_q[-1])
    k = gen_rows(n, cfg.seed, K_FAMILY, device)
    v = gen_rows(n, cfg.seed, V_FAMILY, device)
    idx = gen_rows(n, cfg.seed, IDX_FAMILY, device)
    q = gen_queries((R, g, HEAD_DIM), cfg.seed, Q_FAMILY, device)
    q_idx = gen_queries((R, HEAD_DIM), cfg.seed, QIDX_FAMILY, device)
    return Case(cfg, lay, k, v, idx, q, q_idx)


def bf16_bits(t) -> np.ndarray:
    """uint16 numpy view of a torch bfloat16 tensor (copied to host)."""
    torch = _torch()
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------------------
# inputs of the fused producer store (pre-norm rows, norm weights, angle table)
# ---------------------------------------------------------------------------

def gen_norm_weights(seed: int, device="cpu"):
    """bf16 [4, 128] RMS-norm weights (query, key, index query, index key):
    1 + 0.1 N(0, 1), rounded to bf16."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 100 + 80)
    w = 1.0 + 0.1 * torch.randn((4, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
    return w.to(torch.bfloat16)


def gen_prenorm_rows(shape, seed: int, which: int, device="cpu"):
    """bf16 pre-norm rows [..., 128]: N(0, 1) times a per-row scale drawn
    log-uniformly from [1/4, 16], with the tensor family's 3 outlier channels x8."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 100 + 60 + int(which))
    shape = tuple(shape)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    ch = torch.as_tensor(outlier_channels(seed, 10 + which), device=device)
    x[..., ch] *= 8.0
    u = torch.rand(shape[:-1] + (1,), generator=g, device=device, dtype=torch.float32)
    x = x * torch.exp2(u * 6.0 - 2.0)
    return x.to(torch.bfloat16)


def rope_table(max_pos: int, rotary_dim: int, base: float = 10000.0) -> np.ndarray:
    """float32 [max_pos, rotary_dim]: cos(p * t_d) in columns [0, rd/2) and
    sin(p * t_d) in [rd/2, rd), t_d = base^(-2d / rd), computed in float64 and
    rounded to float32 (an input of the producer, like its weights)."""
    h = rotary_dim // 2
    if h == 0:
        return np.zeros((max_pos, 0), dtype=np.float32)
    t = base ** (-2.0 * np.arange(h, dtype=np.float64) / rotary_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * t[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


PQ_FAMILY, PK_FAMILY, PV_FAMILY, PIQ_FAMILY, PIK_FAMILY = 0, 1, 2, 3, 4


def new_positions(layout: Layout) -> np.ndarray:
    """int32 position (token index in its request) of every step row."""
    out = []
    for b in range(len(layout.seq_lens)):
        s, q = int(layout.seq_lens[b]), int(layout.q_lens[b])
        out.extend(range(s - q, s))
    return np.asarray(out, dtype=np.int32)
