"""CPU oracle of the NVFP4 / MXFP4 block-sparse decode step (test infrastructure).

This package is the plain, slow, float64 / exact-rational statement of what
the decode hot path computes. It is test infrastructure: only the tests, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py``
may import it. It shares no code with the HIP library and imports nothing
from it; the two meet only through the seeded inputs of ``workloads``.

Sources (the pages):
  * ATOM PR "NVFP4 sparse KV" (Summary): 64 B e2m1 payload + 8 B E4M3 block
    scales per token and KV head; decode rows carry (request, causal length);
    attention reads the top-k block ids through the request block table.
  * ATOM PR "[MiniMax-M3.1] FP4 index cache and NVFP4 sparse KV cache"
    (Design, Write path): per 16 elements scale = e4m3(amax / 6), codes
    rounded half-to-even and saturating at 6; (Follow-up: MXFP4 caches): one
    E8M0 scale per 32 elements; (review notes): ties of equal block score and
    ascending id order of the fused top-k.
  * vLLM PR "MXFP4 KV + indexer cache for MiniMax-M3.1" (Claims): 68 B per
    token and head, page = [128 x 64 B][128 x 4 B].

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
(hand-worked cases in ``tests/golden/``, closed forms, exhaustive integer
cross-checks, brute force and library special cases). No function is left
"parity unpinned".
"""
from . import formats, path  # noqa: F401
