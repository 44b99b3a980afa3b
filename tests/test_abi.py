"""The C-ABI library loads on a CPU-only host, exports every symbol include/m3s.h
declares, and its host-side validation rejects bad arguments without touching
the GPU (every call below returns before any HIP call)."""
import ctypes
import os
import re

import pytest

import block_sparse_decode_nvfp4_amd as m3s
from block_sparse_decode_nvfp4_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "m3s.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(m3s.LIB_PATH):
        _build.build()
    return m3s.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(m3s_[a-z_]+)\s*\(", src)))


def test_header_declares_the_four_calls_and_helpers():
    names = declared_functions()
    for n in ("m3s_store", "m3s_decode_rows", "m3s_prefill_rows", "m3s_index_topk", "m3s_sparse_attend"):
        assert n in names
    assert set(names) == set(m3s.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert m3s.m3s_version() == 1
    for s in range(5):
        assert m3s.m3s_status_string(s)
    assert m3s.m3s_status_string(99) == "unknown status"


def _cache(fmt=1, pages=4, page=128, dim=128, heads=1, ptr=4096):
    return m3s.m3s_cache(fmt, pages, page, dim, heads, ptr, ptr, ptr, ptr, ptr, ptr)


def _rows(nreq=1, nrows=1, ptr=4096):
    return m3s.m3s_rows(ptr, None, ptr, ptr, ptr, nreq, nrows)


FAKE = ctypes.c_void_p(4096)   # never dereferenced: validation fails first or the call is not made


def test_store_validation(lib):
    c = _cache()
    E = m3s
    st = lambda cache, k=FAKE, stride=128, slots=FAKE, T=4: lib.m3s_store(
        ctypes.byref(cache) if cache is not None else None, k, k, k, stride, slots, T, None, None)
    assert st(None) == E.ERR_INVALID_ARG
    assert st(_cache(fmt=3)) == E.ERR_UNSUPPORTED
    assert st(_cache(page=256)) == E.ERR_UNSUPPORTED            # 256-token pages are refused
    assert st(_cache(dim=64)) == E.ERR_UNSUPPORTED
    assert st(_cache(heads=2)) == E.ERR_UNSUPPORTED
    assert st(_cache(pages=-1)) == E.ERR_INVALID_ARG
    assert st(c, T=-1) == E.ERR_INVALID_ARG
    assert st(c, T=0) == E.OK                                   # nothing to do, no launch
    assert st(c, slots=None) == E.ERR_INVALID_ARG
    assert st(c, stride=64) == E.ERR_INVALID_ARG
    assert st(c, stride=130) == E.ERR_INVALID_ARG               # rows must stay 16 B aligned
    assert st(c, k=ctypes.c_void_p(4098)) == E.ERR_INVALID_ARG  # misaligned source
    c2 = _cache()
    c2.v_scale = None
    assert st(c2) == E.ERR_INVALID_ARG


def test_decode_rows_validation(lib):
    f = lambda cu=FAKE, seq=FAKE, B=1, R=1, rr=FAKE, rl=FAKE, rb=FAKE: lib.m3s_decode_rows(
        cu, seq, B, R, rr, rl, rb, None, None)
    assert f(B=-1) == m3s.ERR_INVALID_ARG
    assert f(R=-1) == m3s.ERR_INVALID_ARG
    assert f(B=4097) == m3s.ERR_UNSUPPORTED
    assert f(R=65537) == m3s.ERR_UNSUPPORTED
    assert f(cu=None) == m3s.ERR_INVALID_ARG
    assert f(seq=None) == m3s.ERR_INVALID_ARG
    assert f(rr=None) == m3s.ERR_INVALID_ARG
    assert f(rb=None) == m3s.ERR_INVALID_ARG


def _topk(lib, cache=None, q=FAKE, qs=128, bt=FAKE, bts=16, mb=16, rows=None, k=4, flags=0, ids=FAKE,
          ws=FAKE, wsb=1 << 30, init=0, local=0):
    cache = _cache() if cache is None else cache
    rows = _rows() if rows is None else rows
    return lib.m3s_index_topk(ctypes.byref(cache), q, qs, bt, bts, mb, ctypes.byref(rows), k, flags, init, local,
                              ids, ws, wsb, None, None)


def test_index_topk_validation(lib):
    E = m3s
    assert _topk(lib, cache=_cache(page=64)) == E.ERR_UNSUPPORTED
    assert _topk(lib, k=0) == E.ERR_UNSUPPORTED
    assert _topk(lib, k=65) == E.ERR_UNSUPPORTED
    assert _topk(lib, flags=2) == E.ERR_INVALID_ARG
    assert _topk(lib, init=-1) == E.ERR_INVALID_ARG
    assert _topk(lib, local=-1) == E.ERR_INVALID_ARG
    assert _topk(lib, init=8193) == E.ERR_INVALID_ARG
    assert _topk(lib, mb=0) == E.ERR_INVALID_ARG
    assert _topk(lib, bts=8, mb=16) == E.ERR_INVALID_ARG
    assert _topk(lib, bts=9000, mb=8193) == E.ERR_UNSUPPORTED
    assert _topk(lib, bt=None) == E.ERR_INVALID_ARG
    assert _topk(lib, q=None) == E.ERR_INVALID_ARG
    assert _topk(lib, qs=100) == E.ERR_INVALID_ARG
    assert _topk(lib, ids=None) == E.ERR_INVALID_ARG
    assert _topk(lib, rows=_rows(nreq=-1)) == E.ERR_INVALID_ARG
    assert _topk(lib, rows=_rows(nreq=5000)) == E.ERR_UNSUPPORTED
    need = m3s.m3s_workspace_bytes(m3s.OP_INDEX_TOPK, 1, 1, 16, 4, 1)
    assert need > 0
    assert _topk(lib, wsb=need - 1) == E.ERR_WORKSPACE
    assert _topk(lib, ws=None) == E.ERR_WORKSPACE
    assert _topk(lib, rows=_rows(nrows=0)) == E.OK              # no rows: nothing launched


def _attend(lib, cache=None, q=FAKE, qrs=2048, qhs=128, G=16, bt=FAKE, bts=16, mb=16, rows=None, ids=FAKE,
            k=16, scale=1.0, out=FAKE, ws=FAKE, wsb=1 << 30):
    cache = _cache() if cache is None else cache
    rows = _rows() if rows is None else rows
    return lib.m3s_sparse_attend(ctypes.byref(cache), q, qrs, qhs, G, bt, bts, mb, ctypes.byref(rows), ids, k,
                                 scale, out, ws, wsb, None, None)


def test_sparse_attend_validation(lib):
    E = m3s
    assert _attend(lib, G=0) == E.ERR_UNSUPPORTED
    assert _attend(lib, G=17) == E.ERR_UNSUPPORTED
    assert _attend(lib, k=65) == E.ERR_UNSUPPORTED
    assert _attend(lib, scale=float("nan")) == E.ERR_INVALID_ARG
    assert _attend(lib, qhs=64) == E.ERR_INVALID_ARG
    assert _attend(lib, qrs=2050) == E.ERR_INVALID_ARG
    assert _attend(lib, out=None) == E.ERR_INVALID_ARG
    assert _attend(lib, ids=None) == E.ERR_INVALID_ARG
    c = _cache()
    c.k_scale = None
    assert _attend(lib, cache=c) == E.ERR_INVALID_ARG
    need = m3s.m3s_workspace_bytes(m3s.OP_SPARSE_ATTEND, 1, 1, 16, 16, 16)
    assert need > 0
    assert _attend(lib, wsb=need - 1) == E.ERR_WORKSPACE
    # four or fewer blocks fit one split: no workspace needed
    assert m3s.m3s_workspace_bytes(m3s.OP_SPARSE_ATTEND, 1, 1, 16, 4, 16) == 0
    assert _attend(lib, rows=_rows(nrows=0)) == E.OK


def test_workspace_sizes_scale_with_shape(lib):
    a = m3s.m3s_workspace_bytes(m3s.OP_INDEX_TOPK, 64, 8, 1172, 16, 16)
    assert a >= 2 * 64 * 1172 * 4
    b = m3s.m3s_workspace_bytes(m3s.OP_SPARSE_ATTEND, 64, 8, 1172, 16, 16)
    assert b >= 64 * 4 * 16 * 128 * 4
    assert m3s.m3s_workspace_bytes(99, 1, 1, 1, 1, 1) == 0
    assert m3s.m3s_workspace_bytes(m3s.OP_INDEX_TOPK, 1, 1, 1, 0, 1) == 0


def test_prefill_rows_validation(lib):
    f = lambda cu=FAKE, seq=FAKE, B=1, R=1, G=4, rr=FAKE, rl=FAKE, gr=FAKE, gq=FAKE, gb=FAKE: lib.m3s_prefill_rows(
        cu, seq, B, R, G, rr, rl, gr, gq, gb, None, None)
    E = m3s
    assert f(B=-1) == E.ERR_INVALID_ARG
    assert f(R=-1) == E.ERR_INVALID_ARG
    assert f(B=4097) == E.ERR_UNSUPPORTED
    assert f(R=65537) == E.ERR_UNSUPPORTED
    assert f(G=0) == E.ERR_UNSUPPORTED
    assert f(G=4097) == E.ERR_UNSUPPORTED
    assert f(cu=None) == E.ERR_INVALID_ARG
    assert f(seq=None) == E.ERR_INVALID_ARG
    assert f(gr=None) == E.ERR_INVALID_ARG
    assert f(gq=None) == E.ERR_INVALID_ARG
    assert f(gb=None) == E.ERR_INVALID_ARG
    assert f(rr=None) == E.ERR_INVALID_ARG



def test_store_and_rows_validation(lib):
    E = m3s
    f = lambda cache=None, k=FAKE, stride=128, slots=FAKE, T=1, cu=FAKE, seq=FAKE, B=1, R=1, rb=FAKE: \
        lib.m3s_store_and_rows(ctypes.byref(_cache() if cache is None else cache), k, None, None, stride, slots, T,
                               cu, seq, B, R, FAKE, FAKE, rb, None, None)
    assert f(T=-1) == E.ERR_INVALID_ARG
    assert f(slots=None) == E.ERR_INVALID_ARG
    assert f(stride=100) == E.ERR_INVALID_ARG
    assert f(cache=_cache(page=64)) == E.ERR_UNSUPPORTED
    assert f(B=-1) == E.ERR_INVALID_ARG
    assert f(B=5000) == E.ERR_UNSUPPORTED
    assert f(cu=None) == E.ERR_INVALID_ARG
    assert f(rb=None) == E.ERR_INVALID_ARG


def test_store_and_prefill_rows_validation(lib):
    """The one-launch store and prefill row map refuses what either call refuses."""
    E = m3s
    f = lambda cache=None, k=FAKE, stride=128, slots=FAKE, T=1, cu=FAKE, seq=FAKE, B=1, R=1, G=4, gb=FAKE: \
        lib.m3s_store_and_prefill_rows(ctypes.byref(_cache() if cache is None else cache), k, None, None, stride,
                                       slots, T, cu, seq, B, R, G, FAKE, FAKE, FAKE, FAKE, gb, None, None)
    assert f(T=-1) == E.ERR_INVALID_ARG
    assert f(slots=None) == E.ERR_INVALID_ARG
    assert f(stride=100) == E.ERR_INVALID_ARG
    assert f(cache=_cache(page=64)) == E.ERR_UNSUPPORTED
    assert f(B=-1) == E.ERR_INVALID_ARG
    assert f(B=4097) == E.ERR_UNSUPPORTED
    assert f(G=0) == E.ERR_UNSUPPORTED
    assert f(cu=None) == E.ERR_INVALID_ARG
    assert f(gb=None) == E.ERR_INVALID_ARG


def test_qknorm_rope_store_validation(lib):
    """Every call below fails host validation (or has no tokens) and launches nothing."""
    MIS = ctypes.c_void_p(4096 + 8)      # 8-byte aligned only
    I, U, A = m3s.ERR_INVALID_ARG, m3s.ERR_UNSUPPORTED, None

    def f(cache=None, q=FAKE, qs=512, G=4, k=FAKE, v=FAKE, iq=FAKE, ik=FAKE, rs=128, w=FAKE, eps=1e-6,
          pos=FAKE, cs=FAKE, mp=16, rd=64, sl=FAKE, T=3, qo=FAKE, qe=None, iqo=FAKE):
        c = _cache() if cache is None else cache
        return lib.m3s_qknorm_rope_store(ctypes.byref(c), q, qs, G, k, v, iq, ik, rs, w, eps, pos, cs, mp, rd,
                                         sl, T, qo, qe, iqo, None, None)

    assert f(T=0) == m3s.OK                                 # nothing to do: no launch
    assert f(cache=_cache(fmt=3)) == U
    assert f(cache=_cache(page=64)) == U
    assert f(T=-1) == I
    assert f(G=0) == U and f(G=17) == U
    assert f(rd=40) == U and f(rd=144) == U and f(rd=-16) == U
    assert f(eps=-1.0) == I and f(eps=float("nan")) == I and f(eps=float("inf")) == I
    for name in ("q", "k", "v", "iq", "ik", "w", "qo", "iqo", "sl"):
        assert f(**{name: None}) == I, name
    for name in ("q", "k", "v", "iq", "ik", "w", "qo", "iqo", "cs"):
        assert f(**{name: MIS}) == I, name
    assert f(qe=ctypes.c_void_p(4096 + 4)) == I             # e4m3 output needs 8-byte alignment
    assert f(qs=511) == I and f(G=4, qs=504) == I and f(rs=120) == I and f(rs=132) == I
    assert f(pos=None) == I and f(cs=None) == I and f(mp=0) == I
    assert f(cache=m3s.m3s_cache(1, 4, 128, 128, 1, 4096, 4096, None, 4096, 4096, 4096)) == I


def test_index_topk_attend_validation(lib):
    """The fused call validates as the two calls do and launches nothing here."""
    I, U, Wk = m3s.ERR_INVALID_ARG, m3s.ERR_UNSUPPORTED, m3s.ERR_WORKSPACE
    rows = _rows(nreq=1, nrows=2)
    big = 1 << 30

    def f(cache=None, qi=FAKE, qis=128, q=FAKE, qrs=2048, qhs=128, G=16, bt=FAKE, bts=64, mb=64, r=rows, k=16,
          flags=0, ini=0, loc=0, sm=1.0, ids=FAKE, out=FAKE, ws=FAKE, wsb=big):
        c = _cache() if cache is None else cache
        return lib.m3s_index_topk_attend(ctypes.byref(c), qi, qis, q, qrs, qhs, G, bt, bts, mb,
                                         None if r is None else ctypes.byref(r), k, flags, ini, loc, sm, ids, out, ws,
                                         wsb, None, None)

    assert f(r=None) == I
    assert f(cache=_cache(fmt=7)) == U
    assert f(k=0) == U and f(k=65) == U
    assert f(G=0) == U and f(G=17) == U
    assert f(flags=2) == I and f(ini=-1) == I
    assert f(sm=float("nan")) == I
    assert f(qi=None) == I and f(q=None) == I and f(ids=None) == I and f(out=None) == I
    assert f(qis=100) == I and f(qrs=12) == I
    assert f(bt=None) == I and f(bts=10) == I
    assert f(ws=None) == Wk and f(wsb=0) == Wk
    need = m3s.m3s_workspace_bytes(m3s.OP_INDEX_TOPK_ATTEND, 2, 1, 64, 16, 16)
    a256 = lambda n: (n + 255) // 256 * 256
    # the index call's part, the attention's, then 2 x 16 int32 pages of the selected ids
    assert need == a256(m3s.m3s_workspace_bytes(m3s.OP_INDEX_TOPK, 2, 1, 64, 16, 16)) + \
        a256(m3s.m3s_workspace_bytes(m3s.OP_SPARSE_ATTEND, 2, 1, 64, 16, 16)) + 256
    assert f(wsb=need - 1) == Wk
    assert f(r=_rows(nreq=0, nrows=0)) == m3s.OK        # no rows: nothing to do


def test_probe_rejects_bad_arguments(lib):
    """The measurement-only page-read probe validates on the host and launches nothing."""
    import ctypes
    f = lib.m3s_probe_page_reads
    one = ctypes.c_void_p(16)
    assert f(None, one, one, 1, 0, one, 1, None) == m3s.ERR_INVALID_ARG
    assert f(one, one, one, -1, 0, one, 1, None) == m3s.ERR_INVALID_ARG
    assert f(one, one, one, 1, 3, one, 1, None) == m3s.ERR_INVALID_ARG
    assert f(one, one, one, 1, -1, one, 1, None) == m3s.ERR_INVALID_ARG
    assert f(one, one, one, 1, 0, one, 0, None) == m3s.ERR_INVALID_ARG
    assert f(one, one, one, 0, 0, one, 1, None) == m3s.OK


def test_index_topk_attend_noalloc_refuses_sizes_past_the_scratch(lib):
    """The no-allocation call refuses, on the host and before touching a device, any shape
    whose workspace would exceed the library's scratch; bad rows are refused as in the
    workspace call."""
    Wk = m3s.ERR_WORKSPACE

    def f(r, mb=64, k=16, G=16):
        c = _cache(pages=1 << 20)
        return lib.m3s_index_topk_attend_noalloc(ctypes.byref(c), FAKE, 128, FAKE, 2048, 128, G, FAKE, 8192, mb,
                                                 None if r is None else ctypes.byref(r), k, 0, 0, 0, 1.0, FAKE,
                                                 FAKE, None, None)

    assert m3s.NOALLOC_SCRATCH_BYTES == 32 << 20
    big = _rows(nreq=4, nrows=4096)
    assert m3s.m3s_workspace_bytes(m3s.OP_INDEX_TOPK_ATTEND, 4096, 4, 8192, 16, 16) > m3s.NOALLOC_SCRATCH_BYTES
    assert f(big, mb=8192) == Wk
    assert f(None) == m3s.ERR_INVALID_ARG
    assert f(_rows(nreq=1, nrows=-1)) == m3s.ERR_INVALID_ARG


def test_decode_step_validation(lib):
    """The one-launch decode step validates as m3s_store_and_rows and
    m3s_index_topk_attend do, and launches nothing here."""
    I, U, Wk = m3s.ERR_INVALID_ARG, m3s.ERR_UNSUPPORTED, m3s.ERR_WORKSPACE
    big = 1 << 30

    def f(cache=None, k=FAKE, stride=128, slots=FAKE, cu=FAKE, seq=FAKE, B=1, R=2, rq=FAKE, rb=FAKE, qi=FAKE,
          qis=128, q=FAKE, qrs=2048, qhs=128, G=16, bt=FAKE, bts=64, mb=64, topk=16, flags=0, sm=1.0, ids=FAKE,
          out=FAKE, ws=FAKE, wsb=big):
        c = _cache() if cache is None else cache
        return lib.m3s_decode_step(ctypes.byref(c), k, None, None, stride, slots, cu, seq, B, R, rq, FAKE, rb, qi,
                                   qis, q, qrs, qhs, G, bt, bts, mb, topk, flags, 0, 0, sm, ids, out, ws, wsb, None,
                                   None)

    # the store's checks
    assert f(slots=None) == I and f(stride=100) == I
    assert f(cache=_cache(page=64)) == U
    # the row map's
    assert f(B=-1) == I and f(B=5000) == U and f(cu=None) == I and f(rb=None) == I and f(rq=None) == I
    # the index call's and the attention's
    assert f(qi=None) == I and f(q=None) == I and f(ids=None) == I and f(out=None) == I
    assert f(topk=0) == U and f(G=17) == U and f(flags=2) == I and f(sm=float("nan")) == I
    assert f(bt=None) == I and f(bts=10) == I and f(mb=-1) == I
    assert f(ws=None) == Wk and f(wsb=0) == Wk
    need = m3s.m3s_workspace_bytes(m3s.OP_INDEX_TOPK_ATTEND, 2, 1, 64, 16, 16)
    assert f(wsb=need - 1) == Wk
