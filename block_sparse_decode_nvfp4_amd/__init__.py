"""Python binding of libm3s.so, the MI355X decode hot path for block-sparse
attention over NVFP4 / MXFP4 paged caches.

This module only marshals arguments (torch tensors -> device pointers, the
current HIP stream) into the C ABI declared in include/m3s.h; every step of
the path runs in the library's HIP kernels. Loading fails loudly when the
library is missing: there is no fallback.

Functions carry the C names: m3s_store, m3s_decode_rows, m3s_store_and_rows, m3s_prefill_rows,
m3s_store_and_prefill_rows,
m3s_qknorm_rope_store, m3s_index_topk, m3s_sparse_attend, m3s_index_topk_attend, m3s_decode_step,
m3s_workspace_bytes,
m3s_read_device_status, m3s_status_string, m3s_version.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libm3s.so")

PAGE = 128
HEAD_DIM = 128

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
FMT_NVFP4, FMT_MXFP4 = 1, 2
FORMATS = {"nvfp4": FMT_NVFP4, "mxfp4": FMT_MXFP4}
SCALE_BYTES = {FMT_NVFP4: 8, FMT_MXFP4: 4}
OP_INDEX_TOPK, OP_SPARSE_ATTEND, OP_INDEX_TOPK_ATTEND = 1, 2, 3
TOPK_TIE_HIGH_ID = 1
DEV_BITS = {
    "BAD_SLOT": 1 << 0, "BAD_ROWS": 1 << 1, "BAD_LENGTH": 1 << 2, "BAD_PAGE": 1 << 3,
    "BAD_BLOCK_ID": 1 << 4, "INEXACT": 1 << 5, "BAND_OVERFLOW": 1 << 6, "BAD_POSITION": 1 << 7,
    "RANGE": 1 << 8, "STEP_SLOT": 1 << 9,
}

EXPORTS = ("m3s_store", "m3s_decode_rows", "m3s_store_and_rows", "m3s_prefill_rows", "m3s_store_and_prefill_rows",
           "m3s_qknorm_rope_store",
           "m3s_index_topk", "m3s_sparse_attend", "m3s_index_topk_attend",
           "m3s_workspace_bytes", "m3s_read_device_status", "m3s_status_string", "m3s_version",
           "m3s_probe_page_reads", "m3s_index_topk_attend_noalloc", "m3s_decode_step")
NOALLOC_SCRATCH_BYTES = 32 << 20
MAX_GROUPS = 4096
GROUP_ROWS = 64

_c_i32p = ctypes.c_void_p
_lib = None


class M3SError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status}: {m3s_status_string(status)}")


class m3s_cache(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("k_data", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_data", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("idx_data", ctypes.c_void_p), ("idx_scale", ctypes.c_void_p)]


class m3s_rows(ctypes.Structure):
    _fields_ = [("grp_row", ctypes.c_void_p), ("grp_req", ctypes.c_void_p), ("grp_blk", ctypes.c_void_p),
                ("row_req", ctypes.c_void_p), ("row_len", ctypes.c_void_p), ("num_groups", ctypes.c_int32),
                ("num_rows", ctypes.c_int32)]


def load(path: str | None = None):
    """Load libm3s.so (raises if it is missing or not loadable)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with __graft_entry__.build() "
                           "or python block_sparse_decode_nvfp4_amd/_build.py")
    # torch first: the library then binds to the HIP runtime torch has loaded rather
    # than loading a second copy beside it (two runtimes in one process fail launches)
    _torch()
    lib = ctypes.CDLL(p)
    V, I32, I64, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    sig = {
        "m3s_store": (I32, [V, V, V, V, I64, V, I32, V, V]),
        "m3s_decode_rows": (I32, [V, V, I32, I32, V, V, V, V, V]),
        "m3s_prefill_rows": (I32, [V, V, I32, I32, I32, V, V, V, V, V, V, V]),
        "m3s_store_and_rows": (I32, [V, V, V, V, I64, V, I32, V, V, I32, I32, V, V, V, V, V]),
        "m3s_store_and_prefill_rows": (I32, [V, V, V, V, I64, V, I32, V, V, I32, I32, I32, V, V, V, V, V, V, V]),
        "m3s_qknorm_rope_store": (I32, [V, V, I64, I32, V, V, V, V, I64, V, F32, V, V, I32, I32, V, I32,
                                        V, V, V, V, V]),
        "m3s_index_topk": (I32, [V, V, I64, V, I32, I32, V, I32, I32, I32, I32, V, V, SZ, V, V]),
        "m3s_sparse_attend": (I32, [V, V, I64, I64, I32, V, I32, I32, V, V, I32, F32, V, V, SZ, V, V]),
        "m3s_index_topk_attend": (I32, [V, V, I64, V, I64, I64, I32, V, I32, I32, V, I32, I32, I32, I32, F32, V, V,
                                        V, SZ, V, V]),
        "m3s_workspace_bytes": (SZ, [I32, I32, I32, I32, I32, I32]),
        "m3s_read_device_status": (I32, [V, V, V]),
        "m3s_status_string": (ctypes.c_char_p, [I32]),
        "m3s_version": (I32, []),
        "m3s_probe_page_reads": (I32, [V, V, V, I32, I32, V, I32, V]),
        "m3s_index_topk_attend_noalloc": (I32, [V, V, I64, V, I64, I64, I32, V, I32, I32, V, I32, I32, I32, I32,
                                                F32, V, V, V, V]),
        "m3s_decode_step": (I32, [V, V, V, V, I64, V, V, V, I32, I32, V, V, V, V, I64, V, I64, I64, I32, V, I32,
                                  I32, I32, I32, I32, I32, F32, V, V, V, SZ, V, V]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, st):
    if st != OK:
        raise M3SError(fn, st)


def _need(t, name, dtype, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def m3s_version() -> int:
    return int(load().m3s_version())


def m3s_status_string(status: int) -> str:
    return load().m3s_status_string(int(status)).decode()


def m3s_workspace_bytes(op: int, num_rows: int, num_reqs: int, max_blocks: int, topk: int, num_heads: int) -> int:
    return int(load().m3s_workspace_bytes(op, num_rows, num_reqs, max_blocks, topk, num_heads))


class Cache:
    """One KV head's paged planes (k, v, index K; payload + scale each) on a device."""

    def __init__(self, fmt: str, num_pages: int, device="cuda"):
        torch = _torch()
        self.fmt = fmt
        self.format = FORMATS[fmt]
        self.num_pages = int(num_pages)
        sb = SCALE_BYTES[self.format]
        self.planes = {}
        for name in ("k", "v", "idx"):
            self.planes[name] = (torch.zeros((num_pages, PAGE, 64), dtype=torch.uint8, device=device),
                                 torch.zeros((num_pages, PAGE, sb), dtype=torch.uint8, device=device))
        self._struct()

    def _struct(self):
        p = self.planes
        self.c = m3s_cache(self.format, self.num_pages, PAGE, HEAD_DIM, 1,
                           p["k"][0].data_ptr(), p["k"][1].data_ptr(), p["v"][0].data_ptr(), p["v"][1].data_ptr(),
                           p["idx"][0].data_ptr(), p["idx"][1].data_ptr())

    def ref(self):
        return ctypes.byref(self.c)


class Rows:
    """The row map of one step and the index scan's work groups (device tensors), with
    their m3s_rows struct. From m3s_decode_rows: one group per request (grp_row = cu_q,
    grp_req None); from m3s_prefill_rows: 64-row groups."""

    def __init__(self, grp_row, grp_req, grp_blk, row_req, row_len, num_groups: int, num_rows: int):
        self.grp_row, self.grp_req, self.grp_blk = grp_row, grp_req, grp_blk
        self.row_req, self.row_len = row_req, row_len
        self.num_groups, self.num_rows = int(num_groups), int(num_rows)
        self.c = m3s_rows(grp_row.data_ptr(), None if grp_req is None else grp_req.data_ptr(), grp_blk.data_ptr(),
                          row_req.data_ptr(), row_len.data_ptr(), self.num_groups, self.num_rows)

    @property
    def num_reqs(self):
        return self.num_groups

    def ref(self):
        return ctypes.byref(self.c)


def m3s_store(cache: Cache, k, v, idx, slot_mapping, dev_status=None, stream=None):
    """Quantize bf16 rows [T, >=128] of k / v / idx (any may be None) into the planes at slot_mapping."""
    torch = _torch()
    ref = next(t for t in (k, v, idx) if t is not None)
    T = ref.shape[0]
    stride = ref.stride(0)
    for name, t in (("k", k), ("v", v), ("idx", idx)):
        if t is not None:
            _need(t, name, torch.bfloat16)
            if t.shape[0] != T or t.stride(0) != stride or t.stride(1) != 1 or t.shape[1] < HEAD_DIM:
                raise ValueError(f"{name}: rows must share [T, >=128] shape and row stride")
    _need(slot_mapping, "slot_mapping", torch.int32)
    if slot_mapping.numel() != T or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int32 [T]")
    st = load().m3s_store(cache.ref(), _ptr(k), _ptr(v), _ptr(idx), stride, _ptr(slot_mapping), T,
                          _ptr(dev_status), _stream(stream))
    _check("m3s_store", st)


def m3s_qknorm_rope_store(cache: Cache, q, k, v, idx_q, idx_k, norm_weights, eps: float, positions, cos_sin,
                          slot_mapping, q_out=None, idx_q_out=None, q_out_e4m3=None, want_e4m3: bool = False,
                          dev_status=None, stream=None):
    """The fused producer store: RMS norm + rotary of q [T, G, >=128 per head] / k / idx_q / idx_k,
    FP4 store of k, v, idx_k at slot_mapping, query rows out. cos_sin is float32 [max_pos, rotary_dim]
    (rotary_dim = cos_sin.shape[1], 0 for none). Returns (q_out, idx_q_out, q_out_e4m3 or None)."""
    torch = _torch()
    _need(q, "q", torch.bfloat16)
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or q.stride(2) != 1 or q.stride(1) != HEAD_DIM:
        raise ValueError("q must be [T, G, 128] with heads 128 elements apart")
    T, G = q.shape[0], q.shape[1]
    stride = k.stride(0)
    for name, t in (("k", k), ("v", v), ("idx_q", idx_q), ("idx_k", idx_k)):
        _need(t, name, torch.bfloat16)
        if t.shape[0] != T or t.stride(0) != stride or t.stride(1) != 1 or t.shape[1] < HEAD_DIM:
            raise ValueError(f"{name}: rows must share [T, >=128] shape and row stride")
    _need(norm_weights, "norm_weights", torch.bfloat16)
    if tuple(norm_weights.shape) != (4, HEAD_DIM) or not norm_weights.is_contiguous():
        raise ValueError("norm_weights must be a contiguous bf16 [4, 128]")
    _need(cos_sin, "cos_sin", torch.float32)
    if cos_sin.dim() != 2 or not cos_sin.is_contiguous():
        raise ValueError("cos_sin must be a contiguous float32 [max_pos, rotary_dim]")
    rd = cos_sin.shape[1]
    _need(slot_mapping, "slot_mapping", torch.int32)
    if slot_mapping.numel() != T or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int32 [T]")
    if positions is not None:
        _need(positions, "positions", torch.int32)
        if positions.numel() != T or not positions.is_contiguous():
            raise ValueError("positions must be a contiguous int32 [T]")
    dev = q.device
    q_out = torch.empty((T, G, HEAD_DIM), dtype=torch.bfloat16, device=dev) if q_out is None else q_out
    idx_q_out = torch.empty((T, HEAD_DIM), dtype=torch.bfloat16, device=dev) if idx_q_out is None else idx_q_out
    if q_out_e4m3 is None and want_e4m3:
        q_out_e4m3 = torch.empty((T, G, HEAD_DIM), dtype=torch.uint8, device=dev)
    st = load().m3s_qknorm_rope_store(cache.ref(), _ptr(q), q.stride(0), G, _ptr(k), _ptr(v), _ptr(idx_q),
                                      _ptr(idx_k), stride, _ptr(norm_weights), float(eps), _ptr(positions),
                                      _ptr(cos_sin) if rd > 0 else None, cos_sin.shape[0], rd,
                                      _ptr(slot_mapping), T, _ptr(q_out), _ptr(q_out_e4m3), _ptr(idx_q_out),
                                      _ptr(dev_status), _stream(stream))
    _check("m3s_qknorm_rope_store", st)
    return q_out, idx_q_out, q_out_e4m3


def m3s_decode_rows(cu_q, seq_lens, num_rows: int, row_req=None, row_len=None, req_blk=None,
                    dev_status=None, stream=None) -> Rows:
    torch = _torch()
    _need(cu_q, "cu_q", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    B = seq_lens.numel()
    if cu_q.numel() != B + 1:
        raise ValueError("cu_q must have num_reqs + 1 entries")
    dev = cu_q.device
    row_req = torch.empty(num_rows, dtype=torch.int32, device=dev) if row_req is None else row_req
    row_len = torch.empty(num_rows, dtype=torch.int32, device=dev) if row_len is None else row_len
    req_blk = torch.empty(B + 1, dtype=torch.int32, device=dev) if req_blk is None else req_blk
    st = load().m3s_decode_rows(_ptr(cu_q), _ptr(seq_lens), B, num_rows, _ptr(row_req), _ptr(row_len),
                                _ptr(req_blk), _ptr(dev_status), _stream(stream))
    _check("m3s_decode_rows", st)
    return Rows(cu_q, None, req_blk, row_req, row_len, B, num_rows)


def m3s_store_and_rows(cache: Cache, k, v, idx, slot_mapping, cu_q, seq_lens, num_rows: int, row_req, row_len,
                       req_blk, dev_status=None, stream=None):
    """m3s_store and m3s_decode_rows in one launch (outputs written in place)."""
    torch = _torch()
    ref = next(t for t in (k, v, idx) if t is not None)
    T = ref.shape[0]
    stride = ref.stride(0)
    for name, t in (("k", k), ("v", v), ("idx", idx)):
        if t is not None:
            _need(t, name, torch.bfloat16)
            if t.shape[0] != T or t.stride(0) != stride or t.stride(1) != 1 or t.shape[1] < HEAD_DIM:
                raise ValueError(f"{name}: rows must share [T, >=128] shape and row stride")
    _need(slot_mapping, "slot_mapping", torch.int32)
    _need(cu_q, "cu_q", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    B = seq_lens.numel()
    if slot_mapping.numel() != T or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int32 [T]")
    if cu_q.numel() != B + 1:
        raise ValueError("cu_q must have num_reqs + 1 entries")
    st = load().m3s_store_and_rows(cache.ref(), _ptr(k), _ptr(v), _ptr(idx), stride, _ptr(slot_mapping), T,
                                   _ptr(cu_q), _ptr(seq_lens), B, num_rows, _ptr(row_req), _ptr(row_len),
                                   _ptr(req_blk), _ptr(dev_status), _stream(stream))
    _check("m3s_store_and_rows", st)
    return Rows(cu_q, None, req_blk, row_req, row_len, B, num_rows)


def _prefill_rows_out(cu_q, seq_lens, num_rows, max_groups, out):
    torch = _torch()
    _need(cu_q, "cu_q", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    B = seq_lens.numel()
    if cu_q.numel() != B + 1:
        raise ValueError("cu_q must have num_reqs + 1 entries")
    if max_groups is None:
        max_groups = min(MAX_GROUPS, max(1, (num_rows + GROUP_ROWS - 1) // GROUP_ROWS + B))
    dev = cu_q.device
    if out is not None:
        if out.num_groups != max_groups or out.num_rows != num_rows:
            raise ValueError("out was made for other sizes")
        return B, max_groups, out
    row_req = torch.empty(num_rows, dtype=torch.int32, device=dev)
    row_len = torch.empty(num_rows, dtype=torch.int32, device=dev)
    grp_row = torch.empty(max_groups + 1, dtype=torch.int32, device=dev)
    grp_req = torch.empty(max_groups, dtype=torch.int32, device=dev)
    grp_blk = torch.empty(max_groups + 1, dtype=torch.int32, device=dev)
    return B, max_groups, Rows(grp_row, grp_req, grp_blk, row_req, row_len, max_groups, num_rows)


def m3s_prefill_rows(cu_q, seq_lens, num_rows: int, max_groups: int | None = None, dev_status=None,
                     stream=None, out: Rows | None = None) -> Rows:
    """Prefill row map and 64-row scan groups; max_groups defaults to the bound
    ceil(num_rows / 64) + num_reqs (capped at MAX_GROUPS). ``out`` (a Rows from an
    earlier call with the same sizes) is written in place."""
    B, max_groups, rows = _prefill_rows_out(cu_q, seq_lens, num_rows, max_groups, out)
    st = load().m3s_prefill_rows(_ptr(cu_q), _ptr(seq_lens), B, num_rows, max_groups, _ptr(rows.row_req),
                                 _ptr(rows.row_len), _ptr(rows.grp_row), _ptr(rows.grp_req), _ptr(rows.grp_blk),
                                 _ptr(dev_status), _stream(stream))
    _check("m3s_prefill_rows", st)
    return rows


def m3s_store_and_prefill_rows(cache: Cache, k, v, idx, slot_mapping, cu_q, seq_lens, num_rows: int,
                               max_groups: int | None = None, dev_status=None, stream=None,
                               out: Rows | None = None) -> Rows:
    """m3s_store and m3s_prefill_rows in one launch; returns the row map (``out``, from an
    earlier call with the same sizes, is written in place)."""
    torch = _torch()
    ref = next(t for t in (k, v, idx) if t is not None)
    T = ref.shape[0]
    stride = ref.stride(0)
    for name, t in (("k", k), ("v", v), ("idx", idx)):
        if t is not None:
            _need(t, name, torch.bfloat16)
            if t.shape[0] != T or t.stride(0) != stride or t.stride(1) != 1 or t.shape[1] < HEAD_DIM:
                raise ValueError(f"{name}: rows must share [T, >=128] shape and row stride")
    _need(slot_mapping, "slot_mapping", torch.int32)
    if slot_mapping.numel() != T or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int32 [T]")
    B, max_groups, rows = _prefill_rows_out(cu_q, seq_lens, num_rows, max_groups, out)
    st = load().m3s_store_and_prefill_rows(cache.ref(), _ptr(k), _ptr(v), _ptr(idx), stride, _ptr(slot_mapping), T,
                                           _ptr(cu_q), _ptr(seq_lens), B, num_rows, max_groups, _ptr(rows.row_req),
                                           _ptr(rows.row_len), _ptr(rows.grp_row), _ptr(rows.grp_req),
                                           _ptr(rows.grp_blk), _ptr(dev_status), _stream(stream))
    _check("m3s_store_and_prefill_rows", st)
    return rows


def index_workspace(rows: Rows, max_blocks: int, topk: int, device="cuda"):
    torch = _torch()
    n = m3s_workspace_bytes(OP_INDEX_TOPK, rows.num_rows, rows.num_reqs, max_blocks, topk, 1)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def attend_workspace(rows: Rows, max_blocks: int, topk: int, num_heads: int, device="cuda"):
    torch = _torch()
    n = m3s_workspace_bytes(OP_SPARSE_ATTEND, rows.num_rows, rows.num_reqs, max_blocks, topk, num_heads)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def m3s_index_topk(cache: Cache, q_idx, block_table, max_blocks: int, rows: Rows, topk: int, flags: int = 0,
                   topk_ids=None, workspace=None, dev_status=None, stream=None, init_blocks: int = 0,
                   local_blocks: int = 0):
    torch = _torch()
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(block_table, "block_table", torch.int32)
    if q_idx.dim() != 2 or q_idx.stride(1) != 1 or q_idx.shape[1] < HEAD_DIM:
        raise ValueError("q_idx must be [R, >=128] with unit inner stride")
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be [B, stride] with unit inner stride")
    if topk_ids is None:
        topk_ids = torch.empty((rows.num_rows, topk), dtype=torch.int32, device=q_idx.device)
    if workspace is None:
        workspace = index_workspace(rows, max_blocks, topk, q_idx.device)
    st = load().m3s_index_topk(cache.ref(), _ptr(q_idx), q_idx.stride(0), _ptr(block_table), block_table.stride(0),
                               max_blocks, rows.ref(), topk, flags, init_blocks, local_blocks, _ptr(topk_ids),
                               _ptr(workspace), workspace.numel(), _ptr(dev_status), _stream(stream))
    _check("m3s_index_topk", st)
    return topk_ids


def m3s_sparse_attend(cache: Cache, q, block_table, max_blocks: int, rows: Rows, topk_ids, sm_scale: float,
                      out=None, workspace=None, dev_status=None, stream=None):
    torch = _torch()
    _need(q, "q", torch.bfloat16)
    _need(topk_ids, "topk_ids", torch.int32)
    if q.dim() != 3 or q.stride(2) != 1 or q.shape[2] < HEAD_DIM:
        raise ValueError("q must be [R, G, >=128] with unit inner stride")
    G = q.shape[1]
    topk = topk_ids.shape[1]
    if out is None:
        out = torch.empty((rows.num_rows, G, HEAD_DIM), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = attend_workspace(rows, max_blocks, topk, G, q.device)
    st = load().m3s_sparse_attend(cache.ref(), _ptr(q), q.stride(0), q.stride(1), G, _ptr(block_table),
                                  block_table.stride(0), max_blocks, rows.ref(), _ptr(topk_ids), topk,
                                  float(sm_scale), _ptr(out), _ptr(workspace), workspace.numel(),
                                  _ptr(dev_status), _stream(stream))
    _check("m3s_sparse_attend", st)
    return out


def index_attend_workspace(rows: Rows, max_blocks: int, topk: int, num_heads: int, device="cuda"):
    torch = _torch()
    n = m3s_workspace_bytes(OP_INDEX_TOPK_ATTEND, rows.num_rows, rows.num_reqs, max_blocks, topk, num_heads)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def m3s_index_topk_attend(cache: Cache, q_idx, q, block_table, max_blocks: int, rows: Rows, topk: int,
                          sm_scale: float, flags: int = 0, topk_ids=None, out=None, workspace=None, dev_status=None,
                          stream=None, init_blocks: int = 0, local_blocks: int = 0):
    """m3s_index_topk then m3s_sparse_attend on its ids, select and attention split fused.
    Returns (topk_ids, out)."""
    torch = _torch()
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(q, "q", torch.bfloat16)
    _need(block_table, "block_table", torch.int32)
    if q_idx.dim() != 2 or q_idx.stride(1) != 1 or q_idx.shape[1] < HEAD_DIM:
        raise ValueError("q_idx must be [R, >=128] with unit inner stride")
    if q.dim() != 3 or q.stride(2) != 1 or q.shape[2] < HEAD_DIM:
        raise ValueError("q must be [R, G, >=128] with unit inner stride")
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be [B, stride] with unit inner stride")
    G = q.shape[1]
    dev = q.device
    if topk_ids is None:
        topk_ids = torch.empty((rows.num_rows, topk), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((rows.num_rows, G, HEAD_DIM), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = index_attend_workspace(rows, max_blocks, topk, G, dev)
    st = load().m3s_index_topk_attend(cache.ref(), _ptr(q_idx), q_idx.stride(0), _ptr(q), q.stride(0), q.stride(1), G,
                                      _ptr(block_table), block_table.stride(0), max_blocks, rows.ref(), topk, flags,
                                      init_blocks, local_blocks, float(sm_scale), _ptr(topk_ids), _ptr(out),
                                      _ptr(workspace), workspace.numel(), _ptr(dev_status), _stream(stream))
    _check("m3s_index_topk_attend", st)
    return topk_ids, out


def m3s_probe_page_reads(payload, scales, pages, mode: int, sink, stream=None, check: bool = True):
    """Measurement only: read the listed pages with the index scan's load pattern
    (see include/m3s.h). Every page id must lie inside the planes: with check=True the
    ids are checked here (a device-to-host read); a timing loop checks once, then passes
    check=False. Mode 2 streams the first pages.numel() pages of both planes instead."""
    torch = _torch()
    _need(payload, "payload", torch.uint8)
    _need(scales, "scales", torch.uint8)
    _need(pages, "pages", torch.int32)
    _need(sink, "sink", torch.int32)
    P = payload.shape[0]
    if payload.numel() != P * PAGE * 64 or scales.numel() != P * PAGE * 8:
        raise ValueError("payload must be [P, 128, 64] and scales [P, 128, 8]")
    # host-side bounds check of every page id (the kernel trusts them)
    if check and pages.numel() and (int(pages.min()) < 0 or int(pages.max()) >= P):
        raise ValueError("page id outside the planes")
    if mode == 2 and pages.numel() > P:
        raise ValueError("the stream reads more pages than the planes hold")
    st = load().m3s_probe_page_reads(_ptr(payload), _ptr(scales), _ptr(pages), pages.numel(), mode, _ptr(sink),
                                     sink.numel(), _stream(stream))
    _check("m3s_probe_page_reads", st)


def m3s_index_topk_attend_noalloc(cache: Cache, q_idx, q, block_table, max_blocks: int, rows: Rows, topk: int,
                                  sm_scale: float, flags: int = 0, topk_ids=None, out=None, dev_status=None,
                                  stream=None, init_blocks: int = 0, local_blocks: int = 0):
    """m3s_index_topk_attend with the library's own scratch buffer as the workspace (no
    device allocation inside the call; outputs are still the caller's). Returns
    (topk_ids, out)."""
    torch = _torch()
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(q, "q", torch.bfloat16)
    _need(block_table, "block_table", torch.int32)
    if q_idx.dim() != 2 or q_idx.stride(1) != 1 or q_idx.shape[1] < HEAD_DIM:
        raise ValueError("q_idx must be [R, >=128] with unit inner stride")
    if q.dim() != 3 or q.stride(2) != 1 or q.shape[2] < HEAD_DIM:
        raise ValueError("q must be [R, G, >=128] with unit inner stride")
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be [B, stride] with unit inner stride")
    G = q.shape[1]
    dev = q.device
    if topk_ids is None:
        topk_ids = torch.empty((rows.num_rows, topk), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((rows.num_rows, G, HEAD_DIM), dtype=torch.float32, device=dev)
    st = load().m3s_index_topk_attend_noalloc(cache.ref(), _ptr(q_idx), q_idx.stride(0), _ptr(q), q.stride(0),
                                              q.stride(1), G, _ptr(block_table), block_table.stride(0), max_blocks,
                                              rows.ref(), topk, flags, init_blocks, local_blocks, float(sm_scale),
                                              _ptr(topk_ids), _ptr(out), _ptr(dev_status), _stream(stream))
    _check("m3s_index_topk_attend_noalloc", st)
    return topk_ids, out


def m3s_decode_step(cache: Cache, k, v, idx, slot_mapping, cu_q, seq_lens, num_rows: int, row_req, row_len,
                    req_blk, q_idx, q, block_table, max_blocks: int, topk: int, sm_scale: float, flags: int = 0,
                    topk_ids=None, out=None, workspace=None, dev_status=None, stream=None, init_blocks: int = 0,
                    local_blocks: int = 0):
    """One decode step: m3s_store_and_rows then m3s_index_topk_attend, with the store,
    the row map and the index scan in one launch. The step's tokens are its rows
    (k, v, idx and slot_mapping have num_rows rows). Returns (rows, topk_ids, out)."""
    torch = _torch()
    T = num_rows
    stride = None
    for name, t in (("k", k), ("v", v), ("idx", idx)):
        if t is not None:
            _need(t, name, torch.bfloat16)
            stride = t.stride(0) if stride is None else stride
            if t.shape[0] != T or t.stride(0) != stride or t.stride(1) != 1 or t.shape[1] < HEAD_DIM:
                raise ValueError(f"{name}: rows must share [num_rows, >=128] shape and row stride")
    _need(slot_mapping, "slot_mapping", torch.int32)
    _need(cu_q, "cu_q", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(q, "q", torch.bfloat16)
    _need(block_table, "block_table", torch.int32)
    B = seq_lens.numel()
    if slot_mapping.numel() != T or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int32 [num_rows]")
    if cu_q.numel() != B + 1:
        raise ValueError("cu_q must have num_reqs + 1 entries")
    if q_idx.dim() != 2 or q_idx.stride(1) != 1 or q_idx.shape[1] < HEAD_DIM:
        raise ValueError("q_idx must be [R, >=128] with unit inner stride")
    if q.dim() != 3 or q.stride(2) != 1 or q.shape[2] < HEAD_DIM:
        raise ValueError("q must be [R, G, >=128] with unit inner stride")
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be [B, stride] with unit inner stride")
    G = q.shape[1]
    dev = q.device
    rows = Rows(cu_q, None, req_blk, row_req, row_len, B, num_rows)
    if topk_ids is None:
        topk_ids = torch.empty((num_rows, topk), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((num_rows, G, HEAD_DIM), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = index_attend_workspace(rows, max_blocks, topk, G, dev)
    st = load().m3s_decode_step(cache.ref(), _ptr(k), _ptr(v), _ptr(idx), stride or HEAD_DIM, _ptr(slot_mapping),
                                _ptr(cu_q), _ptr(seq_lens), B, num_rows, _ptr(row_req), _ptr(row_len), _ptr(req_blk),
                                _ptr(q_idx), q_idx.stride(0), _ptr(q), q.stride(0), q.stride(1), G,
                                _ptr(block_table), block_table.stride(0), max_blocks, topk, flags, init_blocks,
                                local_blocks, float(sm_scale), _ptr(topk_ids), _ptr(out), _ptr(workspace),
                                workspace.numel(), _ptr(dev_status), _stream(stream))
    _check("m3s_decode_step", st)
    return rows, topk_ids, out


def m3s_read_device_status(dev_status, stream=None) -> int:
    out = ctypes.c_uint32(0)
    st = load().m3s_read_device_status(_ptr(dev_status), ctypes.byref(out), _stream(stream))
    _check("m3s_read_device_status", st)
    return int(out.value)
