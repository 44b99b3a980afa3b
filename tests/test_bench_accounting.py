"""Host-side accounting of bench.py, on the CPU.

- The algorithmic bytes its roofline divides by: every causal index token at 72 B
  (NVFP4: 64 B of e2m1 codes + 8 B of E4M3 scales) or 68 B (MXFP4: + 4 B of E8M0
  scales), the causal block-table entries and the index queries for the index call;
  the distinct selected (request, block) K/V bytes for the attention (ATOM PR
  "[MiniMax-M3.1] FP4 index cache and NVFP4 sparse KV cache", Design; vLLM PR
  "MXFP4 KV + indexer cache for MiniMax-M3.1", Design: 68 B per token and head).
- The counter ingestion behind roofline.traffic: FETCH_SIZE / WRITE_SIZE summed per
  dispatch and scaled by what the same counters read for a copy of known size.
- The source hash that keys the counter record ignores comments and blank lines.
"""
from __future__ import annotations

import csv
import json

import numpy as np
import pytest

import bench
import workloads as W


def _layout(cfg):
    return W.make_layout(cfg.seq_lens, cfg.q_len, cfg.seed)


@pytest.mark.parametrize("name,rb", [("b8x8_150k", 72), ("b8x8_150k_mxfp4", 68)])
def test_index_call_bytes_at_150k(name, rb):
    cfg = W.config(name)
    lay = _layout(cfg)
    R = int(lay.cu_q[-1])
    assert R == 64
    b = bench.step_bytes(cfg, lay, np.full((R, cfg.topk), -1, np.int32), cfg.G)
    assert b["index"] == 8 * 150_000 * rb
    # 1172 causal blocks per request (ceil(150000 / 128)), 4 B each; 256 B of bf16 query per row
    assert b["index_call"] == 8 * 150_000 * rb + 8 * 1172 * 4 + 64 * 256
    if rb == 72:
        assert b["index_call"] == 86_453_888
    assert b["attend"] == 0


def test_step_bytes_hand_example():
    """Two requests of 300 and 1000 tokens, 2 rows each, G = 4, top-k 4, NVFP4."""
    cfg = W.config(0)
    lay = W.make_layout((300, 1000), 2, 0)
    ids = np.array([[0, 2, -1, -1],     # request 0
                    [2, 0, -1, -1],     # request 0: the same two blocks again
                    [7, -1, -1, -1],    # request 1
                    [7, 3, -1, -1]], np.int32)
    b = bench.step_bytes(cfg, lay, ids, 4)
    # distinct (request, block): (0, 0) 128 tokens, (0, 2) 300 - 256 = 44 tokens,
    # (1, 7) 1000 - 896 = 104 tokens, (1, 3) 128 tokens; K and V at 72 B per token
    assert b["attend"] == 2 * 72 * (128 + 44 + 104 + 128) == 58_176
    assert b["index"] == (300 + 1000) * 72
    store = 4 * 3 * 256 + 4 * 3 * 72           # 4 new rows of K, V, index K: bf16 read, planes written
    tables = (3 + 8) * 4                        # causal block-table entries
    queries = 4 * 256 + 4 * 4 * 256             # index query + 4 heads of query, bf16
    outs = 4 * 4 * 128 * 4 + 2 * 4 * 4 * 4      # fp32 output + ids written and read
    assert b["store"] == store
    assert b["other"] == store + tables + queries + outs == 17_420
    assert b["total"] == 93_600 + 58_176 + 17_420
    assert b["index_call"] == 93_600 + tables + 4 * 256


def test_row_lens():
    lay = W.make_layout((300, 1000), 2, 0)
    assert bench.row_lens_of(lay).tolist() == [299, 300, 999, 1000]


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)


def test_counter_ingestion_scales_by_the_copy(tmp_path, monkeypatch):
    """Per step kernel: the median over the steps (a front kernel opens each step) of the
    counter summed per dispatch, scaled by the copy; stage-timing launches outside a step
    sequence do not count."""
    neg = "void at::native::neg_kernel_cuda(float)"
    front = "void m3s::store_rows_kernel<1>(m3s::StoreArgs, m3s::RowsArgs)"
    scan = "void m3s::index_scan_kernel<1, 1, 16, 1>(m3s::IndexArgs)"
    fused = "void m3s::select_attend_kernel<1, 8>(m3s::IndexArgs, m3s::AttendArgs)"
    sel = "void m3s::index_select_kernel<1, 8, 1>(m3s::IndexArgs)"
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    # one dispatch may be reported in several partial rows: they are summed per dispatch
    _counter_csv(fetch, [(1, neg, "FETCH_SIZE", 262144.0), (1, neg, "FETCH_SIZE", 262144.0),
                         (2, neg, "FETCH_SIZE", 524288.0),
                         (3, front, "FETCH_SIZE", 100.0),
                         (4, scan, "FETCH_SIZE", 40000.0), (4, scan, "FETCH_SIZE", 2000.0),
                         (5, fused, "FETCH_SIZE", 20000.0),
                         (6, front, "FETCH_SIZE", 120.0),
                         (7, scan, "FETCH_SIZE", 42000.0),
                         (8, fused, "FETCH_SIZE", 22000.0),
                         (9, front, "FETCH_SIZE", 110.0),
                         (10, scan, "FETCH_SIZE", 43000.0),
                         (11, fused, "FETCH_SIZE", 21000.0),
                         (12, sel, "FETCH_SIZE", 800.0),       # a stage-timing launch: no step
                         (11, fused, "GRBM_COUNT", 1e9)])       # other counters are ignored
    _counter_csv(write, [(1, neg, "WRITE_SIZE", 1048576.0),
                         (3, front, "WRITE_SIZE", 10.0), (4, scan, "WRITE_SIZE", 800.0),
                         (5, fused, "WRITE_SIZE", 2000.0),
                         (6, front, "WRITE_SIZE", 10.0), (7, scan, "WRITE_SIZE", 850.0),
                         (8, fused, "WRITE_SIZE", 2100.0),
                         (9, front, "WRITE_SIZE", 10.0), (10, scan, "WRITE_SIZE", 900.0),
                         (11, fused, "WRITE_SIZE", 2000.0)])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    bench.ingest_pmc(str(fetch), str(write), "b8x8_150k")
    rec = json.loads((tmp_path / "decode_step_b8x8_150k_traffic.json").read_text())
    cal = rec["calibration"]
    # the copy reads and writes 1 GiB: FETCH_SIZE reads half of it in KiB (x2), WRITE_SIZE all (x1)
    assert cal["fetch_scale"] == 2.0 and cal["write_scale"] == 1.0
    k = {e["kernel"]: e for e in rec["step_kernels"]}
    assert [e["kernel"] for e in rec["step_kernels"]] == [
        "store_rows_kernel<1>", "index_scan_kernel<1, 1, 16, 1>", "select_attend_kernel<1, 8>"]
    sk = k["index_scan_kernel<1, 1, 16, 1>"]
    # the fetch pass's last step is followed by a stage-timing launch: a different sequence
    assert sk["fetch_kib"] == 42000.0 and sk["write_kib"] == 850.0 and sk["steps"] == [2, 3]
    assert sk["fetch_bytes"] == 42000 * 1024 * 2
    fk = k["select_attend_kernel<1, 8>"]
    assert fk["fetch_bytes"] == 21000 * 1024 * 2 and fk["write_bytes"] == 2000 * 1024
    assert rec["fused_call_bytes"] == (42000 + 21000) * 1024 * 2 + (850 + 2000) * 1024
    assert rec["step_bytes"] == rec["fused_call_bytes"] + 110 * 1024 * 2 + 10 * 1024
    assert rec["source_sha"] == bench.source_sha(bench.KERNEL_SOURCES)
    assert bench.load_record(str(tmp_path / "decode_step_b8x8_150k_traffic.json"), "b8x8_150k") == rec
    assert bench.load_record(str(tmp_path / "decode_step_b8x8_150k_traffic.json"), "b8x8_skew_450k") is None


def test_trace_ingestion(tmp_path, monkeypatch):
    """Per step kernel: the median duration over the steps; the step's span and the gap to
    the next step."""
    path = tmp_path / "trace.csv"
    cols = ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Workgroup_Size_X"]
    front = "void m3s::store_rows_kernel<1>(m3s::StoreArgs, m3s::RowsArgs)"
    scan = "void m3s::index_scan_kernel<1, 1, 16, 1>(m3s::IndexArgs)"
    att = "m3s::attend_combine_kernel(m3s::AttendArgs)"
    rows, d, t = [], 1, 1000
    for step, (a, b, c) in enumerate([(4000, 20000, 3000), (5000, 21000, 3100), (4500, 22000, 2900)]):
        for name, dur, grid in ((front, a, 13 * 256), (scan, b, 256 * 1024), (att, c, 64 * 256)):
            rows.append((d, name, t, t + dur, grid, 1024 if name == scan else 256))
            d += 1
            t += dur
        t += 8000 + 1000 * step
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        w.writerows(rows)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    bench.ingest_trace(str(path), "b8x8_150k")
    rec = json.loads((tmp_path / "decode_step_b8x8_150k_kernels.json").read_text())
    k = {e["kernel"]: e for e in rec["step_kernels"]}
    assert rec["steps"] == 3
    assert k["index_scan_kernel<1, 1, 16, 1>"]["median_us"] == 21.0
    assert k["index_scan_kernel<1, 1, 16, 1>"]["workgroups"] == 256
    assert k["attend_combine_kernel"]["median_us"] == 3.0
    assert k["store_rows_kernel<1>"]["median_us"] == 4.5
    assert rec["step_span_median_us"] == 29.1
    assert rec["gap_to_next_step_median_us"] == 8.5


def test_kernel_names():
    assert bench.kernel_short("void m3s::index_scan_kernel<1, 1, 16, 1>(m3s::IndexArgs)") == \
        "index_scan_kernel<1, 1, 16, 1>"
    assert bench.kernel_short("m3s::attend_combine_kernel(m3s::AttendArgs)") == "attend_combine_kernel"


def test_code_text_ignores_comments_and_blank_lines():
    a = 'int a = 1;  // one\n/* block\n comment */\n\nconst char* s = "x//y /* z */";\n'
    b = 'int a = 1;\nconst char* s = "x//y /* z */";   // a changed comment\n'
    assert bench.code_text(a).split() == bench.code_text(b).split()
    assert '"x//y /* z */"' in bench.code_text(a)
    assert bench.code_text("int a = 2;") != bench.code_text("int a = 1;")
