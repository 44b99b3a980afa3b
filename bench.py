"""Throughput of the decode hot path (store + decode_rows + index score/top-k + sparse
attend) on one MI355X, on seeded synthetic inputs shaped like the pages' workloads.

One step = one sparse layer's full path for one batch: the store of the step's new
K/V/index rows, the row map, the index top-k and the sparse attention, issued as one
m3s_decode_step call (or, with --calls two, as m3s_store_and_rows +
m3s_index_topk_attend; with --calls separate, as the four calls m3s_store,
m3s_decode_rows, m3s_index_topk, m3s_sparse_attend). Steps are HIP-graph
replays; consecutive steps use different layer copies of the cache (8 by default, >= 2 GB
in total at the default workload) so a step cannot be served from the 256 MB Infinity
Cache left warm by the previous one - as in a real model, where each of the 60 sparse
layers has its own cache.

Prints ONE JSON line (stdout). Extra detail goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode rows/s + achieved HBM GB/s (store+score+top-k+attend), 8 req x 8 rows @150K"
HBM_PEAK_GBS = 8000.0
PRODUCER_ROTARY_DIM = 64   # rotary dims of the producer measurement (half the head)
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "fp8": 5000.0}  # dense, MI355X
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["block_sparse_decode_nvfp4_amd/csrc/" + f for f in (
    "index_topk.hip", "attend_body.hpp", "attend.hip", "store.hip", "rows.hip", "rows_body.hpp", "quant.hpp",
    "fp4.hpp", "launch.hpp", "store_body.hpp", "api.cpp")]   # api.cpp: the launch choices


def traffic_file(workload):
    return os.path.join(PROFILES, f"decode_step_{workload}_traffic.json")


def trace_file(workload):
    return os.path.join(PROFILES, f"decode_step_{workload}_kernels.json")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_text(text):
    """C++ source without comments, trailing blanks or empty lines (what the compiler sees
    of the kernels, so that a comment edit does not invalidate a counter record)."""
    out, i, n, quote = [], 0, len(text), None
    while i < n:
        c = text[i]
        if quote:
            out.append(c)
            if c == "\\" and i + 1 < n:
                out.append(text[i + 1])
                i += 1
            elif c == quote:
                quote = None
        elif c in "\"'":
            quote = c
            out.append(c)
        elif text.startswith("//", i):
            while i < n and text[i] != "\n":
                i += 1
            continue
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
            continue
        else:
            out.append(c)
        i += 1
    lines = (ln.rstrip() for ln in "".join(out).split("\n"))
    return "\n".join(ln for ln in lines if ln)


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def row_lens_of(lay):
    """Causal length of every row: row i of a request with q_len rows sees
    seq_len - q_len + 1 + i tokens."""
    import numpy as np
    return np.concatenate([np.arange(int(s) - int(q) + 1, int(s) + 1, dtype=np.int64)
                           for s, q in zip(lay.seq_lens, lay.q_lens)])


def step_bytes(cfg, lay, ids_np, G):
    import numpy as np
    rb = 72 if cfg.fmt == "nvfp4" else 68
    R = int(lay.cu_q[-1])
    seq = lay.seq_lens.astype(np.int64)
    index = int(seq.sum()) * rb                                   # every causal index token
    pairs = set()
    row_req = np.repeat(np.arange(len(seq)), np.diff(lay.cu_q))
    for r in range(R):
        for j in ids_np[r]:
            if j >= 0:
                pairs.add((int(row_req[r]), int(j)))
    attend = 0
    for b, j in pairs:                                             # distinct (request, block) K+V
        attend += 2 * rb * min(128, int(seq[b]) - 128 * j)
    T = R
    store = T * 3 * 256 + T * 3 * rb                               # read bf16 rows, write planes
    tables = int(((seq + 127) // 128).sum()) * 4                   # causal block-table entries
    queries = R * 256 + R * G * 256                                # q_idx + q (bf16)
    outs = R * G * 128 * 4 + 2 * R * cfg.topk * 4                  # fp32 out + ids (write + read)
    other = store + tables + queries + outs
    index_call = index + tables + R * 256
    # m3s_index_topk_attend: the index call's bytes, the distinct selected K/V, the main
    # query, the fp32 output and the ids it writes
    fused_call = index_call + attend + R * G * 256 + R * G * 128 * 4 + R * cfg.topk * 4
    # m3s_decode_step: the fused call, the store, and the row map (cu_q and seq_lens in;
    # row_req, row_len and the block prefix out)
    B = len(seq)
    step_call = fused_call + store + (2 * B + 1) * 4 + 2 * R * 4 + (B + 1) * 4
    return {"index": index, "attend": attend, "store": store, "other": other,
            "total": index + attend + other, "index_call": index_call, "fused_call": fused_call,
            "step_call": step_call}


def cpu_baseline(cfg, case, nreq, log_fn):
    """The oracle as it stands, timed on the host on `nreq` whole requests of the workload."""
    import numpy as np
    import torch

    import workloads as W
    from oracle import path as P

    lay = case.layout
    reqs = list(range(nreq))
    # untimed: the oracle's own planes for the sampled requests' history
    planes = P.new_planes(cfg.fmt, lay.num_pages)
    slots = W.all_slots(lay)
    new = set(lay.new_tokens.tolist())
    new_rows = {}
    for b in reqs:
        lo, hi = int(lay.tok_off[b]), int(lay.tok_off[b + 1])
        keep = np.array([t not in new for t in range(lo, hi)])
        P.store(planes, cfg.fmt, {n: W.bf16_bits(getattr(case, n)[lo:hi])[keep] for n in ("k", "v", "idx")},
                slots[lo:hi][keep])
    nt = lay.new_tokens
    sel = np.concatenate([np.arange(int(lay.cu_q[b]), int(lay.cu_q[b + 1])) for b in reqs])
    for n in ("k", "v", "idx"):
        t = getattr(case, n)
        new_rows[n] = W.bf16_bits(t[torch.as_tensor(nt[sel], device=t.device)])
    q_idx = W.bf16_bits(case.q_idx)
    q = W.bf16_bits(case.q)
    threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    P.step(planes, cfg.fmt, new_rows, lay.new_slots[sel], lay.cu_q, lay.seq_lens, lay.block_table,
           q_idx, q, cfg.topk, cfg.sm_scale, requests=reqs)
    dt = time.perf_counter() - t0
    rows = int(sum(int(lay.cu_q[b + 1] - lay.cu_q[b]) for b in reqs))
    log_fn(f"[cpu baseline] oracle step on {nreq} request(s) ({rows} rows): {dt:.2f} s")
    return {"value": rows / dt, "unit": "rows/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{nreq} of {len(lay.seq_lens)} requests ({rows} rows) of the same workload, full step "
                      f"(store of their rows, row map, float64 dequantize + score of every causal block, "
                      f"sort top-k, float64 softmax attention), history quantization untimed; {dt:.1f} s"}


COPY_BYTES = 1 << 30          # the calibration copy reads and writes this many bytes


FRONT_KERNELS = ("store_rows_kernel", "store_prefill_rows_kernel", "store_kernel", "decode_rows_kernel",
                 "prefill_rows_kernel")
STEP_OPENERS = FRONT_KERNELS + ("step_scan_kernel",)   # the first kernel of a step, in each call mode


def kernel_short(name):
    """'void m3s::index_scan_kernel<1, 1, 16, 1>(m3s::IndexArgs)' -> 'index_scan_kernel<1, 1, 16, 1>'."""
    n = name.strip()
    if n.startswith("void "):
        n = n[5:]
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):       # the argument list starts at the first '(' outside '<...>'
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    n = n[:cut]
    return n[5:] if n.startswith("m3s::") else n


def _base(short):
    return short.split("<", 1)[0]


def step_sequences(dispatches):
    """dispatches: [(dispatch order, short kernel name, payload)] of the library's kernels.
    Splits them at each kernel that opens a step (the store, or the decode step's first
    kernel) and returns the most
    common kernel-name sequence and the list of runs that have it."""
    dispatches = sorted(dispatches, key=lambda t: t[0])
    runs, cur = [], None
    for d in dispatches:
        if _base(d[1]) in STEP_OPENERS and (cur is None or _base(cur[-1][1]) not in STEP_OPENERS):
            if cur:
                runs.append(cur)
            cur = [d]
        elif cur is not None:
            cur.append(d)
    if cur:
        runs.append(cur)
    count = {}
    for r in runs:
        key = tuple(x[1] for x in r)
        count[key] = count.get(key, 0) + 1
    if not count:
        raise SystemExit("no step found in the profile")
    best = max(count, key=lambda k: (count[k], len(k)))
    return list(best), [r for r in runs if tuple(x[1] for x in r) == best]


def _pmc_dispatches(path, counter):
    """[(dispatch id, short name, counter value in KiB summed over the dispatch)] from a
    rocprofv3 counter CSV."""
    import csv
    acc, names = {}, {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            did = int(row.get("Dispatch_Id") or row.get("Correlation_Id"))
            acc[did] = acc.get(did, 0.0) + float(row["Counter_Value"])
            names[did] = kernel_short(row["Kernel_Name"])
    return [(d, names[d], acc[d]) for d in acc]


def _median(v):
    v = sorted(v)
    n = len(v)
    return 0.5 * (v[(n - 1) // 2] + v[n // 2]) if n else 0.0


def ingest_pmc(fetch_csv, write_csv, config):
    """HBM bytes of every kernel of the decode step, from FETCH_SIZE / WRITE_SIZE counters
    scaled by what the same counters read for the calibration copy (COPY_BYTES read +
    COPY_BYTES written). Per kernel: the median over the steps of the graph replays."""
    import workloads as W
    cfg = W.config(int(config) if config.isdigit() else config)
    fd = _pmc_dispatches(fetch_csv, "FETCH_SIZE")
    wd = _pmc_dispatches(write_csv, "WRITE_SIZE")

    def copy_kib(ds):
        v = [x[2] for x in ds if "neg" in x[1]]
        if not v:
            raise SystemExit("no calibration copy (torch.neg) in the counter file")
        return _median(v)

    copy_f, copy_w = copy_kib(fd), copy_kib(wd)
    f_scale = COPY_BYTES / (copy_f * 1024.0)
    w_scale = COPY_BYTES / (copy_w * 1024.0)
    lib = lambda ds: [x for x in ds if "neg" not in x[1] and "::" not in x[1]]
    seq_f, runs_f = step_sequences(lib(fd))
    seq_w, runs_w = step_sequences(lib(wd))
    if seq_f != seq_w:
        raise SystemExit(f"the two passes ran different steps: {seq_f} / {seq_w}")
    parts = []
    for i, name in enumerate(seq_f):
        fk = _median([r[i][2] for r in runs_f])
        wk = _median([r[i][2] for r in runs_w])
        parts.append({"kernel": name, "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                      "steps": [len(runs_f), len(runs_w)],
                      "fetch_bytes": round(fk * 1024.0 * f_scale), "write_bytes": round(wk * 1024.0 * w_scale)})
    call = [p for p in parts if _base(p["kernel"]) not in FRONT_KERNELS]
    rec = {"workload": cfg.name, "source_sha": source_sha(KERNEL_SOURCES),
           "step_kernels": parts,
           "fused_call_bytes": sum(p["fetch_bytes"] + p["write_bytes"] for p in call),
           "step_bytes": sum(p["fetch_bytes"] + p["write_bytes"] for p in parts),
           "calibration": {"copy_bytes_each_way": COPY_BYTES, "copy_fetch_kib": round(copy_f, 1),
                           "copy_write_kib": round(copy_w, 1), "fetch_scale": round(f_scale, 4),
                           "write_scale": round(w_scale, 4)},
           "commands": ["cd /tmp && export TMPDIR=/tmp  # $R = repository root",
                        *[f"timeout -s KILL 200 rocprofv3 --pmc {c} --output-format csv -d "
                          f"$R/gpurun_out/pmc_{cfg.name}_{d} -o run -- python3 -u $R/bench.py --config {cfg.name} "
                          f"--steps 20 --warmup 2 --stage-reps 10 --no-cpu --copy-calibration"
                          for c, d in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write"))],
                        f"python bench.py --config {cfg.name} --ingest-pmc "
                        f"gpurun_out/pmc_{cfg.name}_fetch/run_counter_collection.csv "
                        f"gpurun_out/pmc_{cfg.name}_write/run_counter_collection.csv"]}
    path = traffic_file(cfg.name)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    log(json.dumps(rec, indent=1))


def ingest_trace(trace_csv, config):
    """Per-kernel durations of the decode step from a rocprofv3 kernel trace: the median,
    over the steps of the graph replays, of each kernel's duration, the step's span (first
    start to last end) and the gap before the next step."""
    import csv
    import workloads as W
    cfg = W.config(int(config) if config.isdigit() else config)
    ds = []
    with open(trace_csv, newline="") as f:
        for row in csv.DictReader(f):
            name = kernel_short(row["Kernel_Name"])
            if "::" in name or not name:
                continue
            ds.append((int(row["Dispatch_Id"]), name, (int(row["Start_Timestamp"]), int(row["End_Timestamp"]),
                                                        int(row["Grid_Size_X"]) // max(1, int(row["Workgroup_Size_X"])))))
    seq, runs = step_sequences(ds)
    runs.sort(key=lambda r: r[0][2][0])
    kern = []
    for i, name in enumerate(seq):
        dur = [(r[i][2][1] - r[i][2][0]) / 1e3 for r in runs]
        kern.append({"kernel": name, "workgroups": runs[0][i][2][2], "median_us": round(_median(dur), 2),
                     "mean_us": round(sum(dur) / len(dur), 2)})
    span = [(r[-1][2][1] - r[0][2][0]) / 1e3 for r in runs]
    starts = [r[0][2][0] for r in runs]
    ends = [r[-1][2][1] for r in runs]
    gaps = [(starts[i + 1] - ends[i]) / 1e3 for i in range(len(runs) - 1) if starts[i + 1] > ends[i]]
    rec = {"workload": cfg.name, "source_sha": source_sha(KERNEL_SOURCES), "steps": len(runs),
           "step_kernels": kern, "step_span_median_us": round(_median(span), 2),
           "gap_to_next_step_median_us": round(_median(gaps), 2) if gaps else None,
           "commands": ["cd /tmp && export TMPDIR=/tmp  # $R = repository root",
                        f"timeout -s KILL 200 rocprofv3 --kernel-trace --stats --output-format csv -d "
                        f"$R/gpurun_out/prof_{cfg.name} -o run -- python3 -u $R/bench.py --config {cfg.name} "
                        f"--steps 100 --warmup 10 --no-cpu",
                        f"python bench.py --config {cfg.name} --ingest-trace "
                        f"gpurun_out/prof_{cfg.name}/run_kernel_trace.csv"]}
    path = trace_file(cfg.name)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    log(json.dumps(rec, indent=1))


def load_record(path, workload, calls=None):
    """A committed profile record, if it was taken on the current kernel code (and, given
    calls, in that call mode: a decode step record opens with the step's scan kernel)."""
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != source_sha(KERNEL_SOURCES) or rec.get("workload") != workload:
        return None
    if calls is not None:
        first = _base(rec["step_kernels"][0]["kernel"]) if rec.get("step_kernels") else ""
        if (first == "step_scan_kernel") != (calls == "step"):
            return None
    return rec


def ceilings(m3s, cfg, dev, layers):
    """Page-read ceilings of the index scan's access pattern (m3s_probe_page_reads): the
    workload's index planes (one per layer, as in the bench), every causal page read once
    per launch in a random order, then the same pages in address order; launches cycle
    over the layers so that no launch is served from the Infinity Cache."""
    import numpy as np
    import torch
    import workloads as W
    lay = W.make_layout(cfg.seq_lens, cfg.q_len, cfg.seed)
    P = lay.num_pages
    npages = int(lay.nblk.sum())
    rng = np.random.default_rng(1234)
    planes = [(torch.randint(0, 255, (P, 128, 64), dtype=torch.uint8, device=dev),
               torch.randint(0, 255, (P, 128, 8), dtype=torch.uint8, device=dev)) for _ in range(layers)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(cus, dtype=torch.int32, device=dev)
    orders = {"random": torch.as_tensor(rng.permutation(P)[:npages].astype(np.int32), device=dev),
              "sequential": torch.arange(npages, dtype=torch.int32, device=dev)}
    res = {"workload": cfg.name, "pages_per_launch": npages, "bytes_per_launch": npages * 128 * 72,
           "layers_cycled": layers, "cus": cus}
    reps = 40
    for order, pages in orders.items():
        for mode in (0, 1):
            for L in range(layers):   # warm-up; the page ids are checked once, here
                m3s.m3s_probe_page_reads(planes[L][0], planes[L][1], pages, mode, sink, check=True)
            best = None
            for trial in range(3):
                ea = torch.cuda.Event(enable_timing=True)
                eb = torch.cuda.Event(enable_timing=True)
                torch.cuda._sleep(3_000_000)
                ea.record()
                for i in range(reps):
                    L = i % layers
                    m3s.m3s_probe_page_reads(planes[L][0], planes[L][1], pages, mode, sink, check=False)
                eb.record()
                torch.cuda.synchronize()
                t = ea.elapsed_time(eb) / reps
                best = t if best is None else min(best, t)
            key = f"{order}_scales_{'2B' if mode == 0 else '16B'}"
            res[key] = {"us_per_launch": round(best * 1e3, 2),
                        "gbs": round(npages * 128 * 72 / (best * 1e-3) / 1e9, 1)}
            log(f"[ceilings] {key}: {best * 1e3:.2f} us, {res[key]['gbs']:.0f} GB/s")

    # plain streams for comparison (probe mode 2): the same bytes front to back, and a
    # stream of every layer's bytes at once (past the Infinity Cache, no launch cycling)
    def stream(pl, n, grid, reps_, cycle):
        sk = torch.zeros(grid, dtype=torch.int32, device=dev)
        idx = torch.arange(n, dtype=torch.int32, device=dev)
        for L in range(len(pl)):
            m3s.m3s_probe_page_reads(pl[L][0], pl[L][1], idx, 2, sk)
        best = None
        for trial in range(3):
            ea = torch.cuda.Event(enable_timing=True)
            eb = torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(3_000_000)
            ea.record()
            for i in range(reps_):
                L = i % len(pl) if cycle else 0
                m3s.m3s_probe_page_reads(pl[L][0], pl[L][1], idx, 2, sk, check=False)
            eb.record()
            torch.cuda.synchronize()
            t = ea.elapsed_time(eb) / reps_
            best = t if best is None else min(best, t)
        return best

    for grid in (cus, 2 * cus):
        best = stream(planes, npages, grid, reps, True)
        key = f"stream_same_bytes_grid{grid}"
        res[key] = {"us_per_launch": round(best * 1e3, 2), "gbs": round(npages * 128 * 72 / (best * 1e-3) / 1e9, 1)}
        log(f"[ceilings] {key}: {best * 1e3:.2f} us, {res[key]['gbs']:.0f} GB/s")
    big = [(torch.cat([p[0] for p in planes]), torch.cat([p[1] for p in planes]))]
    nb_ = big[0][0].shape[0]
    del planes
    best = stream(big, nb_, 8 * cus, 10, False)
    key = f"stream_{nb_ * 128 * 72 >> 20}MB_grid{8 * cus}"
    res[key] = {"us_per_launch": round(best * 1e3, 2), "gbs": round(nb_ * 128 * 72 / (best * 1e-3) / 1e9, 1)}
    log(f"[ceilings] {key}: {best * 1e3:.2f} us, {res[key]['gbs']:.0f} GB/s")
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", default="b8x8_150k")
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--cpu-requests", type=int, default=6)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--stage-reps", type=int, default=20)
    ap.add_argument("--calls", choices=("step", "two", "separate"), default="step",
                    help="step: one m3s_decode_step call (decode workloads; a prefill chunk runs 'two'); "
                         "two: m3s_store_and_rows (decode) or m3s_store_and_prefill_rows (prefill), then "
                         "m3s_index_topk_attend; separate: m3s_store, the row map, m3s_index_topk, "
                         "m3s_sparse_attend")
    ap.add_argument("--separate", action="store_true", help="same as --calls separate")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB float32 copy kernel (torch.neg) whose HBM bytes are known, "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE run, "
                         "WRITE_SIZE run) of 'bench.py --copy-calibration' into the traffic record")
    ap.add_argument("--ingest-trace", metavar="TRACE_CSV",
                    help="no GPU: turn a rocprofv3 kernel_trace.csv of the bench into the per-kernel record")
    ap.add_argument("--graph-layers", type=int, default=0,
                    help="steps captured in one HIP graph (default: all --layers, one step per layer cache, "
                         "as a model's decode graph holds its layers; 1: one graph per step)")
    ap.add_argument("--ceilings", action="store_true",
                    help="measure the page-read ceilings of the index scan's access pattern and exit")
    args = ap.parse_args()
    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.config)
        return
    if args.ingest_trace:
        ingest_trace(args.ingest_trace, args.config)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: the path is one GPU's share (one KV head, one TP rank); "
              f"--gpus {args.gpus} / WORLD_SIZE {world} is not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_decode_nvfp4_amd as m3s
    import workloads as W

    m3s.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = W.config(int(args.config) if args.config.isdigit() else args.config)
    if args.ceilings:
        ceilings(m3s, cfg, dev, max(1, args.layers))
        return
    log(f"[bench] workload {cfg.name}: {cfg.description}")
    t_setup = time.perf_counter()
    case = W.make_case(cfg, dev)
    lay = case.layout
    R = int(lay.cu_q[-1])
    G = case.q.shape[1]
    NL = max(1, args.layers)

    # ---- per-layer caches, history stored by the library (untimed setup)
    slots_all = torch.as_tensor(W.all_slots(lay), device=dev)
    hist = torch.ones(lay.total_tokens, dtype=torch.bool, device=dev)
    new_idx = torch.as_tensor(lay.new_tokens, device=dev)
    hist[new_idx] = False
    hidx = torch.nonzero(hist).flatten()
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    caches = []
    for L in range(NL):
        c = m3s.Cache(cfg.fmt, lay.num_pages, dev)
        for s in range(0, hidx.numel(), 1 << 20):
            h = hidx[s: s + (1 << 20)]
            m3s.m3s_store(c, case.k[h], case.v[h], case.idx[h], slots_all[h].contiguous(), status)
        caches.append(c)
    torch.cuda.synchronize()

    # ---- static step buffers
    k_new = case.k[new_idx].contiguous()
    v_new = case.v[new_idx].contiguous()
    i_new = case.idx[new_idx].contiguous()
    s_new = slots_all[new_idx].contiguous()
    cu_q = torch.as_tensor(lay.cu_q, device=dev)
    seq = torch.as_tensor(lay.seq_lens, device=dev)
    bt = torch.as_tensor(lay.block_table, device=dev)
    prefill = int(lay.q_lens.max()) > 16   # chunks of more than 16 rows: the prefill row map
    row_req = torch.empty(R, dtype=torch.int32, device=dev)
    row_len = torch.empty(R, dtype=torch.int32, device=dev)
    req_blk = torch.empty(len(lay.seq_lens) + 1, dtype=torch.int32, device=dev)
    if prefill:
        rows = m3s.m3s_prefill_rows(cu_q, seq, R, dev_status=status)
    else:
        rows = m3s.m3s_decode_rows(cu_q, seq, R, row_req, row_len, req_blk, status)

    def row_map():
        if prefill:
            m3s.m3s_prefill_rows(cu_q, seq, R, rows.num_groups, status, out=rows)
        else:
            m3s.m3s_decode_rows(cu_q, seq, R, row_req, row_len, req_blk, status)
    ids = torch.empty((R, cfg.topk), dtype=torch.int32, device=dev)
    out = torch.empty((R, G, 128), dtype=torch.float32, device=dev)
    ws_i = m3s.index_workspace(rows, lay.max_blocks, cfg.topk, dev)
    ws_a = m3s.attend_workspace(rows, lay.max_blocks, cfg.topk, G, dev)

    ws_f = m3s.index_attend_workspace(rows, lay.max_blocks, cfg.topk, G, dev)
    calls = "separate" if args.separate else args.calls
    if calls == "step" and prefill:
        calls = "two"
    fused_front = not prefill and calls != "separate"
    fused_attend = calls != "separate"

    def decode_step(c):
        m3s.m3s_decode_step(c, k_new, v_new, i_new, s_new, cu_q, seq, R, row_req, row_len, req_blk, case.q_idx,
                            case.q, bt, lay.max_blocks, cfg.topk, cfg.sm_scale, 0, ids, out, ws_f, status)

    def run_step(c):
        if calls == "step":
            decode_step(c)
            return
        if fused_front:
            m3s.m3s_store_and_rows(c, k_new, v_new, i_new, s_new, cu_q, seq, R, row_req, row_len, req_blk, status)
        elif prefill and calls != "separate":
            m3s.m3s_store_and_prefill_rows(c, k_new, v_new, i_new, s_new, cu_q, seq, R, rows.num_groups, status,
                                           out=rows)
        else:
            m3s.m3s_store(c, k_new, v_new, i_new, s_new, status)
            row_map()
        if fused_attend:
            m3s.m3s_index_topk_attend(c, case.q_idx, case.q, bt, lay.max_blocks, rows, cfg.topk, cfg.sm_scale, 0,
                                      ids, out, ws_f, status)
        else:
            m3s.m3s_index_topk(c, case.q_idx, bt, lay.max_blocks, rows, cfg.topk, 0, ids, ws_i, status)
            m3s.m3s_sparse_attend(c, case.q, bt, lay.max_blocks, rows, ids, cfg.sm_scale, out, ws_a, status)

    for c in caches:  # eager warm-up, checks the status word
        run_step(c)
    torch.cuda.synchronize()
    st = int(status.item())
    if st:
        log(f"[bench] device status {st:#x}")
        sys.exit(3)

    # ---- graphs: one per layer (the whole step), and one holding GL consecutive steps over
    # the layer caches in turn, as a model's decode graph holds its layers (the launch of a
    # graph then comes once per GL steps instead of once per step)
    side = torch.cuda.Stream()
    graphs = []
    for c in caches:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            run_step(c)
        graphs.append(g)
    GL = NL if args.graph_layers <= 0 else min(args.graph_layers, NL)
    multi = None
    if GL > 1:
        multi = torch.cuda.CUDAGraph()
        with torch.cuda.graph(multi, stream=side):
            for c in caches[:GL]:
                run_step(c)
    torch.cuda.synchronize()
    log(f"[bench] setup {time.perf_counter() - t_setup:.1f} s; {NL} layers x {lay.num_pages} pages; "
        f"rows {R}, G {G}, top-k {cfg.topk}; {GL} steps per graph")

    def run_steps(k):
        """k steps: k // GL replays of the multi-step graph, then single-step graphs."""
        done = 0
        if multi is not None:
            for _ in range(k // GL):
                multi.replay()
            done = (k // GL) * GL
        for i in range(done, k):
            graphs[i % NL].replay()

    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] calibration copy: {COPY_BYTES >> 20} MiB read + written, 3 launches")

    # ---- timed region: exactly K steps
    run_steps(args.warmup)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    run_steps(args.steps)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / args.steps
    st = int(status.item())

    # one graph per step, for comparison: the same steps with a graph launch each
    n1 = min(max(args.steps, 1), 8 * NL)
    e2 = torch.cuda.Event(enable_timing=True)
    e3 = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(5_000_000)
    e2.record()
    for i in range(n1):
        graphs[i % NL].replay()
    e3.record()
    torch.cuda.synchronize()
    ms_single = e2.elapsed_time(e3) / n1

    # ---- per-replay distribution: an event between consecutive replays, the whole run
    # queued behind a GPU spin so that the host's enqueue rate does not show; the events'
    # own cost lands inside the intervals, so these read slightly above ms_per_step
    nd = min(args.steps, 100)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nd + 1)]
    torch.cuda._sleep(20_000_000)
    evs[0].record()
    for i in range(nd):
        graphs[i % NL].replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_us = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(nd))

    def pct(f):
        return round(per_us[min(nd - 1, int(round(f * (nd - 1))))], 2)
    step_dist = {"replays": nd, "p10": pct(0.1), "median": pct(0.5), "p90": pct(0.9)}

    # ---- per-stage HIP-event times. Events cannot be recorded inside a captured graph on
    # ROCm, so each stage is launched eagerly, args.stage_reps times back to back (cycling
    # the layer caches), between two events on the stream it runs on; a GPU spin first lets
    # every launch queue up before the GPU reaches it, so no host launch gap lands inside
    # and the events' own cost is spread over the repetitions.
    fused_prefill_front = prefill and calls != "separate"

    def front(c):
        if fused_front:
            m3s.m3s_store_and_rows(c, k_new, v_new, i_new, s_new, cu_q, seq, R, row_req, row_len, req_blk, status)
        elif fused_prefill_front:
            m3s.m3s_store_and_prefill_rows(c, k_new, v_new, i_new, s_new, cu_q, seq, R, rows.num_groups, status,
                                           out=rows)
        else:
            m3s.m3s_store(c, k_new, v_new, i_new, s_new, status)
            row_map()

    front_name = ("store_and_rows" if fused_front else
                  "store_and_prefill_rows" if fused_prefill_front else
                  "store+prefill_rows" if prefill else "store+decode_rows")
    stages = [(front_name, front),
              ("index_topk", lambda c: m3s.m3s_index_topk(c, case.q_idx, bt, lay.max_blocks, rows, cfg.topk, 0,
                                                           ids, ws_i, status)),
              ("sparse_attend", lambda c: m3s.m3s_sparse_attend(c, case.q, bt, lay.max_blocks, rows, ids,
                                                                 cfg.sm_scale, out, ws_a, status)),
              ("index_topk_attend", lambda c: m3s.m3s_index_topk_attend(c, case.q_idx, case.q, bt, lay.max_blocks,
                                                                         rows, cfg.topk, cfg.sm_scale, 0, ids, out,
                                                                         ws_f, status))]
    if not prefill:
        # the fused producer store (norm + rotary + FP4 store + query rows) for the step's new
        # tokens, beside the plain store of the same rows, each into its own one-page cache
        # (the layer caches keep the bytes the step stored)
        T_new = int(new_idx.numel())
        pc = m3s.Cache(cfg.fmt, (T_new + 127) // 128, dev)
        p_slots = torch.arange(T_new, dtype=torch.int32, device=dev)
        p_q = W.gen_prenorm_rows((T_new, G, 128), cfg.seed, W.PQ_FAMILY, dev)
        p_rows = [W.gen_prenorm_rows((T_new, 128), cfg.seed, f, dev)
                  for f in (W.PK_FAMILY, W.PV_FAMILY, W.PIQ_FAMILY, W.PIK_FAMILY)]
        p_w = W.gen_norm_weights(cfg.seed, dev)
        p_cs = torch.as_tensor(W.rope_table(int(lay.seq_lens.max()), PRODUCER_ROTARY_DIM), device=dev)
        p_pos = torch.as_tensor(W.new_positions(lay), device=dev)
        p_out = (torch.empty((T_new, G, 128), dtype=torch.bfloat16, device=dev),
                 torch.empty((T_new, 128), dtype=torch.bfloat16, device=dev))
        stages += [("qknorm_rope_store", lambda c: m3s.m3s_qknorm_rope_store(
                       pc, p_q, *p_rows, p_w, 1e-6, p_pos, p_cs, p_slots, q_out=p_out[0], idx_q_out=p_out[1],
                       dev_status=status)),
                   ("store", lambda c: m3s.m3s_store(pc, k_new, v_new, i_new, p_slots, status)),
                   ("decode_step", decode_step)]
    reps = max(1, args.stage_reps)
    stage_ms = []
    for _, fn in stages:
        best = None
        for trial in range(3):
            ea = torch.cuda.Event(enable_timing=True)
            eb = torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(3_000_000)
            ea.record()
            for i in range(reps):
                fn(caches[(trial * reps + i + 1) % NL])
            eb.record()
            torch.cuda.synchronize()
            t = ea.elapsed_time(eb) / reps
            best = t if best is None else min(best, t)
        stage_ms.append(best)

    st = st | int(status.item())

    ids_np = ids.cpu().numpy()
    by = step_bytes(cfg, lay, ids_np, G)
    rows_per_s = R / (ms_per_step / 1e3)
    gbs_step = by["total"] / (ms_per_step / 1e3) / 1e9
    log(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.2f} us/step (event), wall {wall / args.steps * 1e6:.2f} us/step; "
        f"{ms_single * 1e3:.2f} us/step with one graph launch per step")
    log(f"[bench] per replay ({nd} replays, events between them): p10 {step_dist['p10']:.2f}, "
        f"median {step_dist['median']:.2f}, p90 {step_dist['p90']:.2f} us")
    log(f"[bench] algorithmic bytes/step: index {by['index'] / 1e6:.2f} MB, attend {by['attend'] / 1e6:.2f} MB, "
        f"other {by['other'] / 1e6:.2f} MB, total {by['total'] / 1e6:.2f} MB -> {gbs_step:.0f} GB/s")
    roofline = roofline_index = kernel_split = None
    trace = load_record(trace_file(cfg.name), cfg.name, calls)
    traffic = load_record(traffic_file(cfg.name), cfg.name, calls)
    stage_of = {nm: v for (nm, _), v in zip(stages, stage_ms)}
    if stage_ms:
        names = [nm for nm, _ in stages]
        log("[bench] stages (us, each stage launched back to back): " +
            ", ".join(f"{nm} {v * 1e3:.2f}" for nm, v in zip(names, stage_ms)))
        t_idx = stage_ms[1] / 1e3
        t_fused = stage_ms[3] / 1e3
        call_kernels = None
        if trace:
            call_kernels = [k["kernel"] for k in trace["step_kernels"] if _base(k["kernel"]) not in FRONT_KERNELS]
        if calls == "step":
            # the call the step runs: m3s_decode_step, the whole path's algorithmic bytes
            # over its launch time (HIP events on its stream)
            t_call = stage_of["decode_step"] / 1e3
            ach = by["step_call"] / t_call / 1e9
            step_kernels = [k["kernel"] for k in trace["step_kernels"]] if trace else None
            roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(ach / HBM_PEAK_GBS, 4),
                        "traffic": traffic["step_bytes"] if traffic else None,
                        "kernel": "m3s_decode_step" + (f" ({', '.join(step_kernels)})" if step_kernels else ""),
                        "launch_us": round(t_call * 1e6, 2), "bytes_per_launch": by["step_call"]}
        else:
            # the call the step runs: m3s_index_topk_attend, its algorithmic bytes over its
            # launch time (HIP events on its stream)
            ach = by["fused_call"] / t_fused / 1e9
            roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(ach / HBM_PEAK_GBS, 4),
                        "traffic": traffic["fused_call_bytes"] if traffic else None,
                        "kernel": "m3s_index_topk_attend" + (f" ({', '.join(call_kernels)})" if call_kernels else ""),
                        "launch_us": round(stage_ms[3] * 1e3, 2), "bytes_per_launch": by["fused_call"]}
        ach_i = by["index_call"] / t_idx / 1e9
        roofline_index = {"kernel": "m3s_index_topk (scan + select)", "achieved": round(ach_i, 1),
                          "frac": round(ach_i / HBM_PEAK_GBS, 4), "launch_us": round(stage_ms[1] * 1e3, 2),
                          "bytes_per_launch": by["index_call"]}
        if prefill:
            # A prefill chunk's pages stay in the caches while every 16-row group re-scores
            # them: the scan is bound by the matrix cores, not HBM. Algorithmic work is one
            # 128-dim dot product (256 flop) per (row, causal token); the NVFP4 scan runs on
            # fp16 MFMA, the MXFP4 scan on the scaled fp4 x fp8 MFMA (fp8 rate).
            flop = 256 * int(row_lens_of(lay).astype("int64").sum())
            peak = MFMA_PEAK_TFLOPS["f16" if cfg.fmt == "nvfp4" else "fp8"]
            tf_s = flop / t_idx / 1e12
            roofline = {"bound": "mfma", "achieved": round(tf_s, 1), "peak": peak, "unit": "TFLOP/s",
                        "frac": round(tf_s / peak, 4), "traffic": None,
                        "kernel": "m3s_index_topk (index_scan + index_select kernels)",
                        "launch_us": round(stage_ms[1] * 1e3, 2), "flop_per_launch": flop}
    if trace:
        # per-kernel durations of the step from the committed kernel trace (taken on the
        # current kernel code), with the algorithmic bytes of the kernels that have them
        kb = {"index_scan_kernel": by["index_call"], "step_scan_kernel": by["index_call"] + by["store"]}
        kernel_split = []
        for k in trace["step_kernels"]:
            b = kb.get(_base(k["kernel"]))
            e = {"kernel": k["kernel"], "us": k["median_us"]}
            if b:
                e["bytes"] = b
                e["frac"] = round(b / (k["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
            kernel_split.append(e)
        log("[bench] kernel split (profiles/): " + ", ".join(f"{e['kernel']} {e['us']}" for e in kernel_split))

    cpu = None
    if not args.no_cpu and not prefill:  # the oracle on a 4096-row chunk takes hours
        cpu = cpu_baseline(cfg, case, args.cpu_requests, log)

    res = {
        "metric": METRIC if not prefill else (
            f"prefill rows/s + achieved HBM GB/s (store+prefill_rows+score+top-k+attend), "
            f"{len(lay.seq_lens)} req x {int(lay.q_lens.max())}-token chunk @{int(lay.seq_lens.max()) // 1000}K"),
        "value": round(rows_per_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "requests": len(lay.seq_lens), "rows_per_request": cfg.q_len,
                   "context": [int(x) for x in sorted(set(lay.seq_lens.tolist()))][:4],
                   "heads_per_kv_head": G, "topk": cfg.topk, "cache_format": cfg.fmt, "layers_cycled": NL,
                   "calls": {"step": "m3s_decode_step",
                             "two": ("m3s_store_and_prefill_rows" if prefill else "m3s_store_and_rows") +
                                    ", m3s_index_topk_attend",
                             "separate": "m3s_store, " + ("m3s_prefill_rows" if prefill else "m3s_decode_rows") +
                                         ", m3s_index_topk, m3s_sparse_attend"}[calls]},
        "hbm_gbs_step": round(gbs_step, 1),
        "steps_per_graph": GL,
        "us_per_step_one_graph_each": round(ms_single * 1e3, 2),
        "step_us_dist": step_dist,
        "bytes_per_step": by["total"],
        "stage_us": None if not stage_ms else {nm: round(v * 1e3, 2) for (nm, _), v in zip(stages, stage_ms)},
        "device_status": st,
        "roofline": roofline,
        "roofline_index_topk": roofline_index,
        "kernel_split": kernel_split,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
