#!/usr/bin/env python3
"""Input GB/s parsed end to end on one MI355X, with roofline and CPU baseline.

Default workload: the quote-heavy CSV, 1 GiB, 12 columns, 60% quoted fields
with doubled quotes and embedded newlines, geometric field lengths (mean 40 B,
max 4 KiB), parsed with the five-state RFC 4180 DFA. One step is one ppr_parse
call over the whole input (every step of the path: per-chunk multi-DFA,
composite scan, re-simulation and tagging, offset scans, field emission), with
the input already resident in HBM and output buffers preallocated.

    python bench.py [--steps K] [--warmup W] [--workload csv3|csv1|csv2|csv4|lex5]

Prints one JSON line.
"""
import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
METRIC = "input GB/s parsed end-to-end (1 GiB CSV) and % of MI355X HBM peak"
WORKLOADS = {"csv1": 1, "csv2": 2, "csv3": 3, "csv4": 4, "lex5": 5}
KERNEL_SRC = {"csv": "dfa_parsing_delimiter_amd/csrc/ppr_csv.hip", "lex": "dfa_parsing_delimiter_amd/csrc/ppr_lex.hip"}
KERNEL_NAME = {"csv": "csv_parse_kernel", "lex": "lex_kernel"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_sha(kind):
    h = hashlib.sha256()
    for p in (KERNEL_SRC[kind], "dfa_parsing_delimiter_amd/csrc/ppr_device.h", "dfa_parsing_delimiter_amd/csrc/ppr_host.h"):
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kind, workload, chunk):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "counters_%s_%s_c%d.json" % (KERNEL_NAME[kind], workload, chunk))
    if not os.path.exists(path):
        return None
    c = json.load(open(path))
    if c.get("source_sha") != src_sha(kind):
        return None
    return c.get("hbm_bytes_per_launch")


def cpu_oracle_baseline(kind, data, table_or_dfa, max_seconds=30.0):
    """The oracle as it stands, on the host: one thread over the whole input
    (median of up to 3 runs within the time bound), and all host threads (at
    most 16) each parsing its own contiguous slice as an independent input."""
    import oracle
    runs, res = [], None
    t_end = time.time() + max_seconds
    for i in range(3):
        t0 = time.perf_counter()
        res = oracle.csv_parse(data, table_or_dfa) if kind == "csv" else oracle.lex_restart(data, table_or_dfa)
        runs.append(time.perf_counter() - t0)
        if time.time() + runs[-1] > t_end:
            break
    single = data.size / statistics.median(runs) / 1e9
    cores = min(16, os.cpu_count() or 1)
    slices = [data[i * data.size // cores:(i + 1) * data.size // cores] for i in range(cores)]

    def one(s):
        if kind == "csv":
            oracle.csv_parse(s, table_or_dfa)
        else:
            oracle.lex_restart(s, table_or_dfa)

    with cf.ThreadPoolExecutor(cores) as ex:
        t0 = time.perf_counter()
        list(ex.map(one, slices))
        dt = time.perf_counter() - t0
    return res, {"value": round(single, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
                 "sample": "the whole %d-byte input, sequential C oracle (gcc -O2), median of %d run(s)" % (
                     data.size, len(runs))}, {
        "value": round(data.size / dt / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": "the same input cut into %d contiguous slices parsed as independent inputs, one thread each" % cores}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="csv3", choices=sorted(WORKLOADS))
    ap.add_argument("--chunk", type=int, default=None, help="bytes per thread (default: the workload's, else 32)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline and the parity check")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dfa_parsing_delimiter_amd as ppr
    import workloads as W

    cfg_id = WORKLOADS[args.workload]
    cfg = W.CONFIGS[cfg_id]
    kind = "csv" if cfg["kind"] == "csv" else "lex"
    chunk = args.chunk or cfg.get("chunk_bytes") or 32
    dev = torch.device("cuda:0")
    log("generating", cfg["name"], cfg["n"], "bytes")
    t0 = time.time()
    data = W.generate(cfg_id)
    sha = W.sha256(data)
    log("generated in %.1fs sha256 %s" % (time.time() - t0, sha[:16]))
    d = torch.from_numpy(data).to(dev)
    n = data.size

    if kind == "csv":
        table = W.table(cfg["table"])
        runner = ppr.Parser(table, max_n=n, capacity=max(4096, n // 8), chunk_bytes=chunk, device=dev)
        first = runner(d)
        runner._alloc(first.n_fields)
        n_out = first.n_fields
        out_bytes_per_item = 16
        spec = table
    else:
        dfa = W.lexer_dfa()
        tabs = ppr.LexTables.from_dfa(dfa, dev)
        runner = ppr.Lexer(tabs, max_n=n, capacity=max(4096, n // 3), chunk_bytes=chunk)
        first = runner(d)
        runner._alloc(first.n_tokens)
        n_out = first.n_tokens
        out_bytes_per_item = 12
        spec = dfa
    log("first call:", n_out, "items")

    for _ in range(args.warmup):
        runner.launch(d)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        runner.launch(d)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = ev0.elapsed_time(ev1) / args.steps
    o = runner.results(n)
    got = int(o.n_fields if kind == "csv" else o.n_tokens)
    assert got == n_out, (got, n_out)

    gbs = n / (ms * 1e-3) / 1e9
    alg_bytes = n + out_bytes_per_item * n_out
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    traffic = measured_traffic(kind, args.workload, chunk)
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "pct_of_hbm_peak_input": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "config": {"workload": "%s_%dMiB" % (cfg["name"], n >> 20), "n_bytes": n, "chunk_bytes": chunk,
                   "table": cfg.get("table", "lexer_40_rules"), "items": n_out, "seed": W.seed_of(cfg_id),
                   "input_sha256": sha[:16]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic / (ms * 1e-3) / 1e9, 2),
                     "kernel": KERNEL_NAME[kind], "algorithmic_bytes_per_launch": alg_bytes,
                     "timing": "HIP events on the launch stream over %d back-to-back calls; wall %.3fs" % (
                         args.steps, wall)},
    }
    if not args.no_cpu:
        log("cpu oracle baseline")
        ref, single, allcore = cpu_oracle_baseline(kind, data, spec)
        line["cpu_baseline"] = single
        line["cpu_baseline_all_threads"] = allcore
        # bit-exact check of the timed configuration against the oracle
        keys = (("record_idx", "rec"), ("column_ids", "col"), ("field_offsets", "off"), ("field_lengths", "len")) \
            if kind == "csv" else (("kind", "kind"), ("start", "start"), ("length", "length"))
        res = runner(d)
        ok = (res.n_fields if kind == "csv" else res.n_tokens) == (ref["n_fields"] if kind == "csv" else
                                                                  ref["n_tokens"])
        for a, b in keys:
            ok = ok and bool(np.array_equal(getattr(res, a).cpu().numpy().view(np.uint32), ref[b]))
        line["parity_vs_oracle"] = "bit-exact" if ok else "MISMATCH"
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
