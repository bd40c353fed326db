#!/usr/bin/env python3
"""Input GB/s parsed end to end on one MI355X, with roofline and CPU baseline.

Default workload: the quote-heavy CSV, 1 GiB, 12 columns, 60% quoted fields
with doubled quotes and embedded newlines, geometric field lengths (mean 40 B,
max 4 KiB), parsed with the five-state RFC 4180 DFA. One step is one blocking
ppr_parse call over the whole input (every step of the path: per-chunk
multi-DFA, composite scan, re-simulation and tagging, offset scans, field
emission, scalar read-back), with the input already resident in HBM and the
output buffers preallocated.

    python bench.py [--steps K] [--warmup W] [--workload csv3|csv1|csv2|csv4|lex5] [--chunk L]
                    [--path auto|fused|streaming|single-pass]

Prints one JSON line. Two more modes serve the counter-based traffic figure:

    rocprofv3 --pmc FETCH_SIZE -d DIR1 -o run --output-format csv -- python bench.py --copy-calibration ...
    rocprofv3 --pmc WRITE_SIZE -d DIR2 -o run --output-format csv -- python bench.py --copy-calibration ...
    python bench.py --summarize-pmc DIR1 DIR2 [--workload ...]

--copy-calibration also times a plain 1 GiB device-to-device copy after the
parse, so that each counter can be scaled by what it reads for a copy of known
size; --summarize-pmc writes profiles/hbm_counters_<workload>_chunk<L>.json.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
METRIC = "input GB/s parsed end-to-end (1 GiB CSV) and % of MI355X HBM peak"
WORKLOADS = {"csv1": 1, "csv2": 2, "csv3": 3, "csv4": 4, "lex5": 5}
COPY_BYTES = 1 << 30
# kernels of each path, in launch order (the library records an event before
# the first and after each one)
STAGES = {1: ["csv_codes_kernel", "csv_carries_kernel", "csv_emit_kernel"],
          2: ["csv_reset_kernel", "csv_generic_kernel"],
          3: ["csv_fast_tables_kernel", "csv_fused_kernel"],
          "lex1": ["lex_ids_kernel", "lex_count_kernel", "lex_emit_kernel"],
          "lex2": ["lex_reset_kernel", "lex_kernel"]}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_file(name):
    """the kernel source file that defines kernel `name` (None: not found)"""
    pat = re.compile(r"__global__[^;{]{0,200}?\b%s\s*\(" % re.escape(name))
    for p in sorted(glob.glob(os.path.join(ROOT, "dfa_parsing_delimiter_amd", "csrc", "*.hip"))):
        if pat.search(open(p).read()):
            return p
    return None


def source_sha(kernel=None):
    """hash of the sources a kernel is built from (its .hip file and every shared
    header; every source when no kernel is named): counter summaries taken on other
    sources are stale"""
    csrc = os.path.join(ROOT, "dfa_parsing_delimiter_amd", "csrc")
    files = sorted(glob.glob(os.path.join(csrc, "*.h")))
    kf = kernel_file(kernel) if kernel else None
    files += [kf] if kf else sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.cpp")))
    h = hashlib.sha256()
    for p in files:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def counters_path(workload, chunk):
    return os.path.join(ROOT, "profiles", "hbm_counters_%s_chunk%d.json" % (workload, chunk))


def algorithmic_bytes(stage, n, n_out, out_bytes_per_item):
    """The bytes the method itself must move, attributed to the kernel that moves
    them: the input read once (by the first kernel that reads it), the outputs
    written once (by the kernel that writes them). Intermediates are not counted."""
    if stage in ("csv_codes_kernel", "lex_ids_kernel"):
        return n
    if stage in ("csv_emit_kernel", "lex_emit_kernel"):
        return out_bytes_per_item * n_out
    if stage in ("csv_generic_kernel", "csv_fused_kernel", "lex_kernel"):
        return n + out_bytes_per_item * n_out
    return 0


def host_cpu():
    """what the host offers this process: CPU model, nproc, the cores it may run on"""
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    allowed = sorted(os.sched_getaffinity(0))
    return {"model": model, "nproc": os.cpu_count(), "allowed_cores": len(allowed)}, allowed


def all_core_threads(allowed):
    """threads for the all-core CPU baseline: every core this process may run on,
    but no more than OMP_NUM_THREADS where it is set (the share of the host's
    cores that one GPU's job is given)"""
    k = len(allowed)
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        k = min(k, int(omp))
    return max(1, k)


def cpu_oracle_baseline(kind, data, spec, max_seconds=30.0):
    """The oracle as it stands, on the host: one thread pinned to one core, over
    the whole input (median of up to 3 runs within the time bound); and the
    all-core CPU baseline (the data-parallel method on host threads), checked
    bit-exact against the oracle's result."""
    import numpy as np
    import oracle
    info, allowed = host_cpu()
    runs, res = [], None
    t_end = time.time() + max_seconds
    pin = allowed[len(allowed) // 2]
    os.sched_setaffinity(0, {pin})  # this thread only: the oracle runs in it (ctypes)
    try:
        for _ in range(3):
            t0 = time.perf_counter()
            res = oracle.csv_parse(data, spec) if kind == "csv" else oracle.lex_restart(data, spec)
            runs.append(time.perf_counter() - t0)
            if time.time() + runs[-1] > t_end:
                break
    finally:
        os.sched_setaffinity(0, set(allowed))  # the all-core run's threads inherit this mask
    single = data.size / statistics.median(runs) / 1e9
    cores = all_core_threads(allowed)
    par_runs, par = [], None
    t_end = time.time() + max_seconds
    for _ in range(3):
        t0 = time.perf_counter()
        par = oracle.csv_parse_parallel(data, spec, cores) if kind == "csv" else \
            oracle.lex_restart_parallel(data, spec, cores)
        par_runs.append(time.perf_counter() - t0)
        if time.time() + par_runs[-1] > t_end:
            break
    keys = ("n_fields", "n_records", "error_pos", "end_state", "rec", "col", "off", "len") if kind == "csv" else \
        ("n_tokens", "kind", "start", "length")
    exact = all(np.array_equal(par[k], res[k]) for k in keys)
    return res, {"value": round(single, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
                 "sample": "the whole %d-byte input, sequential C oracle (gcc -O3), one thread pinned to core %d, "
                           "median of %d run(s)" % (data.size, pin, len(runs)),
                 "host": info}, {
        "value": round(data.size / statistics.median(par_runs) / 1e9, 3), "unit": "GB/s", "cores": cores,
        "kind": "all-core CPU baseline",
        "sample": "the whole input, the data-parallel method on %d host threads (per-slice state-transition "
                  "vectors, their serial composition, a tagging pass listing each slice's terminators, prefixes, "
                  "a parallel write; gcc -O3), median of %d run(s)" % (cores, len(par_runs)),
        "threads_rule": "the cores this process may run on (sched_getaffinity: %d), capped by OMP_NUM_THREADS "
                        "(%s)" % (len(allowed), os.environ.get("OMP_NUM_THREADS", "unset")),
        "host": info,
        "parity_vs_oracle": "bit-exact" if exact else "MISMATCH"}


def bandwidth_ceilings(ppr, torch, dev, nbytes=1 << 30, iters=10):
    """The device's own streaming rates (ppr_bandwidth_probe): read, write and
    copy of nbytes, wave-contiguous 16-byte words (pattern 0), 64 bytes per
    lane (pattern 1) and wave-contiguous 4-byte words (pattern 2, the field and
    token stores' shape), averaged over iters launches after 2 warm-ups."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src.fill_(3)
    props = torch.cuda.get_device_properties(dev)
    grid = props.multi_processor_count * 8
    stream = torch.cuda.current_stream()
    out = {"bytes": nbytes, "grid": grid, "block": 256}
    for pat, pname in ((0, "wave_contiguous_16B"), (1, "lane_contiguous_64B"), (2, "wave_contiguous_4B")):
        r = {}
        for mode, mname in ((0, "read"), (1, "write"), (2, "copy")):
            for _ in range(2):
                ppr.bandwidth_probe(mode, pat, src, dst, nbytes, grid)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(iters):
                ppr.bandwidth_probe(mode, pat, src, dst, nbytes, grid)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / iters
            moved = nbytes * (2 if mode == 2 else 1)
            r[mname] = {"us": round(ms * 1e3, 1), "GBps": round(moved / (ms * 1e-3) / 1e9, 1)}
        out[pname] = r
    del src, dst
    return out


def reread_probe(ppr, torch, dev, reps=3):
    """Read probe (pattern 0) over the first `size` bytes of a buffer, cold (after
    reading 1 GiB of other data) and warm (right after reading the same bytes):
    how much a re-read gains from the caches beyond the L2. Prints one JSON line."""
    big = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    other = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    big.fill_(1)
    other.fill_(2)
    sink = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    grid = torch.cuda.get_device_properties(dev).multi_processor_count * 8

    def read(buf, nbytes):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        ppr.bandwidth_probe(0, 0, buf, sink, nbytes, grid)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3

    out = {"probe": "reread", "grid": grid, "block": 256, "sizes": {}}
    for mib in (64, 128, 192, 256, 384, 512):
        nb = mib << 20
        cold, warm = [], []
        for _ in range(reps):
            read(other, 1 << 30)
            cold.append(read(big, nb))
            warm.append(read(big, nb))
        out["sizes"]["%dMiB" % mib] = {"cold_us": round(statistics.median(cold), 1),
                                       "warm_us": round(statistics.median(warm), 1)}
    print(json.dumps(out))


def overlap_probe(args, cfg_id, cfg, ppr, torch, W, np, reps=10):
    """Two parses of the workload with their own workspaces: back to back on one
    stream, and on two streams with the second started once the first's first
    stage (the codes kernel) is done, so that its memory-bound kernel runs beside
    the first's later kernels. Median ms of each, one JSON line."""
    dev = torch.device("cuda:0")
    data = W.generate(cfg_id)
    xa = torch.from_numpy(data).to(dev)
    xb = xa.clone()
    table = W.table(cfg["table"])
    n = data.size
    A = ppr.Parser(table, max_n=n, capacity=max(4096, n // 8), device=dev)
    B = ppr.Parser(table, max_n=n, capacity=max(4096, n // 8), device=dev)
    s1 = torch.cuda.current_stream()
    s2 = torch.cuda.Stream()
    ev = [torch.cuda.Event() for _ in range(8)]
    for e in ev:
        e.record(s1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run(mode):
        e0.record(s1)
        if mode == "one_stream":
            A.launch(xa, s1)
            B.launch(xb, s1)
        else:
            s2.wait_stream(s1)
            A.launch(xa, s1, stage_events=ev)
            s2.wait_event(ev[1])
            B.launch(xb, s2)
            s1.wait_stream(s2)
        e1.record(s1)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    out = {"probe": "overlap", "workload": cfg["name"], "n_bytes": n}
    for mode in ("one_stream", "two_streams"):
        for _ in range(3):
            run(mode)
        out[mode + "_ms"] = round(statistics.median([run(mode) for _ in range(reps)]), 4)
    print(json.dumps(out))


def stream_bench(args, cfg_id, cfg, ppr, torch, W, np):
    """host-to-host GB/s of ppr_parse_stream: the input in pinned host memory, the
    per-field results returned into pinned host arrays (64-bit offsets and
    lengths); wall clock around each call, median of the timed calls"""
    assert cfg["kind"] == "csv", "streaming covers the delimiter-separated parse"
    log("generating", cfg["name"], cfg["n"], "bytes")
    data = W.generate(cfg_id)
    host = torch.empty(data.size, dtype=torch.uint8, pin_memory=True)
    host.numpy()[:] = data
    table = W.table(cfg["table"])
    pb = args.stream << 20
    first = ppr.parse_stream(host, table, pb)
    for _ in range(args.warmup):
        ppr.parse_stream(host, table, pb, capacity=first.n_fields)
    times = []
    for _ in range(args.steps):
        t0 = time.perf_counter()
        g = ppr.parse_stream(host, table, pb, capacity=first.n_fields)
        times.append(time.perf_counter() - t0)
    assert g.n_fields == first.n_fields
    ms = statistics.median(times) * 1e3
    print(json.dumps({"metric": "host-to-host GB/s parsed with overlapped transfers (ppr_parse_stream)",
                      "value": round(data.size / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "ms_per_call": round(ms, 3),
                      "steps": args.steps, "warmup": args.warmup, "partition_bytes": pb,
                      "partitions": g.partitions, "fields": g.n_fields,
                      "config": {"workload": "%s_%dMiB" % (cfg["name"], data.size >> 20), "n_bytes": data.size},
                      "timing": "host wall clock around each blocking call (allocation of the driver's device "
                                "buffers included), median"}), flush=True)


COLUMN_STAGES = ["cols_reset_kernel", "cols_hist_kernel", "cols_scan_kernel#counts", "cols_scan_kernel#bytes",
                 "cols_part_kernel", "cols_bounds_kernel"]


def columns_bench(args, cfg_id, cfg, ppr, torch, W, np):
    """GB/s of the columnar partition (ppr_columns) of the workload's parse: the
    parse's field arrays and the bytes resident in HBM, one blocking call per
    step (every kernel: histogram, scans, scatter, bounds, byte copy)"""
    import oracle
    assert cfg["kind"] == "csv", "the columnar partition follows a delimiter-separated parse"
    mode = {"indexed": ppr.PPR_CSS_INDEXED, "inline": ppr.PPR_CSS_INLINE, "vector": ppr.PPR_CSS_VECTOR}[args.columns]
    log("generating", cfg["name"], cfg["n"], "bytes")
    data = W.generate(cfg_id)
    sha = W.sha256(data)
    n = data.size
    dev = torch.device("cuda:0")
    d = torch.from_numpy(data).to(dev)
    table = W.table(cfg["table"])
    g = ppr.Parser(table, max_n=n, capacity=n // 8 + 4096, device=dev)(d)
    nf, nc = g.n_fields, g.max_columns
    cols = ppr.Columns(nf, nc, n, mode=mode, terminator=0x1E)
    first = cols(d, g)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        cols(d, g)
    torch.cuda.synchronize()
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for a, b in step_ev:
        a.record(stream)
        cols(d, g)
        b.record(stream)
    torch.cuda.synchronize()
    ms = statistics.median(a.elapsed_time(b) for a, b in step_ev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(COLUMN_STAGES) + 1)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    for row in evs:
        cols(d, g, stage_events=row)
    torch.cuda.synchronize()
    stage_ms = {k: statistics.mean(row[i].elapsed_time(row[i + 1]) for row in evs) for i, k in enumerate(COLUMN_STAGES)}
    slot = 0 if mode == ppr.PPR_CSS_INDEXED else 1
    css = first.css_bytes
    field_bytes = css - slot * nf  # the fields' own bytes, read once from the input
    aux = css if mode == ppr.PPR_CSS_VECTOR else 0
    # algorithmic bytes, each attributed to the kernel that moves it: the four field arrays read once (16 B per
    # field: the histogram reads columns and lengths, the partition kernel the rest), the index written once (12 B per
    # field), the field bytes read once and the CSS (and aux) written once (all three by the partition kernel),
    # the bounds (8 B per column)
    alg = {"cols_hist_kernel": 8 * nf, "cols_part_kernel": 8 * nf + 12 * nf + field_bytes + css + aux,
           "cols_bounds_kernel": 8 * (nc + 1)}
    step_alg = 16 * nf + 12 * nf + field_bytes + css + aux + 8 * (nc + 1)
    dominant = max(stage_ms, key=stage_ms.get)
    t_dom = stage_ms[dominant] * 1e-3
    alg_dom = alg.get(dominant, 0)
    line = {"metric": "columnar partition GB/s (input bytes of the parse partitioned per second, ppr_columns)",
            "value": round(n / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": "%s_%dMiB_columns_%s" % (cfg["name"], n >> 20, args.columns), "n_bytes": n,
                       "fields": nf, "columns": nc, "css_bytes": css, "input_sha256": sha[:16],
                       "kernels": COLUMN_STAGES},
            "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(alg_dom / t_dom / 1e9, 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(alg_dom / t_dom / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                         "algorithmic_bytes_per_launch": alg_dom, "kernel_ms": round(stage_ms[dominant], 4),
                         "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
                         "step": {"algorithmic_bytes": step_alg,
                                  "achieved": round(step_alg / (ms * 1e-3) / 1e9, 2),
                                  "frac": round(step_alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
                         "timing": "HIP events on the launch stream around each of %d blocking calls (median); "
                                   "per-kernel events recorded by the library" % args.steps}}
    if not args.no_cpu:
        from oracle import columns as C
        log("cpu oracle baseline (columns)")
        r = oracle.csv_parse(data, table)
        # the oracle as it stands (a Python loop per field) on a bounded sample: the first records' fields
        info, allowed = host_cpu()
        k = min(nf, 3 << 20)
        end = int(r["off"][k - 1] + r["len"][k - 1]) + 1
        t0 = time.perf_counter()
        C.partition(data[:end], r["rec"][:k], r["col"][:k], r["off"][:k], r["len"][:k], mode, 0x1E)
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(end / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                                "sample": "the first %d fields (%d input bytes) of the same parse, oracle partition "
                                          "(numpy stable argsort, then a Python loop per field), one run" % (k, end),
                                "host": info}
        # parity at full size: counts and bounds exactly, every index entry against the oracle parse's fields in
        # stable column order, and 2000 sampled CSS fields byte for byte
        col = r["col"].astype(np.int64)
        order = np.argsort(col, kind="stable")
        lens = r["len"].astype(np.int64)[order]
        offs = np.concatenate([[0], np.cumsum(lens + slot)])
        u32 = lambda t: t.cpu().numpy().view(np.uint32).astype(np.int64)  # noqa: E731
        res = cols(d, g)
        ok = res.css_bytes == int(offs[-1]) and nf == r["n_fields"]
        ok = ok and np.array_equal(u32(res.rec), r["rec"].astype(np.int64)[order])
        ok = ok and np.array_equal(u32(res.length), lens) and np.array_equal(u32(res.css_off), offs[:-1])
        ok = ok and np.array_equal(u32(res.col_first_field),
                                   np.concatenate([[0], np.cumsum(np.bincount(col, minlength=nc))]))
        rng = np.random.default_rng(3)
        css_h = res.css
        for j in rng.integers(0, nf, 2000):
            f = order[j]
            seg = css_h[offs[j]:offs[j] + lens[j]].cpu().numpy().tobytes()
            ok = ok and seg == data[r["off"][f]:r["off"][f] + r["len"][f]].tobytes()
        line["parity_vs_oracle"] = ("bit-exact (index, bounds, CSS size; 2000 sampled CSS fields)" if ok
                                    else "MISMATCH")
    print(json.dumps(line), flush=True)


def numbers_bench(args, cfg_id, cfg, ppr, torch, W, np):
    """GB/s of numeric type inference plus conversion (ppr_infer_types, then
    ppr_convert to the inferred types) over a workload's parse: the input and
    the parse's field arrays resident in HBM, one blocking call of each per
    step"""
    import oracle
    from oracle import numbers as N
    assert cfg["kind"] == "csv", "numbers follow a delimiter-separated parse"
    log("generating", cfg["name"], cfg["n"], "bytes")
    data = W.generate(cfg_id)
    sha = W.sha256(data)
    n = data.size
    dev = torch.device("cuda:0")
    d = torch.from_numpy(data).to(dev)
    table = W.table(cfg["table"])
    g = ppr.Parser(table, max_n=n, capacity=n // 4 + 4096, device=dev)(d)
    F = ppr.Fields.of_parse(d, g)
    nf = g.n_fields
    types, _ = ppr.infer_types(F)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        ppr.infer_types(F)
        ppr.convert(F, types)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for a, b, c in ev:
        a.record(stream)
        ppr.infer_types(F)
        b.record(stream)
        cv = ppr.convert(F, types)
        c.record(stream)
    torch.cuda.synchronize()
    t_inf = [a.elapsed_time(b) for a, b, _ in ev]
    t_cnv = [b.elapsed_time(c) for _, b, c in ev]
    ms = statistics.median([x + y for x, y in zip(t_inf, t_cnv)])
    field_bytes = int(g.field_lengths.to(torch.int64).sum().item())
    # algorithmic bytes: each call reads the field arrays it needs (offset, length, column: 12 B per field) and the
    # fields' bytes; conversion writes 9 B per field (value and status)
    alg = {"num_kernel<infer>": 12 * nf + field_bytes, "num_kernel<convert>": 12 * nf + field_bytes + 9 * nf}
    stage_ms = {"num_kernel<infer>": statistics.mean(t_inf), "num_kernel<convert>": statistics.mean(t_cnv)}
    dominant = max(stage_ms, key=stage_ms.get)
    t_dom = stage_ms[dominant] * 1e-3
    step_alg = sum(alg.values())
    line = {"metric": "numeric type inference + conversion GB/s (input bytes of the parse per second)",
            "value": round(n / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": "%s_%dMiB_numbers" % (cfg["name"], n >> 20), "n_bytes": n, "fields": nf,
                       "columns": int(types.size), "column_types": [N.TYPE_NAMES[int(t)] for t in types],
                       "input_sha256": sha[:16], "kernels": list(alg)},
            "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(alg[dominant] / t_dom / 1e9, 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(alg[dominant] / t_dom / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                         "algorithmic_bytes_per_launch": alg[dominant], "kernel_ms": round(stage_ms[dominant], 4),
                         "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
                         "step": {"algorithmic_bytes": step_alg, "achieved": round(step_alg / (ms * 1e-3) / 1e9, 2),
                                  "frac": round(step_alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
                         "statuses": {"defaulted": int(cv.counts[0]), "mismatch": int(cv.counts[1]),
                                      "inexact": int(cv.counts[2]), "not_converted": int(cv.counts[3])},
                         "timing": "HIP events on the launch stream around each blocking call (a reset kernel and "
                                   "the main kernel each), median of %d steps" % args.steps}}
    if not args.no_cpu:
        log("cpu oracle baseline (numbers)")
        info, _ = host_cpu()
        k = min(nf, 1 << 20)
        off = g.field_offsets[:k].cpu().numpy().view(np.uint32).astype(np.int64)
        ln = g.field_lengths[:k].cpu().numpy().view(np.uint32).astype(np.int64)
        r = oracle.csv_parse(data[:int(off[-1] + ln[-1]) + 1], table)
        t0 = time.perf_counter()
        oft, _ = N.infer(data, r["off"][:k], r["len"][:k], r["col"][:k], int(types.size))
        ov, ost = N.convert(data, r["off"][:k], r["len"][:k], r["col"][:k], types, 0, 0.0)
        dt = time.perf_counter() - t0
        span = int(r["off"][k - 1] + r["len"][k - 1])
        line["cpu_baseline"] = {"value": round(span / dt / 1e9, 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
                                "sample": "the first %d fields (%d input bytes), oracle inference and conversion "
                                          "(Python regular expressions, int(), float()), one run" % (k, span),
                                "host": info}
        _, ft = ppr.infer_types(F, field_types=True)
        ok = np.array_equal(ft[:k].cpu().numpy(), oft)
        ok = ok and np.array_equal(cv.status[:k].cpu().numpy(), ost)
        ok = ok and np.array_equal(cv.values[:k].cpu().numpy(), ov)
        line["parity_vs_oracle"] = ("bit-exact (types, values, statuses) on the first %d fields" % k if ok
                                    else "MISMATCH")
    print(json.dumps(line), flush=True)


def read_pmc(d, counter):
    """counter value of every dispatch, by kernel name, from a rocprofv3 csv output directory"""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under " + d)
    per_dispatch = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
            per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    by_kernel = {}
    for (name, _), v in per_dispatch.items():
        by_kernel.setdefault(name, []).append(v)
    return by_kernel


def short_name(kernel_name):
    for names in STAGES.values():
        for s in names:
            if s + "<" in kernel_name or s + "(" in kernel_name:
                return s
    return None


def summarize_pmc(args, chunk):
    fetch = read_pmc(args.summarize_pmc[0], "FETCH_SIZE")
    write = read_pmc(args.summarize_pmc[1], "WRITE_SIZE")

    def copies(by_kernel):  # the largest single dispatch of a copy kernel: the 1 GiB calibration copy
        v = [x for k, xs in by_kernel.items() if "ppr" not in k and "copy" in k.lower() for x in xs]
        return max(v) if v else None

    copy_f, copy_w = copies(fetch), copies(write)
    if not copy_f or not copy_w:
        raise SystemExit("no copy kernel in the counter output (run the parse with --copy-calibration)")
    fetch = {k: statistics.median(v) for k, v in fetch.items()}
    write = {k: statistics.median(v) for k, v in write.items()}
    # the copy kernel moves COPY_BYTES in each direction; the counters read in KiB
    f_scale = COPY_BYTES / (copy_f * 1024.0)
    w_scale = COPY_BYTES / (copy_w * 1024.0)
    kernels = {}
    for k in set(fetch) | set(write):
        s = short_name(k)
        if s is None:
            continue
        fb = fetch.get(k, 0.0) * 1024.0 * f_scale
        wb = write.get(k, 0.0) * 1024.0 * w_scale
        kernels[s] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "hbm_bytes": round(fb + wb),
                      "fetch_kib_raw": round(fetch.get(k, 0.0), 1), "write_kib_raw": round(write.get(k, 0.0), 1),
                      "source_sha": source_sha(s)}
    out = {"workload": args.workload, "chunk_bytes": chunk, "source_sha": source_sha(),
           "copy_calibration": {"bytes_each_way": COPY_BYTES, "fetch_kib_raw": round(copy_f, 1),
                                "write_kib_raw": round(copy_w, 1), "fetch_scale": round(f_scale, 4),
                                "write_scale": round(w_scale, 4)},
           "kernels": kernels,
           "commands": ["rocprofv3 --pmc %s -d %s -o run --output-format csv -- python3 bench.py --workload %s "
                        "--chunk %d --no-cpu --no-probe --steps 3 --warmup 1 --copy-calibration" % (c, d, args.workload, chunk)
                        for c, d in zip(("FETCH_SIZE", "WRITE_SIZE"), args.summarize_pmc)]
                       + ["python bench.py --workload %s --chunk %d --summarize-pmc %s %s" % (
                           args.workload, chunk, *args.summarize_pmc)]}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    path = counters_path(args.workload, chunk)
    json.dump(out, open(path, "w"), indent=1, sort_keys=True)
    print(json.dumps(out))
    log("wrote", path)


def measured_traffic(workload, chunk, stage):
    """HBM bytes per launch of one kernel from the committed counter summary,
    if it was taken on the current kernel sources (else None)."""
    path = counters_path(workload, chunk)
    if not os.path.exists(path):
        return None
    c = json.load(open(path))
    k = c.get("kernels", {}).get(stage)
    if k is None or k.get("source_sha", c.get("source_sha")) != source_sha(stage):
        return None
    return k["hbm_bytes"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="csv3", choices=sorted(WORKLOADS))
    ap.add_argument("--chunk", type=int, default=None, help="bytes per thread (default: the library's, 64)")
    ap.add_argument("--path", choices=["auto", "fused", "streaming", "single-pass"], default="auto",
                    help="parse kernels to ask the library for (default: its automatic choice)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline and the full-size parity check")
    ap.add_argument("--stream", type=int, default=0, metavar="PARTITION_MIB",
                    help="instead: time ppr_parse_stream over the workload in pinned HOST memory, partitions of this "
                         "many MiB (transfers, parse and returns overlapped; PCIe-inclusive, not the metric)")
    ap.add_argument("--columns", choices=["indexed", "inline", "vector"], default=None,
                    help="instead: time the columnar partition (ppr_columns) of the workload's parse in this mode")
    ap.add_argument("--numbers", action="store_true",
                    help="instead: time numeric type inference and conversion over the workload's parse")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the device bandwidth probe (read / write / copy of 1 GiB)")
    ap.add_argument("--overlap-probe", action="store_true",
                    help="instead: two parses back to back against two streams, the second after the first's codes kernel")
    ap.add_argument("--reread-probe", action="store_true",
                    help="instead: time the read probe over 64-512 MiB cold and right after a read of the same bytes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/hbm_counters_<workload>_chunk<L>.json from two rocprofv3 --pmc runs")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    chunk = args.chunk or (40 if args.workload == "lex5" else 64)  # the library's defaults
    if args.summarize_pmc:
        summarize_pmc(args, chunk)
        return

    import numpy as np
    import torch

    import dfa_parsing_delimiter_amd as ppr
    import workloads as W

    cfg_id = WORKLOADS[args.workload]
    cfg = W.CONFIGS[cfg_id]
    kind = "csv" if cfg["kind"] == "csv" else "lex"
    dev = torch.device("cuda:0")
    if args.reread_probe:
        return reread_probe(ppr, torch, dev)
    if args.overlap_probe:
        return overlap_probe(args, cfg_id, cfg, ppr, torch, W, np)
    if args.stream:
        return stream_bench(args, cfg_id, cfg, ppr, torch, W, np)
    if args.columns:
        return columns_bench(args, cfg_id, cfg, ppr, torch, W, np)
    if args.numbers:
        return numbers_bench(args, cfg_id, cfg, ppr, torch, W, np)
    log("generating", cfg["name"], cfg["n"], "bytes")
    t0 = time.time()
    data = W.generate(cfg_id)
    sha = W.sha256(data)
    log("generated in %.1fs sha256 %s" % (time.time() - t0, sha[:16]))
    d = torch.from_numpy(data).to(dev)
    n = data.size

    if kind == "csv":
        table = W.table(cfg["table"])
        want = {"auto": None, "fused": ppr.PPR_PATH_FUSED, "streaming": ppr.PPR_PATH_STREAMING,
                "single-pass": ppr.PPR_PATH_SINGLE_PASS}[args.path]
        runner = ppr.Parser(table, max_n=n, capacity=max(4096, n // 8), chunk_bytes=chunk, device=dev, path=want)
        first = runner(d)
        runner._alloc(first.n_fields)
        n_out, path = first.n_fields, first.path
        stages = STAGES[path]
        out_bytes_per_item = 16
        spec = table
    else:
        dfa = W.lexer_dfa()
        tabs = ppr.LexTables.from_dfa(dfa, dev)
        want = {"auto": None, "fused": ppr.PPR_PATH_STREAMING, "streaming": ppr.PPR_PATH_STREAMING,
                "single-pass": ppr.PPR_PATH_SINGLE_PASS}[args.path]
        runner = ppr.Lexer(tabs, max_n=n, capacity=max(4096, n // 3), chunk_bytes=args.chunk, path=want)
        first = runner(d)
        runner._alloc(first.n_tokens)
        n_out, path = first.n_tokens, first.path
        stages = STAGES["lex%d" % path]
        out_bytes_per_item = 12
        spec = dfa
    log("first call: %d items, kernels %s" % (n_out, stages))
    stream = torch.cuda.current_stream()

    def step():  # one blocking call: enqueue every kernel, read the scalars back
        runner.launch(d)
        return runner.results(n)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # (1) the metric: K blocking calls, each bracketed by events on the stream;
    # ms_per_step is their median
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for a, b in step_ev:
        a.record(stream)
        o = step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    step_ms = [a.elapsed_time(b) for a, b in step_ev]
    ms = statistics.median(step_ms)
    ms_mean = statistics.mean(step_ms)
    got = int(o.n_fields if kind == "csv" else o.n_tokens)
    assert got == n_out, (got, n_out)

    # (2) per-kernel durations: K back-to-back calls with the library recording
    # an event before, between and after its kernels on the launch stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record(stream)  # creates the events
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for row in evs:
        runner.launch(d, stage_events=row)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_pipelined = e0.elapsed_time(e1) / args.steps
    stage_ms = {s: statistics.mean(row[i].elapsed_time(row[i + 1]) for row in evs) for i, s in enumerate(stages)}
    dominant = max(stage_ms, key=stage_ms.get)
    t_dom = stage_ms[dominant] * 1e-3

    gbs = n / (ms * 1e-3) / 1e9
    alg_dom = algorithmic_bytes(dominant, n, n_out, out_bytes_per_item)
    alg_step = n + out_bytes_per_item * n_out
    traffic = measured_traffic(args.workload, chunk, dominant)
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
                   "input_sha256": sha[:16], "kernels": stages},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(alg_dom / t_dom / 1e9, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(alg_dom / t_dom / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic / t_dom / 1e9, 2),
                     "traffic_bytes_per_launch": traffic,
                     "algorithmic_bytes_per_launch": alg_dom, "kernel_ms": round(stage_ms[dominant], 4),
                     "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
                     "step": {"algorithmic_bytes": alg_step,
                              "achieved": round(alg_step / (ms * 1e-3) / 1e9, 2),
                              "frac": round(alg_step / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
                     "ms_per_step_pipelined": round(ms_pipelined, 4),
                     "ms_per_step_mean": round(ms_mean, 4),
                     "ms_per_step_min_max": [round(min(step_ms), 4), round(max(step_ms), 4)],
                     "timing": "HIP events on the launch stream around each of %d blocking calls (median; wall "
                               "%.3fs); per-kernel events recorded by the library over %d pipelined calls" % (
                                   args.steps, wall, args.steps)},
    }
    if not args.no_probe:
        line["bandwidth_ceilings"] = bandwidth_ceilings(ppr, torch, dev)
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(5):
            dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize()
        cms = c0.elapsed_time(c1) / 5
        line["copy_calibration"] = {"bytes_each_way": COPY_BYTES, "ms": round(cms, 4),
                                    "GBps_read_plus_write": round(2 * COPY_BYTES / (cms * 1e-3) / 1e9, 1)}
        del src, dst
    if not args.no_cpu:
        log("cpu oracle baseline")
        ref, single, allcore = cpu_oracle_baseline(kind, data, spec)
        line["cpu_baseline"] = single
        line["cpu_baseline_all_threads"] = allcore
        # bit-exact check of the timed configuration against the oracle, every output array
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
