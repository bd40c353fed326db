"""GPU parity: ppr_parse (HIP path, through the C ABI) against the CPU oracle.

Bit-exact on every output array and scalar. Covers hand-worked and exhaustive
short inputs, chunk sizes from 1 byte (every byte its own chunk, so the scans do
all the work) to 64, inputs spanning several tiles with ragged tails, unaligned
input pointers, error and capacity paths, and every delimiter-separated
workload at its full size in the configuration the benchmark times. Every
64-byte case runs on both table-driven paths (the streaming kernels, the
automatic choice, and the fused single-pass kernel).
"""
import itertools
import json
import os
import sys

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "csv_examples.jsonl")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ppr():
    import torch
    assert torch.cuda.is_available()
    import dfa_parsing_delimiter_amd as m
    return m


def _dev(b):
    import torch
    arr = np.frombuffer(bytes(b), dtype=np.uint8) if not isinstance(b, np.ndarray) else b
    return torch.from_numpy(np.array(arr, dtype=np.uint8, copy=True)).to("cuda")


def _np(t):
    return t.cpu().numpy().view(np.uint32)


def _same(g, r, what=""):
    assert g.n_fields == r["n_fields"], (what, g.n_fields, r["n_fields"])
    assert g.n_records == r["n_records"], (what, g.n_records, r["n_records"])
    assert g.error_pos == r["error_pos"], (what, g.error_pos, r["error_pos"])
    assert g.end_state == r["end_state"], (what, g.end_state, r["end_state"])
    assert (g.min_columns, g.max_columns) == (r["min_columns"], r["max_columns"]), (
        what, g.min_columns, g.max_columns, r["min_columns"], r["max_columns"])
    assert (g.bad_records, g.first_bad_record) == (r["bad_records"], r["first_bad_record"]), (
        what, g.bad_records, g.first_bad_record, r["bad_records"], r["first_bad_record"])
    for name, key in (("record_idx", "rec"), ("column_ids", "col"), ("field_offsets", "off"),
                      ("field_lengths", "len")):
        a = _np(getattr(g, name))
        if not np.array_equal(a, r[key]):
            bad = np.nonzero(a != r[key])[0]
            raise AssertionError("%s %s differs at %d of %d (first %d: gpu %d oracle %d)" % (
                what, name, bad.size, a.size, bad[0], a[bad[0]], r[key][bad[0]]))


# (chunk_bytes, path) pairs: 64-byte chunks on each table-driven path (None: the automatic choice;
# 1: the streaming kernels; 3: the fused kernel)
STREAMING = 1
FUSED = 3
SINGLE_PASS = 2
FUSED_MAX_AUTO = 8 << 20  # the automatic choice: the fused kernel up to this many bytes, streaming above


def auto_path(n):
    return FUSED if n <= FUSED_MAX_AUTO else STREAMING


def _with_paths(chunks):
    out = []
    for c in chunks:
        out += [(c, None), (c, STREAMING), (c, FUSED)] if c in (None, 64) else [(c, None)]
    return out


def test_golden(ppr):
    for line in open(GOLDEN):
        c = json.loads(line)
        t = W.table(c["table"])
        b = c["input"].encode("latin-1")
        for chunk, path in _with_paths((1, 2, 3, 32, 64)):
            _say("golden", repr(b), chunk, path)
            g = ppr.parse(_dev(b), t, chunk_bytes=chunk, capacity=len(b) + 1, path=path)
            _same(g, oracle.csv_parse(b, t), (b, chunk, path))


@pytest.mark.parametrize("name,alphabet,max_len", [("T5", b',\n"a', 5), ("T6", b'\t\n"#a', 4)])
def test_exhaustive_short(ppr, name, alphabet, max_len):
    t = W.table(name)
    inputs = [bytes(s) for L in range(1, max_len + 1) for s in itertools.product(alphabet, repeat=L)]
    refs = oracle.csv_parse_many(inputs, t)
    _say("exhaustive", name, len(inputs))
    parsers = {cp: ppr.Parser(t, max_n=16, chunk_bytes=cp[0], path=cp[1]) for cp in _with_paths((1, 3, 64))}
    for s, r in zip(inputs, refs):
        for c, P in parsers.items():
            _same(P(_dev(s)), r, (s, c))


@pytest.mark.parametrize("chunk,path", _with_paths([1, 2, 5, 16, 31, 32, 33, 63, 64]))
def test_random_mixed_inputs_every_chunk_size(ppr, chunk, path):
    rng = np.random.default_rng(chunk)
    for name in ("T5", "T6"):
        t = W.table(name)
        alpha = np.frombuffer(b',\n"ab' if name == "T5" else b'\t\n"#ab', dtype=np.uint8)
        P = ppr.Parser(t, max_n=70000, chunk_bytes=chunk, path=path)
        for it in range(12):
            n = int(rng.integers(0, 70000))
            # mostly valid text with rare quotes, so that errors do not end everything early
            p = np.array([0.08, 0.05, 0.01, 0.43, 0.43] if name == "T5" else [0.08, 0.04, 0.01, 0.01, 0.43, 0.43])
            b = alpha[rng.choice(alpha.size, n, p=p / p.sum())]
            _say("random", name, chunk, n)
            _same(P(_dev(b)), oracle.csv_parse(b, t), (name, chunk, n))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
@pytest.mark.parametrize("chunk,path", _with_paths([1, 8, 31, 32, 64]))
def test_workloads_several_tiles_ragged(ppr, cfg, chunk, path):
    t = W.table(W.CONFIGS[cfg]["table"])
    n = (3 << 20) + 12345
    b = W.generate(cfg, n=n, seed=77 + cfg)
    # checked against the workload's number of columns: comment lines and the unterminated final record differ
    expect = W.CONFIGS[cfg]["n_cols"]
    _say("workload", cfg, chunk, path, n)
    g = ppr.parse(_dev(b), t, chunk_bytes=chunk, capacity=n + 1, path=path, expected_columns=expect)
    _same(g, oracle.csv_parse(b, t, expected_columns=expect), (cfg, chunk, path))


def _random_table(rng, absorbing, n_special):
    S = int(rng.integers(1, 9))
    C = int(rng.integers(1, 17))
    nxt = rng.integers(0, S, (S, C)).tolist()
    tag = rng.integers(0, 4, (S, C)).tolist()
    # mostly value/terminator tags so that inputs stay valid for a while
    for s_ in range(S):
        for c in range(C):
            if tag[s_][c] == 3 and rng.random() < 0.8:
                tag[s_][c] = int(rng.integers(0, 3))
    if absorbing and S > 1:
        a = int(rng.integers(0, S))
        nxt[a] = [a] * C
        tag[a] = [3] * C
    K = int(rng.integers(0, C))
    cm = bytearray([K] * 256)
    others = [c for c in range(C) if c != K]
    if others:
        for b in rng.choice(256, size=min(n_special, 256), replace=False):
            cm[int(b)] = int(rng.choice(others))
    return {"name": "rand", "n_states": S, "n_classes": C, "next": nxt, "tag": tag, "start": int(rng.integers(0, S)),
            "accept_mask": int(rng.integers(0, 1 << S)), "class_map": bytes(cm)}


@pytest.mark.parametrize("seed", range(12))
def test_random_tables(ppr, seed):
    """random DFAs: every fast-path variant (symbol code widths 2/3/4, 4- and 8-entry
    vectors, with and without an absorbing state) and the generic fallback (many
    special bytes), against the oracle"""
    rng = np.random.default_rng(1000 + seed)
    for trial in range(6):
        t = _random_table(rng, absorbing=bool(trial % 2), n_special=int(rng.choice([1, 3, 8, 8, 20])))
        specials = [b for b in range(256) if t["class_map"][b] != max(set(t["class_map"]), key=t["class_map"].count)]
        pool = np.array(specials + [ord("a"), ord("b"), ord("z")], dtype=np.uint8)
        for n in (1, 63, 64, 65, 16384, 16385, 100000):
            b = pool[rng.integers(0, pool.size, n)]
            r = oracle.csv_parse(b, t)
            for chunk, path in _with_paths((64, 13)):
                _say("table", seed, trial, t["n_states"], t["n_classes"], len(specials), n, chunk, path)
                g = ppr.parse(_dev(b), t, chunk_bytes=chunk, capacity=n + 1, path=path)
                _same(g, r, (seed, trial, n, chunk, path))


def _full_range_csv(rng, n, sep, quote=ord('"')):
    """records of unquoted fields (any byte but the specials) and quoted fields
    (any byte but the quote, doubled quotes, separators and newlines inside)"""
    specials = {sep, 10, quote}
    plain = np.array([b for b in range(256) if b not in specials], dtype=np.uint8)
    inner = np.array([b for b in range(256) if b != quote], dtype=np.uint8)
    out = bytearray()
    while len(out) < n:
        for f in range(int(rng.integers(1, 6))):
            if f:
                out.append(sep)
            L = int(rng.integers(0, 40))
            if rng.random() < 0.4:
                body = bytearray(inner[rng.integers(0, inner.size, L)].tobytes())
                for i in sorted(rng.integers(0, L + 1, int(rng.integers(0, 3))).tolist(), reverse=True):
                    body[i:i] = bytes([quote, quote])
                out += bytes([quote]) + body + bytes([quote])
            else:
                out += plain[rng.integers(0, plain.size, L)].tobytes()
        out.append(10)
    return np.frombuffer(bytes(out[:n]), dtype=np.uint8)


@pytest.mark.parametrize("seed", range(4))
def test_every_byte_value(ppr, seed):
    """every byte value at every position in a word, in unquoted and quoted
    fields, for T5 and T6 and for random tables whose special bytes are anywhere
    in 0..255 (the table-driven paths tell a special byte from all the others by
    a slot of a few bits and an exact compare)"""
    rng = np.random.default_rng(500 + seed)
    cases = [(W.table("T5"), _full_range_csv(rng, 200003, ord(","))),
             (W.table("T6"), _full_range_csv(rng, 200003, 9))]
    for trial in range(4):
        t = _random_table(rng, absorbing=bool(trial % 2), n_special=int(rng.choice([1, 3, 5, 8])))
        K = max(set(t["class_map"]), key=t["class_map"].count)
        specials = np.array([b for b in range(256) if t["class_map"][b] != K], dtype=np.uint8)
        b = rng.integers(0, 256, 150001).astype(np.uint8)
        if specials.size:
            pick = rng.random(b.size) < 0.3
            b[pick] = specials[rng.integers(0, specials.size, int(pick.sum()))]
        cases.append((t, b))
    for i, (t, b) in enumerate(cases):
        r = oracle.csv_parse(b, t)
        for chunk, path in _with_paths((64, 13)):
            _say("every byte", seed, i, b.size, chunk, path)
            g = ppr.parse(_dev(b), t, chunk_bytes=chunk, capacity=b.size + 1, path=path)
            _same(g, r, (seed, i, chunk, path))


def test_unaligned_input_and_subviews(ppr):
    import torch
    t = W.table("T5")
    b = W.generate(3, n=1 << 20, seed=5)
    d = _dev(b)
    for off in (1, 3, 7, 15, 16):
        _say("unaligned", off)
        view = d[off:]
        g = ppr.parse(view, t, capacity=b.size)
        _same(g, oracle.csv_parse(b[off:], t), off)
        assert g.path == (auto_path(b.size - off) if off == 16 else ppr.PPR_PATH_SINGLE_PASS)


def test_edge_cases(ppr):
    t5, t6 = W.table("T5"), W.table("T6")
    cases = [
        (t5, b""), (t5, b","), (t5, b"\n"), (t5, b'"'), (t5, b"x"),
        (t5, b"," * 100000), (t5, b"\n" * 100001), (t5, b"a" * 300000),
        (t5, b'"' + b"a,\n" * 70000),            # one quoted field left open: error at n
        (t5, b'a"' + b"b" * 90000),              # invalid at byte 1, the rest one field
        (t5, (b'"x""y",' * 9000) + b'"z'),
        (t6, b"#" + b"\t\"" * 50000 + b"\n"),     # one long comment record
        (t6, b"\t" * 70000), (t6, b"\n#\n#x\n"),
    ]
    for t, b in cases:
        for chunk, path in _with_paths((1, 7, 31, 64)):
            _say("edge", t["name"], len(b), chunk, path)
            g = ppr.parse(_dev(b) if b else _dev(b"\0")[:0], t, chunk_bytes=chunk, capacity=len(b) + 2, path=path)
            _same(g, oracle.csv_parse(b, t), (t["name"], len(b), chunk, path))


def test_column_counts_at_scale(ppr):
    """records of 1 to 40 fields (some quoted, with embedded delimiters) over many tiles and ranges: the fewest
    and most fields per record on every path, with the narrowest and widest records placed deep inside; and a
    conforming input (every record 7 fields)"""
    t = W.table("T5")
    rng = np.random.default_rng(31)
    recs = []
    for i in range(300000):
        k = int(rng.integers(2, 39)) if i not in (123457, 200001) else (1 if i == 123457 else 40)
        recs.append(b",".join(b'"a,\nb"' if rng.random() < 0.1 else b"x" * int(rng.integers(0, 6)) for _ in range(k)))
    wide = b"\n".join(recs)  # no trailing newline: the final record is unterminated
    conform = b"\n".join(b",".join(b"%d" % (i * 7 + j) for j in range(7)) for i in range(200000)) + b"\n"
    for what, b in (("varied", wide), ("conforming", conform)):
        for expect in (0, 7, 40):
            r = oracle.csv_parse(b, t, expected_columns=expect)
            assert (what != "varied") or (r["min_columns"], r["max_columns"]) == (1, 40)
            assert (what != "conforming") or (r["min_columns"], r["max_columns"]) == (7, 7)
            assert (what != "conforming" or expect != 7) or r["bad_records"] == 0
            assert (what != "varied" or expect != 40) or r["first_bad_record"] == 0
            for chunk, path in ((None, None), (64, STREAMING), (64, FUSED), (31, None)):
                _say("columns", what, len(b), expect, chunk, path)
                g = ppr.parse(_dev(b), t, chunk_bytes=chunk, capacity=r["n_fields"] + 1, path=path,
                              expected_columns=expect)
                _same(g, r, (what, expect, chunk, path))


def test_invalid_bytes_at_scale(ppr):
    """the first INVALID byte over many tiles and ranges: at byte 1 of 12 MiB (every later byte stays in the
    absorbing state, so every chunk after it holds INVALID bytes), deep inside the input (one bad byte after
    9 MiB of valid CSV), and in the last tile"""
    t = W.table("T5")
    body = W.generate(3, n=12 << 20, seed=21)
    deep = body.copy()
    q = 9 * (1 << 20) + 12345
    deep[q:q + 3] = np.frombuffer(b'x"y', np.uint8)  # a quote inside an unquoted field, then a non-delimiter
    late = np.concatenate([body[: (12 << 20) - 40], np.frombuffer(b'1,2\n"a"b' + b"c" * 31, np.uint8)])
    cases = [("at byte 1", np.concatenate([np.frombuffer(b'a"', np.uint8), body])), ("deep", deep),
             ("last tile", late)]
    for what, b in cases:
        r = oracle.csv_parse(b, t)
        assert 0 <= r["error_pos"] < b.size, (what, r["error_pos"])
        for chunk, path in ((None, None), (64, STREAMING), (64, FUSED), (31, None)):
            _say("invalid", what, b.size, chunk, path, r["error_pos"])
            g = ppr.parse(_dev(b), t, chunk_bytes=chunk, capacity=r["n_fields"] + 1, path=path)
            _same(g, r, (what, chunk, path))


def test_late_agreement_and_dead_paths(ppr):
    """quoted fields of 1-6 KiB: tiles that start inside one agree on their start state only kilobytes in (the
    streaming kernels then run pass 2 over every span of such a tile), among tiles that agree early; and the
    same input with bytes that end the true path (a quote inside an unquoted field) while the other hypotheses
    live on, in the middle of tiles, so that a tile's agreed state is not its true one; 256 MiB, so that each
    range of the streaming kernels holds several tiles"""
    t = W.table("T5")
    b = W.long_field_csv(256 << 20, 7)
    bad = b.copy()
    for q in (100 << 20) + np.arange(5) * 700001:
        bad[q:q + 3] = np.frombuffer(b'x"y', np.uint8)
    for what, x in (("long fields", b), ("dead paths", bad)):
        r = oracle.csv_parse(x, t)
        for path in (None, FUSED):
            _say("late agreement", what, x.size, path, r["n_fields"], r["error_pos"])
            g = ppr.parse(_dev(x), t, capacity=r["n_fields"] + 1, path=path)
            assert g.path == (path or auto_path(x.size))
            _same(g, r, (what, path))


def test_absorbing_state_that_ends_fields(ppr):
    """T5 with its absorbing state tagging field and record delimiters FIELD and RECORD (so that, after the first
    INVALID byte, the rest of the input still ends fields): the streaming kernels must then keep the group indices
    of agreed chunks (no tag bitmaps in their place) and, in tiles whose true path has died, run pass 2 from the
    absorbing state; on a quote-heavy input with INVALID bytes in the middle of tiles"""
    t = dict(W.table("T5"))
    t["tag"] = [list(r) for r in t["tag"]]
    t["tag"][4] = [1, 2, 3, 3]  # INV: FDELIM -> FIELD, RDELIM -> RECORD
    b = W.generate(3, n=96 << 20, seed=29)
    for q in (30 << 20) + np.arange(4) * 1000003:
        b[q:q + 3] = np.frombuffer(b'x"y', np.uint8)
    r = oracle.csv_parse(b, t)
    assert 0 <= r["error_pos"] < b.size
    for path in (None, FUSED):
        _say("absorbing fields", b.size, path, r["n_fields"], r["error_pos"])
        g = ppr.parse(_dev(b), t, capacity=r["n_fields"] + 1, path=path)
        assert g.path == (path or auto_path(b.size))
        _same(g, r, ("absorbing fields", path))


@pytest.mark.parametrize("path,cap", [(None, 100), (None, 20000), (FUSED, 20000), (SINGLE_PASS, 20000)])
def test_capacity_reported(ppr, path, cap):
    """with too few output slots: PPR_ECAPACITY, the counts set, the first cap fields written and nothing past
    them (guard words after each array stay untouched); the binding then resizes and fills"""
    import ctypes
    import torch
    t = W.table("T5")
    b = W.generate(1, n=1 << 20, seed=9)
    r = oracle.csv_parse(b, t)
    assert r["n_fields"] > cap
    P = ppr.Parser(t, max_n=b.size, capacity=cap, path=path)
    guard = 4096
    arrs = [torch.full((cap + guard,), -1, dtype=torch.int32, device="cuda") for _ in range(4)]
    out = ppr.ParseOut()
    out.record_idx, out.column_ids, out.field_offsets, out.field_lengths = [a.data_ptr() for a in arrs]
    out.cap_fields = cap
    d = _dev(b)
    rc = ppr.lib.ppr_parse(ctypes.c_void_p(d.data_ptr()), b.size, ctypes.byref(P.dfa), P.class_map,
                           ctypes.byref(out), P._ws_ptr(), P.ws_bytes, ctypes.byref(P.opts), None)
    assert rc == ppr.PPR_ECAPACITY
    assert out.n_fields == r["n_fields"] and out.n_records == r["n_records"]
    assert out.path == (path or auto_path(b.size))
    for a, key in zip(arrs, ("rec", "col", "off", "len")):
        got = _np(a)
        assert np.array_equal(got[:cap], r[key][:cap]), key
        assert np.all(got[cap:] == 0xffffffff), (key, "written past the capacity")
    # the binding sizes, then fills
    _same(P(d), r, "resized")


@pytest.mark.parametrize("chunk,path", _with_paths([31, None]))
def test_repeatable(ppr, chunk, path):
    """the same workspace reused: nothing left over from the previous call leaks in"""
    t = W.table("T5")
    b = W.generate(3, n=(8 << 20) + 3, seed=11)
    r = oracle.csv_parse(b, t)
    P = ppr.Parser(t, max_n=b.size, chunk_bytes=chunk, path=path)
    d = _dev(b)
    for i in range(5):
        _say("repeat", chunk, i)
        _same(P(d), r, i)
    # a shorter input on the same workspace, then the long one again
    short = b[: (1 << 20) + 77]
    _same(P(_dev(short)), oracle.csv_parse(short, t), "short")
    _same(P(d), r, "again")


def test_path_reported(ppr):
    """the table-driven kernels run for 64-byte chunks on aligned input with an encodable class map (left
    to the library: the fused kernel up to 8 MiB, the streaming kernels above); the single-pass kernel
    otherwise"""
    big = W.generate(3, n=FUSED_MAX_AUTO + 64, seed=6)
    assert ppr.parse(_dev(big), W.table("T5"), capacity=big.size + 1).path == STREAMING
    for name in ("T5", "T6"):
        t = W.table(name)
        b = W.generate(1 if name == "T5" else 4, n=300000, seed=5)
        r = oracle.csv_parse(b, t)
        g = ppr.parse(_dev(b), t, capacity=b.size + 1)
        assert g.path == FUSED, name
        for want in (ppr.PPR_PATH_FUSED, ppr.PPR_PATH_STREAMING, ppr.PPR_PATH_SINGLE_PASS):
            g = ppr.parse(_dev(b), t, capacity=b.size + 1, path=want)
            assert g.path == want, (name, want)
            _same(g, r, (name, want))
        g31 = ppr.parse(_dev(b), t, chunk_bytes=31, capacity=b.size + 1)
        assert g31.path == ppr.PPR_PATH_SINGLE_PASS, name
        g31 = ppr.parse(_dev(b), t, chunk_bytes=31, capacity=b.size + 1, path=ppr.PPR_PATH_FUSED)
        assert g31.path == ppr.PPR_PATH_SINGLE_PASS, name
    with pytest.raises(ppr.PprError):
        ppr.parse(_dev(b), t, capacity=b.size + 1, path=4)
    # more than 8 non-catch-all bytes: not encodable by the streaming classifier
    rng = np.random.default_rng(3)
    t = _random_table(rng, True, 40)
    b = rng.integers(0, 256, 5000).astype(np.uint8)
    g = ppr.parse(_dev(b), t, capacity=b.size + 1)
    assert g.path == ppr.PPR_PATH_SINGLE_PASS
    _same(g, oracle.csv_parse(b, t), "40 specials")


@pytest.mark.parametrize("path,stages", [(STREAMING, 3), (FUSED, 2)])
def test_stage_events(ppr, path, stages):
    """per-kernel HIP events recorded by the library between its kernels"""
    import torch
    t = W.table("T5")
    b = W.generate(3, n=(4 << 20), seed=2)
    d = _dev(b)
    P = ppr.Parser(t, max_n=b.size, path=path)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(stages + 1)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    P.launch(d, stage_events=ev)
    torch.cuda.synchronize()
    o = P.results(b.size)
    assert o.path == path
    times = [ev[i].elapsed_time(ev[i + 1]) for i in range(stages)]
    assert all(x >= 0 for x in times) and sum(times) > 0, times
    assert o.n_fields == oracle.csv_parse(b, t)["n_fields"]


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_full_size_workloads(ppr, cfg):
    """every output array at the workload's full size: in the launch configuration the benchmark times
    (the default 64-byte chunks, the automatic path), on the streaming and the fused kernels, and at the
    workload's own chunk size if it names one"""
    t = W.table(W.CONFIGS[cfg]["table"])
    _say("full", cfg, "generate")
    b = W.generate(cfg)
    _say("full", cfg, "oracle")
    r = oracle.csv_parse(b, t)
    d = _dev(b)
    runs = [(None, None), (None, STREAMING), (None, FUSED)]
    if W.CONFIGS[cfg].get("chunk_bytes"):
        runs.append((W.CONFIGS[cfg]["chunk_bytes"], None))
    for chunk, path in runs:
        _say("full", cfg, "gpu chunk", chunk, path, r["n_fields"])
        g = ppr.Parser(t, max_n=b.size, capacity=r["n_fields"], chunk_bytes=chunk, path=path)(d)
        if chunk is None:
            assert g.path == (path or auto_path(b.size))
        _same(g, r, ("full", cfg, chunk, path))
    del b, d


N_MAX = (1 << 32) - (1 << 16)  # the largest input ppr_parse takes


@pytest.mark.slow
def test_maximum_size(ppr):
    """the largest input the library takes (2^32 - 2^16 bytes of the quote-heavy workload: positions, field
    offsets and lengths near 2^32), every output array, on the streaming and the fused kernels; and a ragged
    size just below it (a partial last tile) on the automatic path"""
    import torch
    t = W.table(W.CONFIGS[3]["table"])
    _say("max: generate", N_MAX)
    b = W.generate(3, n=N_MAX)
    d = _dev(b)
    for n, paths in ((N_MAX, (None, FUSED)), (N_MAX - 4093, (None,))):
        _say("max: oracle", n)
        r = oracle.csv_parse(b[:n], t, cap=n // 16)
        for path in paths:
            _say("max: gpu", n, path, r["n_fields"])
            g = ppr.Parser(t, max_n=n, capacity=r["n_fields"], path=path)(d[:n])
            assert g.path == (path or auto_path(n))
            _same(g, r, ("max", n, path))
            del g
            torch.cuda.empty_cache()
        del r
    del b, d
