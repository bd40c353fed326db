"""The all-core CPU baseline (oracle/cpu_parallel.c) against the sequential oracle.

The baseline runs the data-parallel method on host threads: per-slice
state-transition vectors from every state, a serial composition, then two more
passes per slice from its carried start state (counts, then fields). Its
results must be the oracle's, bit for bit, for any number of slices: the tests
cut inputs at every kind of position (inside quoted fields, escapes, comments,
tokens; one byte per slice), on every workload generator, on invalid input and
with too few output slots.
"""
import itertools

import numpy as np
import pytest

import oracle
import workloads as W

THREADS = (1, 2, 3, 7, 16, 61)


def _same_csv(a, r, what):
    for key in ("n_fields", "n_records", "error_pos", "end_state", "min_columns", "max_columns"):
        assert a[key] == r[key], (what, key, a[key], r[key])
    for key in ("rec", "col", "off", "len"):
        assert np.array_equal(a[key], r[key]), (what, key)


def _same_lex(a, r, what):
    assert a["n_tokens"] == r["n_tokens"], (what, a["n_tokens"], r["n_tokens"])
    for key in ("kind", "start", "length"):
        assert np.array_equal(a[key], r[key]), (what, key)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_csv_workloads(cfg):
    t = W.table("T6" if cfg == 4 else "T5")
    b = W.generate(cfg, n=(1 << 20) + 12345, seed=40 + cfg)
    r = oracle.csv_parse(b, t)
    for T in THREADS:
        _same_csv(oracle.csv_parse_parallel(b, t, T), r, (cfg, T))


def test_csv_edge_cases():
    t5, t6 = W.table("T5"), W.table("T6")
    cases = [
        (t5, b""), (t5, b","), (t5, b"\n"), (t5, b'"'), (t5, b"x"), (t5, b"a,b\n"), (t5, b"a,b"),
        (t5, b"," * 1000), (t5, b"\n" * 1001), (t5, b'"' + b"a,\n" * 700),
        (t5, b'a"' + b"b" * 900),                  # INVALID at byte 1, then the absorbing state
        (t5, (b'"x""y",' * 90) + b'"z'),           # escapes across every cut
        (t6, b"#" + b"\t\"" * 500 + b"\n"), (t6, b"\t" * 700), (t6, b"\n#\n#x\n"),
    ]
    for t, b in cases:
        r = oracle.csv_parse(b, t)
        for T in THREADS + (len(b), len(b) + 5):
            if T == 0:
                continue
            _same_csv(oracle.csv_parse_parallel(b, t, T), r, (t["name"], len(b), T))


def test_csv_exhaustive_one_byte_slices():
    """every input over {a , \\n "} up to 6 bytes, cut into one slice per byte and into 2"""
    t = W.table("T5")
    for n in range(1, 7):
        for tup in itertools.product(b'a,\n"', repeat=n):
            b = bytes(tup)
            r = oracle.csv_parse(b, t)
            for T in {2, n}:
                _same_csv(oracle.csv_parse_parallel(b, t, T), r, (b, T))


def test_csv_capacity_and_invalid():
    t = W.table("T5")
    b = W.generate(3, n=1 << 20, seed=77)
    r = oracle.csv_parse(b, t)
    cap = r["n_fields"] // 3
    a = oracle.csv_parse_parallel(b, t, 16, cap=cap)
    assert a["rc"] == -2 and a["n_fields"] == r["n_fields"] and a["n_records"] == r["n_records"]
    for key in ("rec", "col", "off", "len"):
        assert np.array_equal(a[key], r[key][:cap]), key
    bad = b.copy()
    bad[700001:700004] = np.frombuffer(b'x"y', np.uint8)
    rb = oracle.csv_parse(bad, t)
    assert 0 <= rb["error_pos"] < bad.size
    _same_csv(oracle.csv_parse_parallel(bad, t, 16), rb, "invalid")


def test_csv_rejects_bad_tables():
    t = W.table("T5")
    bad = dict(t, next=[row[:] for row in t["next"]])
    bad["next"][0][0] = 9
    with pytest.raises(ValueError):
        oracle.csv_parse_parallel(b"a,b\n", bad, 4)
    with pytest.raises(ValueError):
        oracle.csv_parse_parallel(b"a,b\n", t, 0)


def test_lex_streams_and_edges():
    d = W.lexer_dfa()
    rng = np.random.default_rng(5)
    cases = [W.gen_tokens(s, n) for s, n in ((1, 1), (2, 39), (3, 4097), (4, (1 << 20) + 7))]
    cases += [np.frombuffer(x, np.uint8) for x in (b"", b"a", b"@", b"//" + b"x" * 700, b'"' + b"q" * 701,
                                                    b" " * 1000, b"1." * 300)]
    cases += [rng.integers(0, 256, int(rng.integers(1, 5000)), dtype=np.uint8) for _ in range(4)]
    for b in cases:
        r = oracle.lex_restart(b, d)
        for T in THREADS + (max(1, b.size),):
            _same_lex(oracle.lex_restart_parallel(b, d, T), r, (b.size, T))


def test_lex_exhaustive_one_byte_slices():
    """every input over a small alphabet that opens and closes strings (with escapes), line comments, numbers and
    identifiers, up to 5 bytes, one slice per byte and two slices"""
    d = W.lexer_dfa()
    for n in range(1, 6):
        for tup in itertools.product(b'a1"/\n\\', repeat=n):
            b = np.frombuffer(bytes(tup), np.uint8)
            r = oracle.lex_restart(b, d)
            for T in (2, n):
                _same_lex(oracle.lex_restart_parallel(b, d, T), r, (bytes(tup), T))


def test_lex_capacity():
    d = W.lexer_dfa()
    b = W.gen_tokens(9, 1 << 18)
    r = oracle.lex_restart(b, d)
    cap = r["n_tokens"] // 2
    a = oracle.lex_restart_parallel(b, d, 16, cap=cap)
    assert a["rc"] == -2 and a["n_tokens"] == r["n_tokens"]
    for key in ("kind", "start", "length"):
        assert np.array_equal(a[key], r[key][:cap]), key
