"""Pins of the columnar-partition oracle (oracle/columns.py) against things
other than itself: hand-worked examples, Python's csv module (each column's
values and the records that have them), the independent recursive-descent
reader on every short input, and invariants of the two terminator variants.

ParPaRaw, Sec. 3 (partitioning, CSS, CSS index, Fig. 5) and the
specialisations passage (inline-terminated and vector-delimited CSS, Fig. 6).
"""
import csv
import io
import itertools
import random

import numpy as np
import pytest

import oracle
import workloads as W
from oracle import columns as C
from tests.rd_reader import read_t5


def _part(b, r, mode=C.MODE_INDEXED, term=0x1F):
    return C.partition(b, r["rec"], r["col"], r["off"], r["len"], mode, term)


def _fields_by_column(p):
    """{column: [(record, bytes), ...]} read back through the index"""
    out = {}
    css = p["css"].tobytes()
    for c in range(p["n_columns"]):
        lo, hi = int(p["col_first_field"][c]), int(p["col_first_field"][c + 1])
        out[c] = [(int(p["rec"][j]), css[p["css_off"][j]:p["css_off"][j] + p["length"][j]]) for j in range(lo, hi)]
    return out


def test_hand_worked():
    """the pages' example string, worked by hand: column 0 holds "1" (record 0) and "2" (record 1), column 1
    holds "Apples" (record 0)"""
    t = W.table("T5")
    b = b"1,Apples\n2\n"
    r = oracle.csv_parse(b, t)
    p = _part(b, r)
    assert p["css"].tobytes() == b"12Apples"
    assert p["col_first_field"].tolist() == [0, 2, 3] and p["col_first_byte"].tolist() == [0, 2, 8]
    assert p["rec"].tolist() == [0, 1, 0] and p["css_off"].tolist() == [0, 1, 2] and p["length"].tolist() == [1, 1, 6]
    p = _part(b, r, C.MODE_INLINE, 0x1E)
    assert p["css"].tobytes() == b"1\x1e2\x1eApples\x1e" and p["col_first_byte"].tolist() == [0, 4, 11]
    assert p["css_off"].tolist() == [0, 2, 4]
    p = _part(b, r, C.MODE_VECTOR)
    assert p["css"].tobytes() == b"1\x002\x00Apples\x00"
    assert p["aux"].tolist() == [0, 1, 0, 1, 0, 0, 0, 0, 0, 0, 1]
    # empty fields keep their entries; a record of one empty field (an empty line) too
    b = b"a,,c\n\n,x\n"
    r = oracle.csv_parse(b, t)
    p = _part(b, r, C.MODE_INLINE, 0x1F)
    assert p["css"].tobytes() == b"a\x1f\x1f\x1f\x1fx\x1fc\x1f"
    assert p["rec"].tolist() == [0, 1, 2, 0, 2, 0] and p["length"].tolist() == [1, 0, 0, 0, 1, 1]
    assert p["col_first_field"].tolist() == [0, 3, 5, 6]
    p = _part(b"", oracle.csv_parse(b"", t))
    assert p["n_columns"] == 0 and p["css_bytes"] == 0 and p["col_first_field"].tolist() == [0]


def _unquote(s: bytes) -> bytes:
    if len(s) >= 2 and s[:1] == b'"' and s[-1:] == b'"':
        return s[1:-1].replace(b'""', b'"')
    return s


def test_matches_csv_module_columns():
    """valid quoted inputs: each column's values (unquoted) and records are what the csv module's rows give"""
    t = W.table("T5")
    rng = random.Random(11)
    checked = 0
    for _ in range(1500):
        recs = []
        for _ in range(rng.randrange(1, 7)):
            row = []
            for _ in range(rng.randrange(1, 6)):
                body = "".join(rng.choice('ab,\n"') for _ in range(rng.randrange(0, 5)))
                row.append('"' + body.replace('"', '""') + '"' if rng.random() < 0.5 or any(
                    ch in body for ch in ',\n"') else body)
            recs.append(",".join(row))
        text = "\n".join(recs) + ("\n" if rng.random() < 0.5 else "")
        if any(x == "" for x in recs):
            continue
        b = text.encode()
        rows = list(csv.reader(io.StringIO(text, newline=""), strict=True))
        r = oracle.csv_parse(b, t)
        for mode in (C.MODE_INDEXED, C.MODE_INLINE, C.MODE_VECTOR):
            got = _fields_by_column(_part(b, r, mode))
            want = {}
            for i, row in enumerate(rows):
                for c, v in enumerate(row):
                    want.setdefault(c, []).append((i, v.encode()))
            assert {c: [(ri, _unquote(s)) for ri, s in v] for c, v in got.items()} == want, text
        checked += 1
    assert checked > 500


def test_exhaustive_vs_recursive_descent():
    """every five-state input up to 6 bytes: the reader's fields, grouped by column in record order"""
    t = W.table("T5")
    inputs = [bytes(x) for L in range(7) for x in itertools.product(b',\n"a', repeat=L)]
    for b, r in zip(inputs, oracle.csv_parse_many(inputs, t)):
        fields, nrec, err = read_t5(b)
        want = {}
        for (rec, col, off, ln) in fields:
            want.setdefault(col, []).append((rec, b[off:off + ln]))
        for mode in (C.MODE_INDEXED, C.MODE_INLINE):
            got = _fields_by_column(_part(b, r, mode))
            assert {c: v for c, v in got.items() if v} == want, (b, mode)


def test_variant_invariants():
    """on the workloads: the inline CSS holds exactly one terminator per field when no field holds one; the
    vector CSS's aux marks exactly the slots; lengths add up; records increase within a column"""
    for cfg in (1, 3, 4):
        t = W.table(W.CONFIGS[cfg]["table"])
        b = W.generate(cfg, n=60000, seed=5)
        r = oracle.csv_parse(b, t)
        nf = r["n_fields"]
        pi = _part(b, r, C.MODE_INLINE, 0x1E)
        assert int(np.count_nonzero(b == 0x1E)) == 0
        assert int(np.count_nonzero(pi["css"] == 0x1E)) == nf
        assert pi["css_bytes"] == int(r["len"].astype(np.int64).sum()) + nf
        pv = _part(b, r, C.MODE_VECTOR)
        assert int(pv["aux"].sum()) == nf and np.array_equal(np.nonzero(pv["aux"])[0], pv["css_off"] + pv["length"])
        px = _part(b, r)
        for c in range(px["n_columns"]):
            lo, hi = px["col_first_field"][c], px["col_first_field"][c + 1]
            assert np.all(np.diff(px["rec"][lo:hi]) > 0)
        assert px["col_first_field"][-1] == nf and px["css_bytes"] == int(r["len"].astype(np.int64).sum())
