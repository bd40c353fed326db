"""Pins of the CSV oracle against things other than itself.

* hand-worked examples (tests/golden/csv_examples.jsonl);
* exhaustive agreement with an independent recursive-descent reader on every
  input up to 8 bytes (five-state table) / 7 bytes (six-state table) over one
  representative byte per symbol class;
* the scan identities the data-parallel method relies on (ParPaRaw, Sec. 3):
  composing per-part state-transition vectors, and combining per-part record
  counts, column offsets (relative/absolute) and last terminators, gives what
  one sequential run over the whole input gives, for every split;
* quote-free inputs against bytes.split, valid quoted inputs against Python's
  csv module (strict), and generator ground truth on every workload.
"""
import csv
import io
import itertools
import json
import os
import random

import numpy as np
import pytest

import oracle
import workloads as W
from tests.rd_reader import read_t5, read_t6

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "csv_examples.jsonl")


def _tuples(r):
    return [tuple(int(r[k][i]) for k in ("rec", "col", "off", "len")) for i in range(r["n_fields"])]


def _all_strings(alphabet: bytes, max_len: int):
    for L in range(max_len + 1):
        for t in itertools.product(alphabet, repeat=L):
            yield bytes(t)


def test_golden_examples():
    cases = [json.loads(line) for line in open(GOLDEN)]
    assert len(cases) >= 10
    for c in cases:
        t = W.table(c["table"])
        r = oracle.csv_parse(c["input"].encode("latin-1"), t)
        assert _tuples(r) == [tuple(f) for f in c["fields"]], c
        assert r["n_records"] == c["n_records"], c
        assert r["error_pos"] == c["error_pos"], c


def _columns_of(fields, n_records):
    """fewest and most fields of any record, counted from a field list (rec, col, off, len)"""
    per = {}
    for f in fields:
        per[f[0]] = per.get(f[0], 0) + 1
    return (min(per.values()), max(per.values())) if n_records else (0, 0)


def test_column_count_examples():
    """fields per record, worked by hand; the first is the pages' example of records with a varying number of
    field delimiters (ParPaRaw, "Inferring or validating number of columns": "1,Apples" then "2")"""
    t = W.table("T5")
    for text, want in ((b"1,Apples\n2\n", (1, 2)), (b"", (0, 0)), (b"a,b,c\nd,e,f", (3, 3)), (b"\n\n", (1, 1)),
                       (b'"x,y",z\n', (2, 2)), (b"a\nb,c,d\n,\n", (1, 3)), (b"a,b\nc", (1, 2))):
        r = oracle.csv_parse(text, t)
        assert (r["min_columns"], r["max_columns"]) == want, (text, r["min_columns"], r["max_columns"])


def test_conformance_examples():
    """records that do not have the expected number of fields, worked by hand (ParPaRaw, "Inferring or
    validating number of columns", and the specialisations passage on rejecting records with an inconsistent
    number of field delimiters): how many, and the first one's index"""
    t = W.table("T5")
    cases = (
        (b"1,Apples\n2\n", 2, (1, 1)),   # the pages' example: the second record has one field
        (b"1,Apples\n2\n", 1, (1, 0)),
        (b"1,Apples\n2\n", 3, (2, 0)),
        (b"", 3, (0, -1)),
        (b"\n\n", 1, (0, -1)),           # an empty line is a record of one empty field
        (b"\n\n", 2, (2, 0)),
        (b"a,b\nc,d\ne", 2, (1, 2)),     # the unterminated final record
        (b'"x,y",z\n"p\nq",r', 2, (0, -1)),
        (b'"x,y",z\n"p\nq",r', 3, (2, 0)),
        (b"a,b,c\nd,e\nf,g,h\n,,,\n", 3, (2, 1)),
        (b"a,b\nc,d", 0, (0, -1)),         # no expectation
    )
    for text, expect, want in cases:
        r = oracle.csv_parse(text, t, expected_columns=expect)
        assert (r["bad_records"], r["first_bad_record"]) == want, (text, expect, r["bad_records"],
                                                                   r["first_bad_record"])


def _conformance_of(fields, n_records, expect):
    per = {}
    for f in fields:
        per[f[0]] = per.get(f[0], 0) + 1
    bad = [i for i in range(n_records) if per.get(i, 0) != expect]
    return len(bad), (bad[0] if bad else -1)


@pytest.mark.parametrize("name,alphabet,max_len,reader", [("T5", b',\n"a', 7, read_t5), ("T6", b'\t\n"#a', 6, read_t6)])
def test_conformance_exhaustive_vs_recursive_descent(name, alphabet, max_len, reader):
    """every input up to max_len bytes, expected counts 1 to 3: the independent reader's records"""
    t = W.table(name)
    inputs = list(_all_strings(alphabet, max_len))
    for expect in (1, 2, 3):
        got = oracle.csv_parse_many(inputs, t, expected_columns=expect)
        for s, r in zip(inputs, got):
            fields, nrec, err = reader(s)
            assert (r["bad_records"], r["first_bad_record"]) == _conformance_of(fields, nrec, expect), (s, expect)


@pytest.mark.parametrize("name,alphabet,max_len,reader", [
    ("T5", b',\n"a', 8, read_t5),
    ("T6", b'\t\n"#a', 7, read_t6),
])
def test_exhaustive_vs_recursive_descent(name, alphabet, max_len, reader):
    t = W.table(name)
    inputs = list(_all_strings(alphabet, max_len))
    got = oracle.csv_parse_many(inputs, t)
    bad = 0
    for s, r in zip(inputs, got):
        fields, nrec, err = reader(s)
        if _tuples(r) != fields or r["n_records"] != nrec or r["error_pos"] != err or \
                (r["min_columns"], r["max_columns"]) != _columns_of(fields, nrec):
            bad += 1
            if bad < 5:
                print("mismatch", s, _tuples(r), r["n_records"], r["error_pos"], "reader:", fields, nrec, err)
    assert bad == 0
    assert len(inputs) == sum(len(alphabet) ** L for L in range(max_len + 1))


def _run_from(t, s, data):
    return oracle.csv_parse(data, t, start_state=s)


def _vector(t, data):
    """state-transition vector of a string: end state from every start state"""
    return [_run_from(t, s, data)["end_state"] for s in range(t["n_states"])]


def _tags(t, s, data):
    """tag of every byte when running from state s, read off the DFA table
    (used only to cut the oracle's output into per-part carries)"""
    tags, st = [], s
    for b in data:
        c = t["class_map"][b]
        tags.append(t["tag"][st][c])
        st = t["next"][st][c]
    return tags


def _carry(tags, base):
    """(terminators, records, column carry, last terminator, first invalid) of one part"""
    F, R, I = 1, 2, 3
    nterm = sum(1 for x in tags if x in (F, R))
    nrec = sum(1 for x in tags if x == R)
    last_r = max((i for i, x in enumerate(tags) if x == R), default=None)
    if last_r is None:
        col = ("rel", sum(1 for x in tags if x == F))
    else:
        col = ("abs", sum(1 for x in tags[last_r + 1:] if x == F))
    last_t = max((base + i for i, x in enumerate(tags) if x in (F, R)), default=None)
    first_i = min((base + i for i, x in enumerate(tags) if x == I), default=None)
    return nterm, nrec, col, last_t, first_i


def _op(x, y):
    """combine carries of an earlier part x with a later part y:
    sums for counts, the resolved-wins rule for columns, last defined
    terminator, first defined invalid byte"""
    col = y[2] if y[2][0] == "abs" else (x[2][0], x[2][1] + y[2][1])
    return (x[0] + y[0], x[1] + y[1], col, y[3] if y[3] is not None else x[3],
            x[4] if x[4] is not None else y[4])


@pytest.mark.parametrize("name,alphabet,max_len", [("T5", b',\n"a', 6), ("T6", b'\t\n"#a', 5)])
def test_scan_identities_every_split(name, alphabet, max_len):
    """(vec(u) o vec(v))[s] == run(s, uv) with (a o b)[i] = b[a[i]], a earlier;
    and the per-part carries combined with the scan operators reproduce the
    oracle's whole-input record index, column and offsets."""
    t = W.table(name)
    S = t["n_states"]
    for s in _all_strings(alphabet, max_len):
        whole = _vector(t, s)
        r = oracle.csv_parse(s, t)
        for cut in range(len(s) + 1):
            u, v = s[:cut], s[cut:]
            vu, vv = _vector(t, u), _vector(t, v)
            assert [vv[vu[i]] for i in range(S)] == whole, (s, cut)
            # carries: run u from the start state, v from u's end state
            su = vu[t["start"]]
            cu = _carry(_tags(t, t["start"], u), 0)
            cv = _carry(_tags(t, su, v), cut)
            tot = _op(_op((0, 0, ("abs", 0), None, None), cu), cv)
            n = len(s)
            final = 1 if n > 0 and _tags(t, t["start"], s)[-1] != 2 else 0
            assert tot[0] + final == r["n_fields"], (s, cut)
            assert tot[1] + final == r["n_records"], (s, cut)
            if final:
                # the final field's column, record and start come from the carries
                assert r["col"][-1] == tot[2][1] and tot[2][0] == "abs", (s, cut)
                assert r["rec"][-1] == tot[1], (s, cut)
                assert r["off"][-1] == (0 if tot[3] is None else tot[3] + 1), (s, cut)
            first_invalid = tot[4]
            if first_invalid is not None:
                assert r["error_pos"] == first_invalid, (s, cut)


def test_operators_associative():
    """the column operator and the other carries are associative on random parts"""
    rng = random.Random(7)
    for _ in range(2000):
        parts = []
        for _ in range(3):
            col = (rng.choice(["rel", "abs"]), rng.randrange(5))
            parts.append((rng.randrange(5), rng.randrange(5), col, rng.choice([None, rng.randrange(100)]),
                          rng.choice([None, rng.randrange(100)])))
        a, b, c = parts
        assert _op(_op(a, b), c) == _op(a, _op(b, c))


def _split_reader(b: bytes, fd=b",", rd=b"\n"):
    """quote-free reference: str.split with the final-record rule"""
    if not b:
        return [], 0
    lines = b.split(rd)
    trailing = b.endswith(rd)
    if trailing:
        lines = lines[:-1]
    fields, off = [], 0
    for r, line in enumerate(lines):
        for c, f in enumerate(line.split(fd)):
            fields.append((r, c, off, len(f)))
            off += len(f) + 1
    return fields, len(lines)


def test_quote_free_matches_split():
    t = W.table("T5")
    rng = random.Random(11)
    alphabet = b",\nab9 \r"
    inputs = [bytes(rng.choice(alphabet) for _ in range(rng.randrange(0, 200))) for _ in range(3000)]
    inputs += [W.generate(2, n=1 << 16, seed=s).tobytes() for s in range(3)]
    for s, r in zip(inputs, oracle.csv_parse_many(inputs, t)):
        fields, nrec = _split_reader(s)
        assert _tuples(r) == fields and r["n_records"] == nrec and r["error_pos"] == -1


def _unquote(raw: bytes) -> bytes:
    if raw[:1] == b'"':
        assert raw[-1:] == b'"'
        return raw[1:-1].replace(b'""', b'"')
    return raw


def test_valid_quoted_matches_csv_module():
    """Python's csv module (strict) on valid five-state inputs without blank lines"""
    t = W.table("T5")
    rng = random.Random(5)
    checked = 0
    for _ in range(3000):
        recs = []
        for _ in range(rng.randrange(1, 6)):
            row = []
            for _ in range(rng.randrange(1, 5)):
                body = "".join(rng.choice('ab,\n"') for _ in range(rng.randrange(0, 6)))
                if rng.random() < 0.5 or any(ch in body for ch in ',\n"'):
                    row.append('"' + body.replace('"', '""') + '"')
                else:
                    row.append(body)
            recs.append(",".join(row))
        text = "\n".join(recs) + ("\n" if rng.random() < 0.5 else "")
        if any(r == "" for r in recs):
            continue  # the csv module skips blank lines
        b = text.encode()
        r = oracle.csv_parse(b, t)
        assert r["error_pos"] == -1
        rows = list(csv.reader(io.StringIO(text, newline=""), strict=True))
        ours = {}
        for (rec, col, off, ln) in _tuples(r):
            ours.setdefault(rec, []).append(_unquote(b[off:off + ln]).decode())
        assert [ours[i] for i in range(r["n_records"])] == rows, text
        assert (r["min_columns"], r["max_columns"]) == (min(map(len, rows)), max(map(len, rows))), text
        expect = len(rows[0])
        rc = oracle.csv_parse(b, t, expected_columns=expect)
        bad = [i for i, row in enumerate(rows) if len(row) != expect]
        assert (rc["bad_records"], rc["first_bad_record"]) == (len(bad), bad[0] if bad else -1), text
        checked += 1
    assert checked > 1000


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_generator_ground_truth(cfg):
    """the generator places every field itself; the oracle must find exactly those"""
    t = W.table(W.CONFIGS[cfg]["table"])
    for seed in (1, 2):
        for n in (0, 1, 17, 1 << 18):
            b, truth = W.generate(cfg, n=n, seed=seed, truth=True)
            r = oracle.csv_parse(b, t)
            assert r["error_pos"] == -1
            assert r["n_fields"] == truth["n_fields"] and r["n_records"] == truth["n_records"]
            for k in ("rec", "col", "off", "len"):
                assert np.array_equal(r[k], truth[k]), (cfg, seed, n, k)
