"""GPU parity of numeric type inference and conversion (ppr_infer_types,
ppr_convert) against the oracle (oracle/numbers.py, applied to the oracle's
own parse of the same bytes).

ParPaRaw, "Type inference" and "Default values for empty strings"
(capabilities section); Sec. 3 (conversion to the column's type, threads
alone on short fields and collaborating on long ones). Bit-exact on every
field's type, every column's type, every value (int64, or the double's bits)
and every status: on mixed numeric texts (all widths and their bounds, beyond
int64, inside and outside the exactly converted class, zero-padded and long
digit strings, text with long numeric prefixes, empty fields), with inferred
and with imposed column types, through a parse's arrays and through a CSS
index, on a numeric CSV workload, and on blocks whose long numbers overflow
the workgroup's queue.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle import columns as C
from oracle import numbers as N

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ppr():
    import torch
    assert torch.cuda.is_available()
    import dfa_parsing_delimiter_amd as m
    return m


def _dev(b):
    import torch
    if not len(b):
        return torch.zeros(0, dtype=torch.uint8, device="cuda")
    return torch.from_numpy(np.array(np.frombuffer(bytes(b), np.uint8), copy=True)).to("cuda")


def _u(t, dt=np.uint32):
    return t.cpu().numpy().view(dt)


def _parse(ppr, b):
    t = W.table("T5")
    d = _dev(b)
    g = ppr.parse(d, t, capacity=len(b) + 2)
    r = oracle.csv_parse(b, t)
    assert g.n_fields == r["n_fields"] and g.max_columns == r["max_columns"]
    return d, g, r


def _check_infer(ppr, F, b, off, length, col, nc, what):
    ct, ft = ppr.infer_types(F, field_types=True)
    oft, oct = N.infer(b, off, length, col, nc)
    got = ft.cpu().numpy()
    if not np.array_equal(got, oft):
        bad = np.nonzero(got != oft)[0]
        j = bad[0]
        raise AssertionError("%s field types differ at %d of %d (first %d: %r gpu %s oracle %s)" % (
            what, bad.size, got.size, j, bytes(b[off[j]:off[j] + length[j]])[:80], N.TYPE_NAMES[got[j]],
            N.TYPE_NAMES[oft[j]]))
    assert np.array_equal(ct, oct), (what, ct, oct)
    return oct


def _check_convert(ppr, F, b, off, length, col, types, what, idef=-77, fdef=3.25):
    cv = ppr.convert(F, types, int_default=idef, float_default=fdef)
    ov, ost = N.convert(b, off, length, col, types, idef, fdef)
    st, v = cv.status.cpu().numpy(), _u(cv.values, np.int64)
    if not (np.array_equal(st, ost) and np.array_equal(v, ov)):
        bad = np.nonzero((st != ost) | (v != ov))[0]
        j = bad[0]
        raise AssertionError("%s conversion differs at %d of %d (first %d: %r column type %s: gpu %d %x oracle %d %x)"
                             % (what, bad.size, st.size, j, bytes(b[off[j]:off[j] + length[j]])[:80],
                                N.TYPE_NAMES[types[col[j]]], st[j], v[j] & 0xffffffffffffffff, ost[j],
                                ov[j] & 0xffffffffffffffff))
    assert np.array_equal(cv.counts, np.bincount(ost, minlength=5)[1:5]), what


IMPOSED = [
    lambda nc: np.full(nc, N.FLOAT64),
    lambda nc: np.full(nc, N.INT64),
    lambda nc: np.arange(nc) % 7,
]


@pytest.mark.parametrize("seed,rows,cols", [(1, 20000, 10), (2, 3000, 40), (3, 50, 3), (4, 1, 1)])
def test_mixed_texts_through_parse(ppr, seed, rows, cols):
    b = W.numeric_csv(seed, rows, cols)
    d, g, r = _parse(ppr, b)
    F = ppr.Fields.of_parse(d, g)
    nc = g.max_columns
    print("numbers mixed", seed, rows, cols, g.n_fields, flush=True)
    oct = _check_infer(ppr, F, b, r["off"], r["len"], r["col"], nc, (seed, "infer"))
    _check_convert(ppr, F, b, r["off"], r["len"], r["col"], oct.astype(np.uint32), (seed, "inferred types"))
    for k, mk in enumerate(IMPOSED):
        _check_convert(ppr, F, b, r["off"], r["len"], r["col"], mk(nc).astype(np.uint32), (seed, "imposed", k))


def test_through_css_index(ppr):
    b = W.numeric_csv(5, 8000, 12)
    d, g, r = _parse(ppr, b)
    cols = ppr.columns(d, g, mode=ppr.PPR_CSS_INDEXED)
    F = ppr.Fields.of_columns(cols)  # the GPU's CSS and index
    want = C.partition(b, r["rec"], r["col"], r["off"], r["len"], C.MODE_INDEXED)  # the oracle's, for the oracle
    css = want["css"].tobytes()
    off, ln = want["css_off"], want["length"]
    col = np.repeat(np.arange(want["n_columns"]), np.diff(want["col_first_field"]))
    print("numbers css", g.n_fields, flush=True)
    oct = _check_infer(ppr, F, css, off, ln, col, cols.n_columns, "css infer")
    _check_convert(ppr, F, css, off, ln, col, np.full(cols.n_columns, N.FLOAT64, np.uint32), "css float")
    _check_convert(ppr, F, css, off, ln, col, oct.astype(np.uint32), "css inferred")


def test_numeric_workload(ppr):
    """the numeric CSV workload's generator (integers and one-point decimals of 1 to 12 digits), 8 MiB"""
    b = W.generate(2, n=8 << 20, seed=21)
    d, g, r = _parse(ppr, b)
    F = ppr.Fields.of_parse(d, g)
    print("numbers workload", g.n_fields, flush=True)
    oct = _check_infer(ppr, F, b, r["off"], r["len"], r["col"], g.max_columns, "workload infer")
    # (column 0 holds the input's unterminated alphanumeric remainder, so it is TEXT)
    assert all(t in (N.INT8, N.INT16, N.INT32, N.INT64, N.FLOAT64) for t in oct[1:]), oct
    _check_convert(ppr, F, b, r["off"], r["len"], r["col"], oct.astype(np.uint32), "workload convert")


def test_long_numbers_overflow_the_queue(ppr):
    """every field longer than a thread's 32 bytes and still a number: more than a workgroup's queue of 256 per
    2048 fields, so threads also finish long fields alone; plus long texts with numeric prefixes"""
    rng = np.random.default_rng(7)
    rows = []
    for i in range(6000):
        z = "0" * int(rng.integers(30, 80))
        rows.append(",".join([z + str(int(rng.integers(0, 10 ** 6))), "-" + z + "1." + "0" * int(rng.integers(0, 40)),
                              z + "5e-" + "0" * 40 + "3", "1" * int(rng.integers(33, 70)) + ("x" if i % 2 else "")]))
    b = ("\n".join(rows) + "\n").encode()
    d, g, r = _parse(ppr, b)
    F = ppr.Fields.of_parse(d, g)
    oct = _check_infer(ppr, F, b, r["off"], r["len"], r["col"], g.max_columns, "long infer")
    _check_convert(ppr, F, b, r["off"], r["len"], r["col"], oct.astype(np.uint32), "long inferred")
    _check_convert(ppr, F, b, r["off"], r["len"], r["col"], np.full(g.max_columns, N.FLOAT64, np.uint32), "long float")


def test_edges_and_errors(ppr):
    import torch
    # no fields: every column EMPTY
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    F = ppr.Fields(_dev(b"x"), e, e, n_columns=3, col=e)
    ct, _ = ppr.infer_types(F)
    assert list(ct) == [0, 0, 0]
    cv = ppr.convert(F, np.zeros(3, np.uint32))
    assert cv.values.numel() == 0 and list(cv.counts) == [0, 0, 0, 0]
    # one column, no column array; a column id beyond n_columns; a span past the bytes
    text = b"12 -7 1.5 x"
    off = torch.tensor([0, 3, 6, 10, 9], dtype=torch.int32, device="cuda")
    ln = torch.tensor([2, 2, 3, 1, 5], dtype=torch.int32, device="cuda")
    F1 = ppr.Fields(_dev(text), off, ln)
    ct, ft = ppr.infer_types(F1, field_types=True)
    assert list(ft.cpu().numpy()) == [N.INT8, N.INT8, N.FLOAT64, N.TEXT, N.TEXT] and list(ct) == [N.TEXT]
    col = torch.tensor([0, 1, 0, 5, 1], dtype=torch.int32, device="cuda")
    F2 = ppr.Fields(_dev(text), off, ln, n_columns=2, col=col)
    ct, _ = ppr.infer_types(F2)
    assert list(ct) == [N.FLOAT64, N.TEXT]  # (the field of column 5 counts in no column)
    cv = ppr.convert(F2, np.array([N.FLOAT64, N.INT8], np.uint32), int_default=9)
    st = list(cv.status.cpu().numpy())
    assert st == [N.ST_OK, N.ST_OK, N.ST_OK, N.ST_TEXT, N.ST_MISMATCH], st
    assert cv.values.cpu().numpy().view(np.float64)[0] == 12.0 and cv.values[1].item() == -7
    for nc in (0, 4097):
        with pytest.raises((ppr.PprError, ValueError)):
            ppr.infer_types(ppr.Fields(_dev(text), off, ln, n_columns=nc))
    with pytest.raises(ppr.PprError):
        ppr.convert(F1, np.array([7], np.uint32))
