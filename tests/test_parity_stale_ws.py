"""Workspaces need no initialisation: every single-pass entry point clears its
look-back statuses before its first tile runs.

White-box regression test. A status word is [63:34] call epoch, [33:32] flag,
[31:0] payload; the count statuses of the parse and the lexer are [63:32]
epoch, [31:0] value. Before each call under test the whole workspace is
filled with words shaped like that very call's statuses (its epoch, the
"inclusive" flag, an in-range payload): the pattern that stale data of
another entry point or input size can leave where the statuses now lie. The
results must match the oracle bit for bit.

The coming call's epoch is read off the library: a call's epoch is one more
than the previous call's (ppr_columns draws two), and the generic parse path's
first status word (tile 0, inclusive) follows the 256-byte workspace header.
Payloads are chosen so that even a library that read them would stay in
bounds (state 1, identifier 0, counts 0).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle import columns as C

pytestmark = pytest.mark.gpu

STREAMING, SINGLE_PASS, FUSED = 1, 2, 3


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


def _u32(t):
    return t.cpu().numpy().view(np.uint32).astype(np.int64)


def _status(epoch, flag, payload):
    return (epoch << 34) | (flag << 32) | payload


def _signed(w):
    return w - (1 << 64) if w >= 1 << 63 else w


def _epoch_now(ppr):
    """the epoch of the latest library call (a one-tile parse on the generic path, read back)"""
    p = ppr.Parser(W.table("T5"), max_n=64, path=SINGLE_PASS)
    p(_dev(b"a,b\n"))
    w = int(p.ws[p.ws_off + 256:p.ws_off + 264].cpu().numpy().view(np.uint64)[0])
    assert (w >> 32) & 3 == 2 and (w >> 34) > 0, hex(w)
    return w >> 34


def _fill(ws, off, nbytes, words):
    """the workspace [off, off + nbytes) as 64-bit words, cycling through `words`"""
    import torch
    v = ws[off:off + nbytes].view(torch.int64).view(-1)
    for i, w in enumerate(words):
        v[i::len(words)] = _signed(w)
    torch.cuda.synchronize()


def _same_parse(g, r, what):
    assert (g.n_fields, g.n_records, g.error_pos, g.end_state) == (
        r["n_fields"], r["n_records"], r["error_pos"], r["end_state"]), what
    assert (g.min_columns, g.max_columns) == (r["min_columns"], r["max_columns"]), what
    for name, key in (("record_idx", "rec"), ("column_ids", "col"), ("field_offsets", "off"),
                      ("field_lengths", "len")):
        assert np.array_equal(_u32(getattr(g, name)), r[key]), (what, name)


@pytest.mark.parametrize("path", [SINGLE_PASS, FUSED])
def test_parse(ppr, path):
    t = W.table("T5")
    b = W.generate(1, n=(3 << 20) + 5, seed=71)
    r = oracle.csv_parse(b, t)
    d = _dev(b)
    p = ppr.Parser(t, max_n=b.size, capacity=r["n_fields"], path=path)
    for rep in range(2):
        e = _epoch_now(ppr) + 1
        print("stale parse", path, rep, e, flush=True)
        # vector statuses (state 1) and count statuses (0) of epoch e, alternately
        _fill(p.ws, p.ws_off, p.ws_bytes, [_status(e, 2, 1), e << 32])
        g = p(d)
        assert g.path == path
        _same_parse(g, r, (path, rep))


def test_lex(ppr):
    d = W.lexer_dfa()
    T = ppr.LexTables.from_dfa(d)
    b = W.gen_tokens(9, (2 << 20) + 3)
    r = oracle.lex_restart(b, d)
    lx = ppr.Lexer(T, max_n=b.size, capacity=b.size + 1, path=SINGLE_PASS)
    x = _dev(b)
    for rep in range(2):
        e = _epoch_now(ppr) + 1
        print("stale lex", rep, e, flush=True)
        _fill(lx.ws, lx.ws_off, lx.ws_bytes, [_status(e, 2, 0), e << 32])
        g = lx(x)
        assert g.path == SINGLE_PASS and g.n_tokens == r["n_tokens"]
        for key in ("kind", "start", "length"):
            assert np.array_equal(_u32(getattr(g, key)), r[key]), (rep, key)


def test_columns(ppr):
    t = W.table("T5")
    b = W.generate(1, n=(2 << 20) + 11, seed=72)
    r = oracle.csv_parse(b, t)
    d = _dev(b)
    g = ppr.parse(d, t, capacity=r["n_fields"])
    nc = r["max_columns"]
    want = C.partition(b, r["rec"], r["col"], r["off"], r["len"], C.MODE_INLINE, 0x1F)
    cols = ppr.Columns(g.n_fields, nc, b.size, mode=C.MODE_INLINE, terminator=0x1F)
    for rep in range(2):
        e = _epoch_now(ppr) + 1
        print("stale columns", rep, e, flush=True)
        # the two scans' statuses (epochs e and e + 1), both "inclusive, sum 0"
        _fill(cols.ws, cols.ws_off, cols.ws_bytes, [_status(e, 2, 0), _status(e + 1, 2, 0)])
        got = cols(d, g)
        assert got.css_bytes == want["css_bytes"], rep
        assert np.array_equal(got.css.cpu().numpy(), want["css"]), rep
        for name, key in (("rec", "rec"), ("css_off", "css_off"), ("length", "length")):
            assert np.array_equal(_u32(getattr(got, name)), want[key]), (rep, name)
