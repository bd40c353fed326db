"""GPU parity: ppr_lex (HIP path, through the C ABI) against the CPU oracles.

The expected tokens come from the restart lexer over the grammar's DFA (no
table is involved on that side); the GPU runs on tables built by the library's
host builder. Bit-exact on (kind, start, length) and the token count.
"""
import json
import os
import sys

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

STREAMING, SINGLE_PASS = 1, 2
STREAM_MIN_AUTO = 8 << 20  # the automatic choice: the streaming kernels above this many bytes (40-byte chunks)


def auto_path(n, chunk=None):
    return STREAMING if (chunk in (None, 40) and n > STREAM_MIN_AUTO) else SINGLE_PASS


GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lex_examples.jsonl")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ppr():
    import torch
    assert torch.cuda.is_available()
    import dfa_parsing_delimiter_amd as m
    return m


@pytest.fixture(scope="module")
def tables(ppr):
    return {"lexer": (W.lexer_dfa(), ppr.LexTables.from_dfa(W.lexer_dfa())),
            "toy": (W.toy_dfa(), ppr.LexTables.from_dfa(W.toy_dfa()))}


def _dev(b):
    import torch
    arr = np.frombuffer(bytes(b), dtype=np.uint8) if not isinstance(b, np.ndarray) else b
    return torch.from_numpy(np.array(arr, dtype=np.uint8, copy=True)).to("cuda")


def _np(t):
    return t.cpu().numpy().view(np.uint32)


def _same(g, r, what=""):
    assert g.n_tokens == r["n_tokens"], (what, g.n_tokens, r["n_tokens"])
    for key in ("kind", "start", "length"):
        a = _np(getattr(g, key))
        if not np.array_equal(a, r[key]):
            bad = np.nonzero(a != r[key])[0]
            raise AssertionError("%s %s differs at %d of %d (first %d: gpu %d oracle %d)" % (
                what, key, bad.size, a.size, bad[0], a[bad[0]], r[key][bad[0]]))


# (chunk, path): the streaming kernels at the default 40-byte chunks, asked for
# or left to the library; the single-pass kernel asked for or at other chunk sizes
PATHS = [(1, None), (2, None), (32, None), (None, None), (None, STREAMING), (None, SINGLE_PASS)]


def test_golden(ppr, tables):
    for line in open(GOLDEN):
        c = json.loads(line)
        d, T = tables[c["grammar"]]
        b = c["input"].encode()
        for chunk, path in PATHS:
            _say("golden", repr(b), chunk, path)
            g = ppr.lex(_dev(b), T, chunk_bytes=chunk, capacity=len(b) + 1, path=path)
            _same(g, oracle.lex_restart(b, d), (b, chunk, path))


@pytest.mark.parametrize("chunk,path", [(1, None), (3, None), (16, None), (31, None), (32, None), (40, None),
                                        (40, STREAMING), (40, SINGLE_PASS), (64, None)])
def test_streams_several_tiles(ppr, tables, chunk, path):
    d, T = tables["lexer"]
    for seed in (1, 2):
        n = (2 << 20) + 777 * seed
        b = W.gen_tokens(seed, n)
        _say("stream", chunk, path, seed, n)
        g = ppr.lex(_dev(b), T, chunk_bytes=chunk, capacity=n + 1, path=path)
        _same(g, oracle.lex_restart(b, d), (chunk, path, seed))
        assert g.path == (path or auto_path(n, chunk))


def test_random_bytes_and_edges(ppr, tables):
    d, T = tables["lexer"]
    rng = np.random.default_rng(4)
    cases = [b"", b"a", b"@", b"//" + b"x" * 70000, b'"' + b"q" * 70001, b" " * 100000, b"1." * 30000]
    cases += [rng.integers(0, 256, int(rng.integers(1, 50000)), dtype=np.uint8).tobytes() for _ in range(6)]
    for b in cases:
        for chunk, path in [(1, None), (7, None), (32, None), (None, None), (None, STREAMING), (None, SINGLE_PASS)]:
            _say("edge", len(b), chunk, path)
            g = ppr.lex(_dev(b) if b else _dev(b"\0")[:0], T, chunk_bytes=chunk, capacity=len(b) + 1, path=path)
            _same(g, oracle.lex_restart(b, d), (len(b), chunk, path))


def test_streaming_ragged_tiles_and_ranges(ppr, tables):
    """the streaming kernels at lengths around their 20 KiB tiles and 40-byte chunks (a last chunk of 1 byte,
    a last tile of one chunk), and with more tiles than ranges (the 1024 ranges then hold one or two tiles)"""
    d, T = tables["lexer"]
    tile = 512 * 40
    for n in (1, 39, 40, 41, tile - 1, tile, tile + 1, 3 * tile + 40 * 17 + 1, 1500 * tile + 12345):
        b = W.gen_tokens(7, n)
        _say("ragged", n)
        g = ppr.lex(_dev(b), T, capacity=n + 1, path=STREAMING)
        assert g.path == STREAMING
        _same(g, oracle.lex_restart(b, d), n)


def test_streaming_needs_aligned_input(ppr, tables):
    """an input that does not start on 8 bytes runs the single-pass kernel, with the same tokens"""
    d, T = tables["lexer"]
    b = W.gen_tokens(8, 300000)
    buf = _dev(np.concatenate([np.zeros(3, np.uint8), b]))
    g = ppr.lex(buf[3:], T, capacity=b.size + 1, path=STREAMING)
    assert g.path == SINGLE_PASS
    _same(g, oracle.lex_restart(b, d), "misaligned")
    assert ppr.lex(_dev(b), T, capacity=b.size + 1, path=STREAMING).path == STREAMING


def test_minimal_automaton_and_identifier_fold(ppr, tables):
    """the second pass steps the minimal automaton of the fold when the prepared tables hold one, and re-folds
    the identifiers otherwise; both against the oracle. Without the automaton or the fold rows the streaming
    kernels do not run."""
    d, T = tables["lexer"]
    assert 0 < T.prep.n_states <= T.k, T.prep.n_states
    assert 0 < T.prep.n_rows <= T.k, T.prep.n_rows
    b = W.gen_tokens(3, (1 << 20) + 5)
    r = oracle.lex_restart(b, d)
    _same(ppr.lex(_dev(b), T, capacity=b.size + 1, path=STREAMING), r, "streaming")
    _same(ppr.lex(_dev(b), T, capacity=b.size + 1, path=SINGLE_PASS), r, "minimal automaton")
    for field in ("n_rows", "n_states"):
        saved = getattr(T.prep, field)
        setattr(T.prep, field, 0)
        try:
            g = ppr.lex(_dev(b), T, capacity=b.size + 1, path=STREAMING)
            assert g.path == SINGLE_PASS
            _same(g, r, "without " + field)
        finally:
            setattr(T.prep, field, saved)


@pytest.mark.slow
def test_full_size_lexer_workload(ppr, tables):
    d, T = tables["lexer"]
    _say("full lexer: generate")
    b = W.generate(5)
    _say("full lexer: oracle")
    r = oracle.lex_restart(b, d)
    _say("full lexer: gpu", r["n_tokens"])
    d_b = _dev(b)
    for path in (None, SINGLE_PASS):
        g = ppr.Lexer(T, max_n=b.size, capacity=r["n_tokens"], path=path)(d_b)
        assert g.path == (path or auto_path(b.size))
        _same(g, r, ("full", path))


@pytest.mark.parametrize("path,cap", [(STREAMING, 1000), (STREAMING, 100000), (SINGLE_PASS, 1000),
                                      (SINGLE_PASS, 100000)])
def test_capacity_reported(ppr, tables, path, cap):
    """with too few output slots: PPR_ECAPACITY, the token count set, the first cap tokens written and nothing
    past them (guard words after each array stay untouched); the binding then resizes and fills"""
    import ctypes
    import torch
    d, T = tables["lexer"]
    b = W.gen_tokens(11, (1 << 20) + 33)
    r = oracle.lex_restart(b, d)
    Lx = ppr.Lexer(T, max_n=b.size, capacity=cap, path=path)
    guard = 4096
    arrs = [torch.full((cap + guard,), -1, dtype=torch.int32, device="cuda") for _ in range(3)]
    o = ppr.TokensOut()
    o.kind, o.start, o.length = [a.data_ptr() for a in arrs]
    o.cap_tokens = cap
    d_b = _dev(b)
    rc = ppr.lib.ppr_lex(ctypes.c_void_p(d_b.data_ptr()), b.size, ctypes.byref(T.c), ctypes.byref(T.prep),
                         ctypes.byref(o), Lx._ws_ptr(), Lx.ws_bytes, ctypes.byref(Lx.opts), None)
    assert rc == ppr.PPR_ECAPACITY
    assert o.n_tokens == r["n_tokens"] and o.path == path
    for a, key in zip(arrs, ("kind", "start", "length")):
        got = _np(a)
        assert np.array_equal(got[:cap], r[key][:cap]), key
        assert np.all(got[cap:] == 0xffffffff), (key, "written past the capacity")
    _same(Lx(d_b), r, "resized")


@pytest.mark.parametrize("path", [STREAMING, SINGLE_PASS])
def test_repeatable(ppr, tables, path):
    """the same workspace reused: nothing from the previous call leaks in (a shorter input, then the long one)"""
    d, T = tables["lexer"]
    b = W.gen_tokens(12, (6 << 20) + 5)
    r = oracle.lex_restart(b, d)
    Lx = ppr.Lexer(T, max_n=b.size, capacity=b.size + 1, path=path)
    dev = _dev(b)
    for i in range(3):
        _say("lex repeat", path, i)
        _same(Lx(dev), r, (path, i))
    short = b[: (1 << 20) + 9]
    _same(Lx(_dev(short)), oracle.lex_restart(short, d), "short")
    _same(Lx(dev), r, "again")


def test_automatic_path_by_size(ppr, tables):
    """left to the library, the single-pass kernel up to 8 MiB and the streaming kernels above; both exact"""
    d, T = tables["lexer"]
    b = W.gen_tokens(14, STREAM_MIN_AUTO + 41)
    dev = _dev(b)
    for n in (STREAM_MIN_AUTO, STREAM_MIN_AUTO + 41):
        _say("lex auto", n)
        g = ppr.lex(dev[:n], T, capacity=n + 1)
        assert g.path == auto_path(n), (n, g.path)
        _same(g, oracle.lex_restart(b[:n], d), ("auto", n))


def test_stage_events_streaming(ppr, tables):
    """the streaming lexer records an event before its kernels and after the first two, the count and the emit
    kernel"""
    import torch
    d, T = tables["lexer"]
    b = W.gen_tokens(13, 4 << 20)
    Lx = ppr.Lexer(T, max_n=b.size, capacity=b.size + 1, path=STREAMING)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    Lx.launch(_dev(b), stage_events=ev)
    torch.cuda.synchronize()
    o = Lx.results(b.size)
    assert o.path == STREAMING
    times = [ev[i].elapsed_time(ev[i + 1]) for i in range(3)]
    assert all(x >= 0 for x in times) and sum(times) > 0, times
    assert o.n_tokens == oracle.lex_restart(b, d)["n_tokens"]


N_MAX = (1 << 32) - (1 << 16)  # the largest input ppr_lex takes


@pytest.mark.slow
def test_maximum_size(ppr, tables):
    """the largest input the library takes (2^32 - 2^16 bytes: copies of the seeded token stream, token
    starts near 2^32), every output array, on the streaming and the single-pass kernels; and a ragged size just
    below it (a partial last tile) on the automatic path"""
    import torch
    d, T = tables["lexer"]
    _say("max lexer: generate", N_MAX)
    unit = W.generate(5)
    b = np.empty(N_MAX, dtype=np.uint8)
    for i in range(0, N_MAX, unit.size):
        b[i:i + unit.size] = unit[:min(unit.size, N_MAX - i)]
    del unit
    d_b = _dev(b)
    for n, paths in ((N_MAX, (None, SINGLE_PASS)), (N_MAX - 4093, (None,))):
        _say("max lexer: oracle", n)
        r = oracle.lex_restart(b[:n], d)
        for path in paths:
            _say("max lexer: gpu", n, path, r["n_tokens"])
            g = ppr.Lexer(T, max_n=n, capacity=r["n_tokens"], path=path)(d_b[:n])
            assert g.path == (path or auto_path(n))
            _same(g, r, ("max", n, path))
            del g
            torch.cuda.empty_cache()
        del r
    del b, d_b
