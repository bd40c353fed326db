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


def test_golden(ppr, tables):
    for line in open(GOLDEN):
        c = json.loads(line)
        d, T = tables[c["grammar"]]
        b = c["input"].encode()
        for chunk in (1, 2, 32, None):
            _say("golden", repr(b), chunk)
            g = ppr.lex(_dev(b), T, chunk_bytes=chunk, capacity=len(b) + 1)
            _same(g, oracle.lex_restart(b, d), (b, chunk))


@pytest.mark.parametrize("chunk", [1, 3, 16, 31, 32, 40, 64])
def test_streams_several_tiles(ppr, tables, chunk):
    d, T = tables["lexer"]
    for seed in (1, 2):
        n = (2 << 20) + 777 * seed
        b = W.gen_tokens(seed, n)
        _say("stream", chunk, seed, n)
        g = ppr.lex(_dev(b), T, chunk_bytes=chunk, capacity=n + 1)
        _same(g, oracle.lex_restart(b, d), (chunk, seed))


def test_random_bytes_and_edges(ppr, tables):
    d, T = tables["lexer"]
    rng = np.random.default_rng(4)
    cases = [b"", b"a", b"@", b"//" + b"x" * 70000, b'"' + b"q" * 70001, b" " * 100000, b"1." * 30000]
    cases += [rng.integers(0, 256, int(rng.integers(1, 50000)), dtype=np.uint8).tobytes() for _ in range(6)]
    for b in cases:
        for chunk in (1, 7, 32, None):
            _say("edge", len(b), chunk)
            g = ppr.lex(_dev(b) if b else _dev(b"\0")[:0], T, chunk_bytes=chunk, capacity=len(b) + 1)
            _same(g, oracle.lex_restart(b, d), (len(b), chunk))


def test_minimal_automaton_and_identifier_fold(ppr, tables):
    """the second pass steps the minimal automaton of the fold when the prepared tables hold one, and re-folds
    the identifiers otherwise; both against the oracle"""
    d, T = tables["lexer"]
    assert 0 < T.prep.n_states <= T.k, T.prep.n_states
    b = W.gen_tokens(3, (1 << 20) + 5)
    r = oracle.lex_restart(b, d)
    _same(ppr.lex(_dev(b), T, capacity=b.size + 1), r, "minimal automaton")
    saved = T.prep.n_states
    T.prep.n_states = 0
    try:
        _same(ppr.lex(_dev(b), T, capacity=b.size + 1), r, "identifier fold")
    finally:
        T.prep.n_states = saved


@pytest.mark.slow
def test_full_size_lexer_workload(ppr, tables):
    d, T = tables["lexer"]
    _say("full lexer: generate")
    b = W.generate(5)
    _say("full lexer: oracle")
    r = oracle.lex_restart(b, d)
    _say("full lexer: gpu", r["n_tokens"])
    g = ppr.Lexer(T, max_n=b.size, capacity=r["n_tokens"])(_dev(b))
    _same(g, r, "full")
