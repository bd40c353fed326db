"""GPU parity of ppr_lex on seeded random token DFAs and on tables not built by
the library.

* random DFAs of 3 to 8 states and 2 to 8 byte classes (closures of k = 60 to
  about 8,000 identifiers), through the library's table builder, on both
  kernels and several chunk sizes;
* the same DFAs' tables written by the oracle's closure (oracle/lex_closure.py)
  and handed to LexTables(...) directly;
* closures of more than 4096 identifiers: random DFAs (their minimal automaton
  is small and steps from LDS) and a 120-byte keyword chain (k = 7264, a
  minimal automaton of 122 states x 121 columns, too large for LDS, so that the
  single-pass kernel steps the fold table and reads the final-state table from
  global memory);
* tables naming an identifier at or beyond k are rejected (PPR_EINVAL);
* grammars of 64 and 65 byte columns, either side of the streaming kernels'
  limit (their column table holds each column times 4 in a byte).

Expected tokens: the restart lexer over the DFA ("Lexing on the GPU: the scan
is the easy part", "A lexer is a prefix scan"; no table is involved on that
side). Bit-exact on (kind, start, length) and the token count.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle import lex_closure

pytestmark = pytest.mark.gpu

STREAMING, SINGLE_PASS = 1, 2
# (seed, states, byte classes, share of undefined moves)
SMALL = [(2, 4, 3, 0.3), (3, 5, 3, 0.4), (4, 4, 5, 0.2), (5, 6, 3, 0.5), (6, 3, 8, 0.3), (7, 5, 4, 0.3),
         (11, 7, 3, 0.2), (17, 6, 4, 0.1)]
LARGE = [(14, 8, 3, 0.1), (18, 8, 2, 0.1)]  # closures of 7354 and 7927 identifiers
LDS_STEP = 48 << 10  # minimal automata up to this size are stepped from LDS
LDS_KINDS = 4096     # final-state tables up to this many entries are read from LDS


@pytest.fixture(scope="module")
def ppr():
    import torch
    assert torch.cuda.is_available()
    import dfa_parsing_delimiter_amd as m
    return m


def _dev(b):
    import torch
    return torch.from_numpy(np.array(np.frombuffer(bytes(b), np.uint8), copy=True)).to("cuda")


def _same(g, r, what):
    assert g.n_tokens == r["n_tokens"], (what, g.n_tokens, r["n_tokens"])
    for key in ("kind", "start", "length"):
        a = getattr(g, key).cpu().numpy().view(np.uint32)
        if not np.array_equal(a, r[key]):
            bad = np.nonzero(a != r[key])[0]
            raise AssertionError("%s %s differs at %d of %d (first %d: gpu %d oracle %d)" % (
                what, key, bad.size, a.size, bad[0], a[bad[0]], r[key][bad[0]]))


def _inputs(d, seed):
    """random bytes, and bytes drawn from a few classes only (long tokens), with ragged sizes"""
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 256, (1 << 20) + 333, dtype=np.uint8).tobytes()
    cols = np.unique(d["delta"][0], return_index=True)[1][:3]  # a byte of each of three start-row classes
    b = rng.choice(cols.astype(np.uint8), (1 << 19) + 77).tobytes()
    return [a, b, a[:5000], b""]


def _run(ppr, T, d, seed, paths):
    for j, b in enumerate(_inputs(d, seed)):
        r = oracle.lex_restart(b, d)
        for chunk, path in paths:
            print("random dfa", seed, "input", j, len(b), chunk, path, flush=True)
            x = _dev(b) if b else _dev(b"\0")[:0]
            g = ppr.lex(x, T, chunk_bytes=chunk, capacity=len(b) + 1, path=path)
            _same(g, r, (seed, j, chunk, path))


PATHS = [(None, None), (None, STREAMING), (None, SINGLE_PASS), (7, None), (32, None)]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "seed%d" % c[0])
def test_random_dfas_library_tables(ppr, case):
    seed, Q, m, p = case
    d = W.random_token_dfa(seed, Q, m, p)
    _run(ppr, ppr.LexTables.from_dfa(d), d, seed, PATHS)


@pytest.mark.parametrize("case", SMALL[:6], ids=lambda c: "seed%d" % c[0])
def test_random_dfas_closure_tables(ppr, case):
    """tables written by the oracle's closure, passed to LexTables(...) as arrays"""
    seed, Q, m, p = case
    d = W.random_token_dfa(seed, Q, m, p)
    t = lex_closure.build_tables(d)
    T = ppr.LexTables(np.array(t["initial_state"], dtype=np.uint16), np.array(t["merge_table"], dtype=np.uint16),
                      np.array(t["final_states"], dtype=np.uint16), t["k"], t["identity"])
    _run(ppr, T, d, seed, [(None, None), (None, SINGLE_PASS), (13, None)])


@pytest.mark.parametrize("case", LARGE, ids=lambda c: "seed%d" % c[0])
def test_large_random_closures(ppr, case):
    seed, Q, m, p = case
    d = W.random_token_dfa(seed, Q, m, p)
    T = ppr.LexTables.from_dfa(d)
    assert T.k > LDS_KINDS
    _run(ppr, T, d, seed, [(None, None), (None, SINGLE_PASS), (16, None)])


def test_keyword_chain_final_states_from_global(ppr):
    d, word = W.keyword_chain_dfa(120, 5)
    T = ppr.LexTables.from_dfa(d)
    nq, m = int(T.prep.n_states), int(T.prep.m)
    assert T.k > LDS_KINDS
    # the minimal automaton does not fit LDS, so the kernel steps the fold table
    # and reads the final-state table from global memory
    assert nq == 0 or nq * m * 4 + nq * 2 > LDS_STEP, (nq, m)
    rng = np.random.default_rng(9)
    parts = []
    for _ in range(20000):  # keyword prefixes and pieces of the keyword, whole keywords, stray bytes
        i = int(rng.integers(0, len(word)))
        j = int(rng.integers(i, len(word) + 1))
        parts.append(word[:j] if rng.random() < 0.5 else word[i:j])
        if rng.random() < 0.3:
            parts.append(bytes([int(rng.integers(0, 256))]))
    for b in (b"".join(parts), rng.integers(0, 256, 300001, dtype=np.uint8).tobytes()):
        r = oracle.lex_restart(b, d)
        for chunk, path in [(None, None), (None, SINGLE_PASS), (5, None), (64, None)]:
            print("keyword chain", len(b), chunk, path, flush=True)
            g = ppr.lex(_dev(b), T, chunk_bytes=chunk, capacity=len(b) + 1, path=path)
            assert g.path == SINGLE_PASS  # (no fold rows for the streaming kernels)
            _same(g, r, ("chain", len(b), chunk, path))


def test_prepare_rejects_identifiers_out_of_range(ppr):
    d = W.random_token_dfa(2, 4, 3, 0.3)
    t = lex_closure.build_tables(d)
    k = t["k"]
    init = np.array(t["initial_state"], dtype=np.uint16)
    merge = np.array(t["merge_table"], dtype=np.uint16)
    fin = np.array(t["final_states"], dtype=np.uint16)
    ppr.LexTables(init, merge, fin, k, 0)  # the tables as built are accepted
    for r, c, v in [(3, 5, k), (k - 1, k - 1, k + 7), (1, 0, 0x7fff), (2, 2, 0x8000 | k)]:
        bad = merge.copy()
        bad[r, c] = v
        with pytest.raises(ppr.PprError) as e:
            ppr.LexTables(init, bad, fin, k, 0)
        assert e.value.code == ppr.PPR_EINVAL, (r, c, v)
    bad_init = init.copy()
    bad_init[ord("x")] = k
    with pytest.raises(ppr.PprError) as e:
        ppr.LexTables(bad_init, merge, fin, k, 0)
    assert e.value.code == ppr.PPR_EINVAL
    with pytest.raises(ppr.PprError) as e:
        ppr.LexTables(init, merge, fin, k, k)  # identity beyond k
    assert e.value.code == ppr.PPR_EINVAL


@pytest.mark.parametrize("n_cols", [64, 65])
def test_column_limit_of_streaming_kernels(ppr, n_cols):
    """64 byte columns (the largest column times 4 is 252) run on the streaming kernels; 65 fall back to the
    single-pass kernel, on the automatic path and when the streaming kernels are asked for; the same tokens"""
    d = W.many_columns_dfa(n_cols)
    T = ppr.LexTables.from_dfa(d)
    assert int(T.prep.m) == n_cols
    assert (int(T.prep.n_rows) > 0) == (n_cols <= 64), (n_cols, int(T.prep.n_rows))
    want = STREAMING if n_cols <= 64 else SINGLE_PASS
    rng = np.random.default_rng(n_cols)
    b = rng.integers(0, 256, (9 << 20) + 123, dtype=np.uint8).tobytes()  # above the automatic threshold
    r = oracle.lex_restart(b, d)
    x = _dev(b)
    for path in (None, STREAMING):
        print("columns", n_cols, "path", path, r["n_tokens"], flush=True)
        g = ppr.lex(x, T, capacity=len(b) + 1, path=path)
        assert g.path == want, (n_cols, path, g.path)
        _same(g, r, (n_cols, path))
