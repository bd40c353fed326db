"""Pins of the lexer oracles.

* hand-worked token streams (tests/golden/lex_examples.jsonl);
* the toy grammar's closure size, k = 12, counted by hand;
* the table-driven fold over tables written from the definition equals the
  restart lexer on every input up to a length over one byte per byte class,
  and on random streams (a wrong composition order, a wrong flag rule or a
  dropped identity case breaks this);
* the same equality and the table laws on seeded random token DFAs (3 to 6
  states, 3 to 8 byte classes);
* the restart lexer reproduces the generator's own token sequence on the
  40-rule grammar's synthetic streams.
"""
import itertools
import json
import os
import random

import numpy as np
import pytest

import oracle
import workloads as W
from oracle import lex_closure
from workloads import lexgrammar as G

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lex_examples.jsonl")


def _np_tables(t):
    return (np.array(t["initial_state"], dtype=np.uint16), np.array(t["merge_table"], dtype=np.uint16),
            np.array(t["final_states"], dtype=np.uint16), t["k"])


def _named(r, d):
    return [(d["kind_names"][int(r["kind"][i])], int(r["start"][i]), int(r["length"][i]))
            for i in range(r["n_tokens"])]


def test_golden_examples():
    dfas = {"toy": W.toy_dfa(), "lexer": W.lexer_dfa()}
    cases = [json.loads(line) for line in open(GOLDEN)]
    for c in cases:
        d = dfas[c["grammar"]]
        r = oracle.lex_restart(c["input"].encode(), d)
        assert _named(r, d) == [tuple(t) for t in c["tokens"]], c


def test_toy_closure_size():
    t = lex_closure.build_tables(W.toy_dfa())
    assert t["k"] == 12


def _byte_classes(d):
    """one representative byte per distinct column of delta"""
    seen, reps = set(), []
    for b in range(256):
        col = tuple(int(x) for x in d["delta"][:, b])
        if col not in seen:
            seen.add(col)
            reps.append(b)
    return bytes(reps)


def _small_grammar():
    esc = G.Cat(G.lit("\\"), G.Set(b'"n'))
    rules = [
        ("WS", G.plus(G.Set(b" \n"))),
        ("COMMENT", G.Cat(G.lit("//"), G.Star(G.anybut("\n")))),
        ("IDENT", G.plus(G.Set(G.rng("a", "c")))),
        ("INT", G.plus(G.Set(G.rng("0", "2")))),
        ("STRING", G.Cat(G.lit('"'), G.Star(G.Alt(G.anybut('"\\\n'), esc)), G.lit('"'))),
        ("OP/", G.lit("/")),
        ("OP=", G.lit("=")),
        ("OP==", G.lit("==")),
    ]
    return G.compile_rules(rules)


@pytest.mark.parametrize("which,max_len", [("toy", 7), ("small", 5)])
def test_fold_equals_restart_exhaustive(which, max_len):
    d = W.toy_dfa() if which == "toy" else _small_grammar()
    t = _np_tables(lex_closure.build_tables(d))
    reps = _byte_classes(d)
    count = 0
    for L in range(max_len + 1):
        for s in itertools.product(reps, repeat=L):
            s = bytes(s)
            a = oracle.lex_restart(s, d)
            b = oracle.lex_fold(s, *t)
            assert _named(a, d) == _named(b, d), s
            count += 1
    assert count == sum(len(reps) ** L for L in range(max_len + 1))


def test_fold_equals_restart_random():
    d = _small_grammar()
    t = _np_tables(lex_closure.build_tables(d))
    rng = random.Random(3)
    alphabet = b' \n/abc012"\\n=x#'
    for _ in range(300):
        s = bytes(rng.choice(alphabet) for _ in range(rng.randrange(0, 300)))
        a = oracle.lex_restart(s, d)
        b = oracle.lex_fold(s, *t)
        assert _named(a, d) == _named(b, d)


def test_table_laws_small_grammar():
    """identity is neutral on both sides and the table is associative (flag bits
    masked off), so any scan order gives the fold's prefixes"""
    t = lex_closure.build_tables(_small_grammar())
    M = np.array(t["merge_table"], dtype=np.int64)
    k, ID = t["k"], 0x7FFF
    rows = np.arange(k)
    assert np.array_equal(M[rows, 0] & ID, rows) and np.array_equal(M[0, rows] & ID, rows)
    rng = np.random.default_rng(0)
    a, b, c = rng.integers(0, k, (3, 20000))
    assert np.array_equal(M[M[a, b] & ID, c], M[a, M[b, c] & ID])


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_restart_reproduces_generator_tokens(seed):
    d = W.lexer_dfa()
    for n in (0, 1, 2, 100, 1 << 18):
        b, truth = W.gen_tokens(seed, n, truth=True)
        r = oracle.lex_restart(b, d)
        assert r["n_tokens"] == truth["n_tokens"]
        assert np.array_equal(r["kind"], truth["kind"])
        assert np.array_equal(r["start"], truth["start"])
        assert np.array_equal(r["length"], truth["length"])
        assert not np.any(r["kind"] == 0), "synthetic streams hold no ERROR tokens"


# seeded random token DFAs: (seed, states, byte classes, share of undefined moves)
RANDOM_DFAS = [(2, 4, 3, 0.3), (3, 5, 3, 0.4), (4, 4, 5, 0.2), (5, 6, 3, 0.5), (6, 3, 8, 0.3), (7, 5, 4, 0.3)]


@pytest.mark.parametrize("seed,Q,m,p", RANDOM_DFAS)
def test_fold_equals_restart_random_dfas(seed, Q, m, p):
    """on random DFAs of several sizes the closure's tables, folded, give the
    restart lexer's tokens: on every input up to 4 bytes over one byte per
    class, and on random byte streams"""
    d = W.random_token_dfa(seed, Q, m, p)
    t = _np_tables(lex_closure.build_tables(d))
    reps = _byte_classes(d)
    for L in range(5):
        for s in itertools.product(reps, repeat=L):
            s = bytes(s)
            a, b = oracle.lex_restart(s, d), oracle.lex_fold(s, *t)
            assert _named(a, d) == _named(b, d), (seed, s)
    rng = np.random.default_rng(seed)
    for _ in range(40):
        s = rng.integers(0, 256, int(rng.integers(0, 2000)), dtype=np.uint8).tobytes()
        a, b = oracle.lex_restart(s, d), oracle.lex_fold(s, *t)
        assert _named(a, d) == _named(b, d), seed


@pytest.mark.parametrize("seed,Q,m,p", RANDOM_DFAS[:3])
def test_table_laws_random_dfas(seed, Q, m, p):
    t = lex_closure.build_tables(W.random_token_dfa(seed, Q, m, p))
    M = np.array(t["merge_table"], dtype=np.int64)
    k, ID = t["k"], 0x7FFF
    rows = np.arange(k)
    assert np.array_equal(M[rows, 0] & ID, rows) and np.array_equal(M[0, rows] & ID, rows)
    rng = np.random.default_rng(seed)
    a, b, c = rng.integers(0, k, (3, 5000))
    assert np.array_equal(M[M[a, b] & ID, c], M[a, M[b, c] & ID])


def test_identity_byte_clears_flag():
    """hand-worked: 'b' keeps every state and ends no token, so its element has
    the identity's maps but is not the empty string: after "aa" (a token ends
    before the second 'a') the 'b' continues the second token"""
    delta = np.full((2, 256), -1, dtype=np.int16)
    delta[0, ord("a")], delta[0, ord("b")], delta[1, ord("b")] = 1, 0, 1
    delta[0, :][delta[0, :] < 0] = 0  # the start row is total
    d = {"n_states": 2, "q0": 0, "delta": delta, "kind": np.array([0, 1], dtype=np.uint16),
         "kind_names": ("ERROR", "A")}
    want = [("A", 0, 1), ("A", 1, 2)]
    assert _named(oracle.lex_restart(b"aab", d), d) == want
    t = lex_closure.build_tables(d)
    assert _named(oracle.lex_fold(b"aab", *_np_tables(t)), d) == want
