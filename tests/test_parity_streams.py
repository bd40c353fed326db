"""GPU parity with calls in flight on several streams at once.

Two CSV parses (the streaming kernels on the quote-heavy recipe, the fused
kernel on the tiny recipe) and one lexer call are enqueued without waiting
(ppr_parse_async / ppr_lex_async), each on its own stream with its own
workspace, so that their kernels can run at the same time; then the same three
calls again, each on the stream of another. Every result must equal the
oracle's: the library keeps no state between calls outside the workspace the
caller passes, so concurrent calls must not interfere.
"""
import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ppr():
    import torch
    assert torch.cuda.is_available()
    import dfa_parsing_delimiter_amd as m
    return m


def _np(t, k):
    return t[:k].cpu().numpy().view(np.uint32)


def _check_parse(P, o, r, what):
    assert int(o.n_fields) == r["n_fields"], (what, int(o.n_fields), r["n_fields"])
    assert int(o.n_records) == r["n_records"], what
    assert int(o.error_pos) == r["error_pos"], what
    k = r["n_fields"]
    for a, key in zip(P.out_arrays, ("rec", "col", "off", "len")):
        assert np.array_equal(_np(a, k), r[key]), (what, key)


def _check_lex(L, o, r, what):
    assert int(o.n_tokens) == r["n_tokens"], (what, int(o.n_tokens), r["n_tokens"])
    k = r["n_tokens"]
    for a, key in zip(L.out_arrays, ("kind", "start", "length")):
        assert np.array_equal(_np(a, k), r[key]), (what, key)


def test_concurrent_calls_on_three_streams(ppr):
    import torch
    t5 = W.table("T5")
    a = W.generate(3, n=48 << 20)  # streaming kernels
    b = W.generate(1)               # 1 MiB: the fused kernel
    d_lex = W.lexer_dfa()
    T = ppr.LexTables.from_dfa(d_lex)
    c = W.gen_tokens(W.seed_of(5), 24 << 20)  # streaming lexer
    ra, rb, rc = oracle.csv_parse(a, t5), oracle.csv_parse(b, t5), oracle.lex_restart(c, d_lex)
    da, db, dc = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda") for x in (a, b, c))
    streams = [torch.cuda.Stream() for _ in range(3)]  # default priority
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())  # the inputs were copied on the current stream
    Pa = ppr.Parser(t5, max_n=a.size, capacity=ra["n_fields"])
    Pb = ppr.Parser(t5, max_n=b.size, capacity=rb["n_fields"])
    L = ppr.Lexer(T, max_n=c.size, capacity=rc["n_tokens"])
    for rot in range(3):
        sa, sb, sc = streams[rot % 3], streams[(rot + 1) % 3], streams[(rot + 2) % 3]
        for x in (Pa.out_arrays + Pb.out_arrays + L.out_arrays):
            x.fill_(-1)  # (on the current stream: the launches below wait for it)
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        print("rotation", rot, flush=True)
        Pa.launch(da, sa)
        Pb.launch(db, sb)
        L.launch(dc, sc)
        torch.cuda.synchronize()
        oa, ob, oc = Pa.results(a.size, sa), Pb.results(b.size, sb), L.results(c.size, sc)
        assert int(oa.path) == ppr.PPR_PATH_STREAMING and int(ob.path) == ppr.PPR_PATH_FUSED
        assert int(oc.path) == ppr.PPR_PATH_STREAMING
        _check_parse(Pa, oa, ra, ("quote-heavy", rot))
        _check_parse(Pb, ob, rb, ("tiny", rot))
        _check_lex(L, oc, rc, ("lexer", rot))
