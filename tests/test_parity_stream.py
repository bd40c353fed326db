"""GPU parity of parsing in partitions (the resumable parse and the host
streaming driver) against one oracle run over the whole input.

ParPaRaw's end-to-end streaming passage cuts the input into partitions that
are transferred, parsed and returned in turn. Here a partition's parse
continues the previous one (PPR_PARSE_CONTINUE: its end state and open
column; PPR_PARSE_PARTIAL: its open field is left to the next), and
ppr_parse_stream drives that over host memory. Both must give exactly the
fields and scalars of a single parse: bit-exact against the oracle, with cut
points anywhere (inside quoted fields, at delimiters, inside multi-partition
fields), on every parse path, on invalid input and on a non-accepting end.
"""
import ctypes

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


def _say(*a):
    print(*a, flush=True)


def _same_stream(g, r, what, u64=True):
    assert (g.n_fields, g.n_records, g.error_pos, g.end_state, g.min_columns, g.max_columns, g.bad_records,
            g.first_bad_record) == (r["n_fields"], r["n_records"], r["error_pos"], r["end_state"], r["min_columns"],
                                    r["max_columns"], r["bad_records"], r["first_bad_record"]), (
        what, g.n_fields, r["n_fields"], g.n_records, r["n_records"], g.error_pos, r["error_pos"], g.end_state,
        r["end_state"], g.min_columns, r["min_columns"], g.max_columns, r["max_columns"], g.bad_records,
        r["bad_records"], g.first_bad_record, r["first_bad_record"])
    for name, key in (("record_idx", "rec"), ("column_ids", "col"), ("field_offsets", "off"),
                      ("field_lengths", "len")):
        a = np.asarray(getattr(g, name)).astype(np.uint64)
        b = r[key].astype(np.uint64)
        if not np.array_equal(a, b):
            bad = np.nonzero(a != b)[0]
            raise AssertionError("%s %s differs at %d of %d (first %d: gpu %d oracle %d)" % (
                what, name, bad.size, a.size, bad[0], a[bad[0]], b[bad[0]]))


def _pieces_parse(ppr, b, t, cuts, chunk=None, path=None, expect=0):
    """parse b in pieces [cuts[i], cuts[i+1]) with the resumable ABI and compose the results on the host the way
    one parse numbers them: record indices and offsets shifted, the first field of a piece started where the
    field left open by the previous piece started"""
    import torch
    P = ppr.Parser(t, max_n=max(1, max(c1 - c0 for c0, c1 in zip(cuts, cuts[1:]))), capacity=len(b) + 2,
                   chunk_bytes=chunk, path=path, expected_columns=expect)
    state, col, open_start, rec_base = t["start"], 0, 0, 0
    parts = {k: [] for k in ("rec", "col", "off", "len")}
    err, fbad, bad, cmin, cmax, paths = -1, -1, 0, None, 0, set()
    for i, (c0, c1) in enumerate(zip(cuts, cuts[1:])):
        last = i == len(cuts) - 2
        P.opts.flags = (ppr.PPR_PARSE_CONTINUE if i else 0) | (0 if last else ppr.PPR_PARSE_PARTIAL)
        P.opts.start_state, P.opts.start_column = (state, col) if i else (0, 0)
        piece = np.ascontiguousarray(b[c0:c1])
        d = torch.from_numpy(piece).cuda() if piece.size else torch.zeros(0, dtype=torch.uint8, device="cuda")
        g = P(d)
        paths.add(g.path)
        nf = g.n_fields
        rec = g.record_idx.cpu().numpy().view(np.uint32).astype(np.uint64) + rec_base
        off = g.field_offsets.cpu().numpy().view(np.uint32).astype(np.uint64) + c0
        ln = g.field_lengths.cpu().numpy().view(np.uint32).astype(np.uint64)
        if nf:
            ln[0] += c0 - open_start
            off[0] = open_start
        parts["rec"].append(rec)
        parts["col"].append(g.column_ids.cpu().numpy().view(np.uint32))
        parts["off"].append(off)
        parts["len"].append(ln)
        if err < 0 and g.error_pos >= 0:
            err = c0 + g.error_pos
        if fbad < 0 and g.first_bad_record >= 0:
            fbad = rec_base + g.first_bad_record
        bad += g.bad_records
        if g.n_records:
            cmin = g.min_columns if cmin is None else min(cmin, g.min_columns)
            cmax = max(cmax, g.max_columns)
        # the carry for the next piece (read back through ppr_parse_results: tail of this piece)
        o = P.results(piece.size)
        if nf:
            open_start = c0 + o.tail_start
        rec_base += g.n_records
        state, col = g.end_state, o.tail_column
    res = {k: np.concatenate(v) if v else np.zeros(0, np.uint64) for k, v in parts.items()}

    class R:
        pass
    out = R()
    out.record_idx, out.column_ids, out.field_offsets, out.field_lengths = res["rec"], res["col"], res["off"], res["len"]
    out.n_fields, out.n_records, out.error_pos, out.end_state = res["rec"].size, rec_base, err, state
    out.min_columns, out.max_columns, out.bad_records, out.first_bad_record = cmin or 0, cmax, bad, fbad
    return out, paths


def _cases():
    t5, t6 = W.table("T5"), W.table("T6")
    c3 = W.generate(3, n=(3 << 20) + 101, seed=41)
    c1 = W.generate(1, n=(1 << 20) + 7, seed=42)
    c4 = W.generate(4, n=(2 << 20) + 3, seed=43)
    bad = c3.copy()
    bad[2_000_003:2_000_006] = np.frombuffer(b'q"z', np.uint8)   # an INVALID byte deep inside
    open_end = np.concatenate([c1, np.frombuffer(b'\n"never closed,\n', np.uint8)])  # non-accepting end
    return [("c3", c3, t5, 12), ("c1", c1, t5, 8), ("c4", c4, t6, 512), ("invalid", bad, t5, 12),
            ("open_end", open_end, t5, 8)]


@pytest.mark.parametrize("chunk,path", [(None, 3), (None, 1), (31, None)])
def test_resumable_pieces(ppr, chunk, path):
    """the resumable ABI by itself: pieces cut at random places (and at 0-byte and 1-byte pieces), composed on the
    host, equal one parse; on the fused, streaming and generic kernels"""
    rng = np.random.default_rng(7)
    for name, b, t, expect in _cases():
        n = b.size
        cuts = sorted(set([0, n] + [int(x) for x in rng.integers(0, n, 6)] + [n // 2, n // 2 + 1, n // 2 + 1]))
        cuts = [0] + [c for c in cuts if 0 < c < n] + [n]
        cuts.insert(2, cuts[1])  # an empty piece
        r = oracle.csv_parse(b, t, expected_columns=expect)
        _say("pieces", name, n, len(cuts) - 1, chunk, path)
        g, paths = _pieces_parse(ppr, b, t, cuts, chunk, path, expect)
        _same_stream(g, r, (name, chunk, path, cuts))


@pytest.mark.parametrize("pb", [100, 4099, 65536, (1 << 20) + 13, 8 << 20])
def test_stream_driver(ppr, pb):
    """ppr_parse_stream over host memory: partitions of 100 bytes (thousands of them, fields spanning many) up to
    larger than the input"""
    for name, b, t, expect in _cases():
        r = oracle.csv_parse(b, t, expected_columns=expect)
        _say("stream", name, b.size, pb)
        g = ppr.parse_stream(b, t, pb, expected_columns=expect)
        assert g.partitions == max(1, -(-b.size // pb))
        _same_stream(g, r, (name, pb))


def test_stream_edges(ppr):
    """empty input, one byte, an input ending exactly at a partition boundary on a record delimiter, a field
    longer than many partitions, capacity too small (the counts are still reported), a pageable output"""
    import torch
    t = W.table("T5")
    cases = [b"", b"x", b"a,b\n" * 25, b"q" * 5000 + b",z", b'"' + b"a\n," * 3000 + b'"\n1,2']
    for b in cases:
        for pb in (1, 7, 100):
            r = oracle.csv_parse(b, t)
            g = ppr.parse_stream(np.frombuffer(b, np.uint8), t, pb)
            _same_stream(g, r, (b[:20], pb))
    b = W.generate(1, n=200000, seed=3)
    r = oracle.csv_parse(b, t)
    dfa, cm = ppr.make_dfa(t)
    o = ppr.StreamOut()
    arrs = [np.zeros(100, np.uint64), np.zeros(100, np.uint32), np.zeros(100, np.uint64), np.zeros(100, np.uint64)]
    o.record_idx, o.column_ids, o.field_offsets, o.field_lengths = [a.ctypes.data for a in arrs]
    o.cap_fields = 100
    rc = ppr.lib.ppr_parse_stream(b.ctypes.data, b.size, ctypes.byref(dfa), cm, ctypes.byref(o), 7000, None)
    assert rc == ppr.PPR_ECAPACITY and o.n_fields == r["n_fields"] and o.n_records == r["n_records"]
    assert np.array_equal(arrs[2], r["off"][:100].astype(np.uint64))
    g = ppr.parse_stream(b, t, 7000, pinned=False)
    _same_stream(g, r, "pageable")
    with pytest.raises(ppr.PprError):
        ppr.parse_stream(b, t, 0)
