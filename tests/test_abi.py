"""C ABI checks that need no GPU: the library loads, exports every function
include/ppr.h declares, rejects bad arguments before touching the device, and
its host-side lexer table builder agrees with the oracles."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads as W
from oracle import lex_closure

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "ppr.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:PPR_API\s+)?(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(ppr_[a-z_]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    import dfa_parsing_delimiter_amd as ppr
    names = _declared_functions()
    assert names == sorted(["ppr_parse_workspace_bytes", "ppr_parse", "ppr_parse_async", "ppr_parse_results",
                            "ppr_lex_fold_bytes", "ppr_lex_prepare", "ppr_lex_workspace_bytes", "ppr_lex",
                            "ppr_lex_async", "ppr_lex_results", "ppr_lex_build_tables", "ppr_version",
                            "ppr_bandwidth_probe", "ppr_parse_noalloc", "ppr_parse_stream", "ppr_columns",
                            "ppr_columns_workspace_bytes", "ppr_numbers_workspace_bytes", "ppr_infer_types",
                            "ppr_convert"]), names
    for nm in names:
        assert hasattr(ppr.lib, nm), nm
    assert "gfx950" in ppr.version()


def test_workspace_sizes():
    import dfa_parsing_delimiter_amd as ppr
    L = ppr.lib
    o = ppr.ParseOpts()
    assert L.ppr_parse_workspace_bytes(0, ctypes.byref(o)) >= 256
    o.chunk_bytes = 65
    assert L.ppr_parse_workspace_bytes(1000, ctypes.byref(o)) == 0
    o.chunk_bytes = 31
    ws = L.ppr_parse_workspace_bytes(1 << 30, ctypes.byref(o))
    tiles = -(-(1 << 30) // (1024 * 31))  # single-pass tiles: 1024 threads x 31 bytes
    assert ws >= 256 + tiles * 72
    assert L.ppr_parse_workspace_bytes(1 << 32, ctypes.byref(o)) == 0
    # the largest input of one call: 2^32 - 2^16 bytes (positions up to the last tile's end fit 32 bits)
    assert L.ppr_parse_workspace_bytes((1 << 32) - (1 << 16) + 1, ctypes.byref(o)) == 0
    assert L.ppr_parse_workspace_bytes((1 << 32) - (1 << 16), ctypes.byref(o)) > 0
    o.chunk_bytes = 0
    assert L.ppr_lex_workspace_bytes((1 << 32) - (1 << 16) + 1, ctypes.byref(o)) == 0
    assert L.ppr_lex_workspace_bytes((1 << 32) - (1 << 16), ctypes.byref(o)) > 0


def _call_parse(table, n=10, cm=None, chunk=0):
    import dfa_parsing_delimiter_amd as ppr
    d, cmap = ppr.make_dfa(table)
    out = ppr.ParseOut()
    opts = ppr.ParseOpts()
    opts.chunk_bytes = chunk
    # fake, never-dereferenced device pointers: validation happens first
    return ppr.lib.ppr_parse_async(ctypes.c_void_p(4096), n, ctypes.byref(d), cm if cm is not None else cmap,
                                   ctypes.byref(out), ctypes.c_void_p(4096), 1 << 20, ctypes.byref(opts), None)


def test_bad_tables_rejected_on_host():
    import dfa_parsing_delimiter_amd as ppr
    t = W.table("T5")
    bad = dict(t, next=[row[:] for row in t["next"]])
    bad["next"][0][0] = 7  # beyond n_states
    assert _call_parse(bad) == ppr.PPR_EINVAL
    bad = dict(t, tag=[row[:] for row in t["tag"]])
    bad["tag"][1][1] = 4
    assert _call_parse(bad) == ppr.PPR_EINVAL
    bad = dict(t, start=5)
    assert _call_parse(bad) == ppr.PPR_EINVAL
    cm = bytearray(t["class_map"])
    cm[65] = 4  # class beyond n_classes
    assert _call_parse(t, cm=bytes(cm)) == ppr.PPR_EINVAL
    assert _call_parse(t, chunk=65) == ppr.PPR_EINVAL
    assert _call_parse(t, n=1 << 32) == ppr.PPR_ETOOBIG
    assert _call_parse(t, n=(1 << 32) - (1 << 16) + 1) == ppr.PPR_ETOOBIG


def _library_tables(d):
    import dfa_parsing_delimiter_amd as ppr
    return ppr.LexTables.build_host(d)


def test_library_lexer_tables_toy_match_definition():
    d = W.toy_dfa()
    init, merge, fin, k, ident = _library_tables(d)
    ref = lex_closure.build_tables(d)
    assert k == ref["k"] == 12 and ident == 0
    # identifiers may differ between builders only by a renumbering; with the
    # same breadth-first order they coincide here
    assert np.array_equal(merge, np.array(ref["merge_table"], dtype=np.uint16))
    assert np.array_equal(init, np.array(ref["initial_state"], dtype=np.uint16))
    assert np.array_equal(fin, np.array(ref["final_states"], dtype=np.uint16))


def test_library_lexer_tables_40_rules_fold_equals_restart():
    d = W.lexer_dfa()
    init, merge, fin, k, ident = _library_tables(d)
    assert k == 2159
    for seed in (1, 2, 3):
        b = W.gen_tokens(seed, 1 << 18)
        a = oracle.lex_restart(b, d)
        f = oracle.lex_fold(b, init, merge, fin, k)
        for key in ("kind", "start", "length"):
            assert np.array_equal(a[key], f[key])
    # random bytes (errors, restarts everywhere)
    rng = np.random.default_rng(0)
    for _ in range(20):
        b = rng.integers(0, 256, rng.integers(0, 4000), dtype=np.uint8)
        a = oracle.lex_restart(b, d)
        f = oracle.lex_fold(b, init, merge, fin, k)
        assert a["n_tokens"] == f["n_tokens"]
        for key in ("kind", "start", "length"):
            assert np.array_equal(a[key], f[key])


def test_library_lexer_tables_laws():
    d = W.lexer_dfa()
    init, merge, fin, k, ident = _library_tables(d)
    M = merge.astype(np.int64)
    rows = np.arange(k)
    assert np.array_equal(M[rows, ident] & 0x7FFF, rows)
    assert np.array_equal(M[ident, rows] & 0x7FFF, rows)
    rng = np.random.default_rng(1)
    a, b, c = rng.integers(0, k, (3, 200000))
    assert np.array_equal(M[M[a, b] & 0x7FFF, c], M[a, M[b, c] & 0x7FFF])


def test_lexer_builder_rejects_bad_dfa():
    import dfa_parsing_delimiter_amd as ppr
    d = W.toy_dfa()
    delta = np.array(d["delta"], dtype=np.int16)
    delta[0, 5] = -1  # start row must be total
    kind = np.array(d["kind"], dtype=np.uint16)
    k = ctypes.c_uint32()
    rc = ppr.lib.ppr_lex_build_tables(delta.ctypes.data, kind.ctypes.data, delta.shape[0], 0, 32768, ctypes.byref(k),
                                      None, None, None, None)
    assert rc == ppr.PPR_EINVAL
    delta = np.array(d["delta"], dtype=np.int16)
    rc = ppr.lib.ppr_lex_build_tables(delta.ctypes.data, kind.ctypes.data, delta.shape[0], 0, 5, ctypes.byref(k),
                                      None, None, None, None)
    assert rc == ppr.PPR_ECAPACITY and k.value == 6


def test_struct_layouts_match_header(tmp_path):
    """the ctypes mirrors of the C structs have the header's sizes and field offsets (gcc reads the header)"""
    import subprocess
    import dfa_parsing_delimiter_amd as ppr
    structs = {"ppr_dfa_t": ppr.Dfa, "ppr_parse_out_t": ppr.ParseOut, "ppr_parse_opts_t": ppr.ParseOpts,
               "ppr_lex_tables_t": ppr.LexTablesC, "ppr_lex_prepared_t": ppr.LexPrepared,
               "ppr_tokens_out_t": ppr.TokensOut}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "ppr.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append('printf("%s size %%zu\\n", sizeof(%s));' % (cname, cname))
        for f, _ in py._fields_:
            lines.append('printf("%s %s %%zu\\n", offsetof(%s, %s));' % (cname, f, cname, f))
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)
