"""CPU oracle (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import, call, link or run anything in this package. It shares
no code, header, table or helper with the GPU library, and it never imports it.

* ``csv_parse``: one sequential DFA run over the whole input
  (csv_oracle.c; ParPaRaw, Sec. 3 and "validating format"), and the fewest and
  most fields of any record, counted from its per-field record indices
  (ParPaRaw, "Inferring or validating number of columns"); given an expected
  number of columns, the records that do not have it: how many, and the first
  (same passage, and the specialisations passage: rejecting records with an
  inconsistent number of field delimiters).
* ``lex_restart``: the restart lexer, one state variable over the bytes
  (lex_oracle.c; "Lexing on the GPU", "A lexer is a prefix scan").
* ``lex_fold``: the sequential table-driven fold over initial/merge/final
  tables (lex_oracle.c; same page, tables and harness).
* ``lex_closure.build_tables``: the merge tables written out from their
  definition with plain tuples (small grammars only).
* ``columns.partition``: the columnar partition of one parse's fields into
  per-column concatenated symbol strings and their index (ParPaRaw, Sec. 3,
  Fig. 5; inline-terminated and vector-delimited variants, Fig. 6).
* ``numbers.infer`` / ``numbers.convert``: each field's minimal numeric type
  and each column's (the maximum over its fields), and the fields' values in
  their column's type (ParPaRaw, "Type inference", "Default values for empty
  strings"; Sec. 3, conversion to the column's type).

Beside the oracle, and not part of it: ``csv_parse_parallel`` and
``lex_restart_parallel`` (cpu_parallel.c), the all-core CPU baseline that the
benchmark times: the data-parallel method on host threads, checked bit-exact
against the oracle by ``tests/test_cpu_parallel.py``.

Every function is pinned by ``tests/test_oracle_*.py`` against hand-worked
examples, exhaustive enumeration and independent readers; see those tests.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "_liboracle.so")
_SRCS = [os.path.join(_HERE, "csv_oracle.c"), os.path.join(_HERE, "lex_oracle.c"), os.path.join(_HERE, "cpu_parallel.c")]


def build(force: bool = True) -> str:
    """Compile the oracle with plain gcc -O3."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O3", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread", "-o", tmp]
                       + _SRCS, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None
_P = ctypes.c_void_p
_U64 = ctypes.c_uint64
_U32 = ctypes.c_uint32


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        L.oracle_csv_parse.argtypes = [_P, _U64, _U32, _U32, _U32, _U32, _P, _P, _P, _P, _P, _P, _P, _U64, _P, _P,
                                       _P, _P]
        L.oracle_csv_parse.restype = ctypes.c_int
        L.oracle_csv_parse_many.argtypes = [_P, _P, _U64, _U32, _U32, _U32, _U32, _P, _P, _P, _P, _P, _P, _P, _U64,
                                            _P, _P, _P, _P]
        L.oracle_csv_parse_many.restype = ctypes.c_int
        L.oracle_lex_restart.argtypes = [_P, _U64, _U32, _P, _P, _P, _P, _P, _U64, _P]
        L.oracle_lex_restart.restype = ctypes.c_int
        L.oracle_lex_fold.argtypes = [_P, _U64, _P, _P, _P, _U32, ctypes.c_uint16, _P, _P, _P, _U64, _P]
        L.oracle_lex_fold.restype = ctypes.c_int
        L.cpu_parallel_csv_parse.argtypes = [_P, _U64, _U32, _U32, _U32, _U32, _P, _P, _P, _P, _P, _P, _P, _U64,
                                             _U32, _P, _P, _P, _P, _P, _P]
        L.cpu_parallel_csv_parse.restype = ctypes.c_int
        L.cpu_parallel_lex_restart.argtypes = [_P, _U64, _U32, _U32, _P, _P, _P, _P, _P, _U64, _U32, _P]
        L.cpu_parallel_lex_restart.restype = ctypes.c_int
        _lib = L
    return _lib


def _as_u8(data) -> np.ndarray:
    if isinstance(data, (bytes, bytearray, memoryview)):
        return np.frombuffer(bytes(data), dtype=np.uint8)
    a = np.ascontiguousarray(data)
    assert a.dtype == np.uint8
    return a


def _tables(d):
    S, C = d["n_states"], d["n_classes"]
    nxt = np.array(d["next"], dtype=np.uint8).reshape(S, C)
    tag = np.array(d["tag"], dtype=np.uint8).reshape(S, C)
    cm = np.frombuffer(bytes(d["class_map"]), dtype=np.uint8)
    return np.ascontiguousarray(nxt), np.ascontiguousarray(tag), np.ascontiguousarray(cm)


def _columns(rec, n_records):
    """fewest and most fields of any record (0, 0 without records): the fields
    of record r are those whose record index is r"""
    if n_records == 0:
        return 0, 0
    per_record = np.bincount(rec.astype(np.int64), minlength=n_records)
    return int(per_record.min()), int(per_record.max())


def _conformance(rec, n_records, expected):
    """records whose number of fields is not `expected` (0: no expectation):
    how many, and the index of the first (-1: none)"""
    if not expected or n_records == 0:
        return 0, -1
    per_record = np.bincount(rec.astype(np.int64), minlength=n_records)
    bad = np.nonzero(per_record != expected)[0]
    return int(bad.size), (int(bad[0]) if bad.size else -1)


def csv_parse(data, d: dict, start_state: int | None = None, cap: int | None = None,
              expected_columns: int = 0) -> dict:
    """Sequential parse of one input under DFA table d (workloads.dfa format).
    Returns the four per-field arrays (uint32) and the scalars; with
    expected_columns > 0 also bad_records / first_bad_record (records whose
    number of fields differs from it)."""
    b = _as_u8(data)
    n = b.size
    nxt, tag, cm = _tables(d)
    cap = n + 1 if cap is None else cap
    out = {k: np.empty(cap, dtype=np.uint32) for k in ("rec", "col", "off", "len")}
    nf, nr, err, es = _U64(), _U64(), ctypes.c_int64(), _U32()
    s0 = d["start"] if start_state is None else start_state
    rc = lib().oracle_csv_parse(b.ctypes.data, n, d["n_states"], d["n_classes"], s0, d["accept_mask"],
                                nxt.ctypes.data, tag.ctypes.data, cm.ctypes.data, out["rec"].ctypes.data,
                                out["col"].ctypes.data, out["off"].ctypes.data, out["len"].ctypes.data, cap,
                                ctypes.byref(nf), ctypes.byref(nr), ctypes.byref(err), ctypes.byref(es))
    k = int(nf.value)
    if rc != 0:
        raise ValueError("oracle capacity too small: %d fields" % k)
    res = {key: v[:k] for key, v in out.items()}
    res.update(n_fields=k, n_records=int(nr.value), error_pos=int(err.value), end_state=int(es.value))
    res["min_columns"], res["max_columns"] = _columns(res["rec"], res["n_records"])
    res["bad_records"], res["first_bad_record"] = _conformance(res["rec"], res["n_records"], expected_columns)
    return res


def csv_parse_many(inputs, d: dict, expected_columns: int = 0) -> list:
    """Parse many independent inputs (each from the start state) in one call."""
    blobs = [bytes(x) for x in inputs]
    starts = np.zeros(len(blobs) + 1, dtype=np.uint64)
    np.cumsum([len(x) for x in blobs], out=starts[1:])
    b = np.frombuffer(b"".join(blobs) + b"\0", dtype=np.uint8)
    cap = int(starts[-1]) + len(blobs) + 1
    nxt, tag, cm = _tables(d)
    out = {k: np.empty(cap, dtype=np.uint32) for k in ("rec", "col", "off", "len")}
    cnt = len(blobs)
    base = np.zeros(cnt + 1, dtype=np.uint64)
    nr = np.zeros(cnt, dtype=np.uint64)
    err = np.zeros(cnt, dtype=np.int64)
    es = np.zeros(cnt, dtype=np.uint32)
    rc = lib().oracle_csv_parse_many(b.ctypes.data, starts.ctypes.data, cnt, d["n_states"], d["n_classes"],
                                     d["start"], d["accept_mask"], nxt.ctypes.data, tag.ctypes.data, cm.ctypes.data,
                                     out["rec"].ctypes.data, out["col"].ctypes.data, out["off"].ctypes.data,
                                     out["len"].ctypes.data, cap, base.ctypes.data, nr.ctypes.data, err.ctypes.data,
                                     es.ctypes.data)
    if rc != 0:
        raise ValueError("oracle capacity too small")
    res = []
    for j in range(cnt):
        lo, hi = int(base[j]), int(base[j + 1])
        r = {key: v[lo:hi] for key, v in out.items()}
        r.update(n_fields=hi - lo, n_records=int(nr[j]), error_pos=int(err[j]), end_state=int(es[j]))
        r["min_columns"], r["max_columns"] = _columns(r["rec"], r["n_records"])
        r["bad_records"], r["first_bad_record"] = _conformance(r["rec"], r["n_records"], expected_columns)
        res.append(r)
    return res


def _tok_out(cap):
    return {k: np.empty(cap, dtype=np.uint32) for k in ("kind", "start", "length")}


def lex_restart(data, d: dict) -> dict:
    """Restart lexer over the token DFA d (workloads.lexgrammar format)."""
    b = _as_u8(data)
    n = b.size
    cap = n + 1
    out = _tok_out(cap)
    delta = np.ascontiguousarray(d["delta"], dtype=np.int16)
    kind = np.ascontiguousarray(d["kind"], dtype=np.uint16)
    nt = _U64()
    rc = lib().oracle_lex_restart(b.ctypes.data, n, d["q0"], delta.ctypes.data, kind.ctypes.data,
                                  out["kind"].ctypes.data, out["start"].ctypes.data, out["length"].ctypes.data, cap,
                                  ctypes.byref(nt))
    k = int(nt.value)
    assert rc == 0
    res = {key: v[:k] for key, v in out.items()}
    res["n_tokens"] = k
    return res


def lex_fold(data, initial_state, merge_table, final_states, k: int, flag_mask: int = 0x8000) -> dict:
    """Sequential fold over lexer tables (any builder's)."""
    b = _as_u8(data)
    n = b.size
    cap = n + 1
    out = _tok_out(cap)
    init = np.ascontiguousarray(initial_state, dtype=np.uint16).reshape(256)
    merge = np.ascontiguousarray(merge_table, dtype=np.uint16).reshape(k * k)
    fin = np.ascontiguousarray(final_states, dtype=np.uint16).reshape(k)
    nt = _U64()
    rc = lib().oracle_lex_fold(b.ctypes.data, n, init.ctypes.data, merge.ctypes.data, fin.ctypes.data, k, flag_mask,
                               out["kind"].ctypes.data, out["start"].ctypes.data, out["length"].ctypes.data, cap,
                               ctypes.byref(nt))
    kk = int(nt.value)
    assert rc == 0
    res = {key: v[:kk] for key, v in out.items()}
    res["n_tokens"] = kk
    return res


def csv_parse_parallel(data, d: dict, threads: int, cap: int | None = None) -> dict:
    """The all-core CPU baseline (not the oracle): csv_parse's result, computed
    by the data-parallel method on `threads` host threads."""
    b = _as_u8(data)
    n = b.size
    nxt, tag, cm = _tables(d)
    cap = n + 1 if cap is None else cap
    out = {k: np.empty(cap, dtype=np.uint32) for k in ("rec", "col", "off", "len")}
    nf, nr, err, es, cmin, cmax = _U64(), _U64(), ctypes.c_int64(), _U32(), _U32(), _U32()
    rc = lib().cpu_parallel_csv_parse(b.ctypes.data, n, d["n_states"], d["n_classes"], d["start"], d["accept_mask"],
                                      nxt.ctypes.data, tag.ctypes.data, cm.ctypes.data, out["rec"].ctypes.data,
                                      out["col"].ctypes.data, out["off"].ctypes.data, out["len"].ctypes.data, cap,
                                      threads, ctypes.byref(nf), ctypes.byref(nr), ctypes.byref(err),
                                      ctypes.byref(es), ctypes.byref(cmin), ctypes.byref(cmax))
    k = int(nf.value)
    if rc == -1:
        raise ValueError("cpu_parallel_csv_parse: invalid table or thread count")
    res = {key: v[:min(k, cap)] for key, v in out.items()}
    res.update(n_fields=k, n_records=int(nr.value), error_pos=int(err.value), end_state=int(es.value), rc=rc,
               min_columns=int(cmin.value), max_columns=int(cmax.value))
    return res


def lex_restart_parallel(data, d: dict, threads: int, cap: int | None = None) -> dict:
    """The all-core CPU baseline (not the oracle): lex_restart's result, computed
    by the data-parallel method on `threads` host threads."""
    b = _as_u8(data)
    n = b.size
    cap = n + 1 if cap is None else cap
    out = _tok_out(cap)
    delta = np.ascontiguousarray(d["delta"], dtype=np.int16)
    kind = np.ascontiguousarray(d["kind"], dtype=np.uint16)
    nt = _U64()
    rc = lib().cpu_parallel_lex_restart(b.ctypes.data, n, delta.shape[0], d["q0"], delta.ctypes.data,
                                        kind.ctypes.data, out["kind"].ctypes.data, out["start"].ctypes.data,
                                        out["length"].ctypes.data, cap, threads, ctypes.byref(nt))
    k = int(nt.value)
    if rc == -1:
        raise ValueError("cpu_parallel_lex_restart: invalid table or thread count")
    res = {key: v[:min(k, cap)] for key, v in out.items()}
    res["n_tokens"] = k
    res["rc"] = rc
    return res
