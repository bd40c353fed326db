"""Seeded synthetic workloads (inputs only).

The only module shared by the CPU oracle's tests and the HIP path's tests and
benchmark. It holds:

* the byte generators (``gen.c``: xoshiro256** seeded through splitmix64),
* the DFA tables of the delimiter-separated workloads (``dfa.py``),
* the lexer's token grammar and its DFA (``lexgrammar.py``),
* the five workload configurations.

None of it parses: no state-transition vector, composition, scan, tag or merge
table appears here.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import subprocess

import numpy as np

from . import dfa as _dfa
from . import lexgrammar as _lexgrammar

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "_libworkloads.so")

MiB = 1 << 20
GiB = 1 << 30
SEED_BASE = 0xC0FFEE00


def build(force: bool = True) -> str:
    """Compile gen.c into a shared library next to it (plain gcc, -O2)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", "-o", tmp, _SRC],
                       check=True)
        os.replace(tmp, _LIB)
    return _LIB


class CsvParams(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("n", ctypes.c_uint64), ("n_cols", ctypes.c_uint32),
                ("len_kind", ctypes.c_uint32), ("len_lo", ctypes.c_uint32), ("len_hi", ctypes.c_uint32),
                ("geo_den", ctypes.c_uint32), ("comment_max", ctypes.c_uint32),
                ("fdelim", ctypes.c_uint8), ("rdelim", ctypes.c_uint8), ("quote", ctypes.c_uint8),
                ("comment", ctypes.c_uint8), ("pad", ctypes.c_uint32),
                ("thr_quoted", ctypes.c_uint64), ("thr_emb_f", ctypes.c_uint64), ("thr_emb_r", ctypes.c_uint64),
                ("thr_escape", ctypes.c_uint64), ("thr_comment", ctypes.c_uint64)]


class Truth(ctypes.Structure):
    _fields_ = [("rec", ctypes.c_void_p), ("col", ctypes.c_void_p), ("off", ctypes.c_void_p),
                ("len", ctypes.c_void_p), ("cap", ctypes.c_uint64), ("count", ctypes.c_uint64),
                ("records", ctypes.c_uint64)]


class TokenEntry(ctypes.Structure):
    _fields_ = [("pattern", ctypes.c_uint32), ("kind", ctypes.c_uint32), ("lit_off", ctypes.c_uint32),
                ("lit_len", ctypes.c_uint32), ("weight", ctypes.c_uint32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        L.wl_gen_csv.argtypes = [ctypes.POINTER(CsvParams), ctypes.c_void_p, ctypes.POINTER(Truth)]
        L.wl_gen_csv.restype = ctypes.c_int
        L.wl_gen_tokens.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.POINTER(TokenEntry), ctypes.c_uint32,
                                    ctypes.c_char_p, ctypes.c_char_p, ctypes.c_char_p, ctypes.c_uint32,
                                    ctypes.c_uint8, ctypes.c_void_p, ctypes.POINTER(Truth)]
        L.wl_gen_tokens.restype = ctypes.c_int
        for f in ("wl_splitmix64_stream", "wl_xoshiro_seeded_stream"):
            getattr(L, f).argtypes = [ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint64]
            getattr(L, f).restype = None
        L.wl_xoshiro_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64]
        L.wl_xoshiro_stream.restype = None
        _lib = L
    return _lib


def _thr(p: float) -> int:
    return min(int(p * 18446744073709551616.0), (1 << 64) - 1)


# ---------------------------------------------------------------- configs

CONFIGS = {
    1: dict(name="tiny_csv", kind="csv", table="T5", n=1 * MiB, n_cols=8, len_kind=0, len_lo=0, len_hi=24,
            quoted=0.20, emb_f=0.05, emb_r=0.05, escape=0.05),
    2: dict(name="numeric_csv", kind="csv", table="T5", n=256 * MiB, n_cols=16, len_kind=2, len_lo=1, len_hi=12,
            quoted=0.0, emb_f=0.0, emb_r=0.0, escape=0.0),
    3: dict(name="quote_heavy_csv", kind="csv", table="T5", n=1 * GiB, n_cols=12, len_kind=1, len_hi=4096,
            geo_den=41, quoted=0.60, emb_f=0.0, emb_r=0.10, escape=0.10, chunk_bytes=31),
    4: dict(name="wide_tsv", kind="csv", table="T6", n=1 * GiB, n_cols=512, len_kind=0, len_lo=0, len_hi=16,
            quoted=0.02, emb_f=0.05, emb_r=0.05, escape=0.05, comment=0.01, comment_max=80),
    5: dict(name="lexer_tokens", kind="lex", n=512 * MiB),
}


def seed_of(cfg_id: int) -> int:
    return SEED_BASE + cfg_id


def table(name: str) -> dict:
    return _dfa.TABLES[name]()


def csv_params(cfg_id: int, n: int | None = None, seed: int | None = None) -> CsvParams:
    c = CONFIGS[cfg_id]
    assert c["kind"] == "csv"
    t = table(c["table"])
    names = t["class_names"]
    # recover the delimiter bytes from the class map (first byte of each named class)
    first = {}
    for b in range(256):
        first.setdefault(t["class_map"][b], b)
    p = CsvParams()
    p.seed = seed_of(cfg_id) if seed is None else seed
    p.n = c["n"] if n is None else n
    p.n_cols = c["n_cols"]
    p.len_kind = c["len_kind"]
    p.len_lo = c.get("len_lo", 0)
    p.len_hi = c["len_hi"]
    p.geo_den = c.get("geo_den", 0)
    p.comment_max = c.get("comment_max", 0)
    p.fdelim = first[names.index("FDELIM")]
    p.rdelim = first[names.index("RDELIM")]
    p.quote = first[names.index("QUOTE")]
    p.comment = first[names.index("COMMENT")] if "COMMENT" in names and c.get("comment") else 0
    p.thr_quoted = _thr(c["quoted"])
    p.thr_emb_f = _thr(c["emb_f"])
    p.thr_emb_r = _thr(c["emb_r"])
    p.thr_escape = _thr(c["escape"])
    p.thr_comment = _thr(c.get("comment", 0.0))
    return p


def _truth_arrays(cap):
    arrs = {k: np.zeros(cap, dtype=np.uint32) for k in ("rec", "col", "off", "len")}
    t = Truth(arrs["rec"].ctypes.data, arrs["col"].ctypes.data, arrs["off"].ctypes.data, arrs["len"].ctypes.data,
              cap, 0, 0)
    return t, arrs


def gen_csv(params: CsvParams, truth: bool = False, out: np.ndarray | None = None):
    """Generate params.n bytes. With truth=True also return the placed fields
    (record, column, offset, length) and the record count."""
    n = int(params.n)
    buf = np.empty(n, dtype=np.uint8) if out is None else out
    assert buf.dtype == np.uint8 and buf.size >= n and buf.flags.c_contiguous
    if truth:
        cap = n + 1
        t, arrs = _truth_arrays(cap)
        rc = lib().wl_gen_csv(ctypes.byref(params), buf.ctypes.data, ctypes.byref(t))
        if rc != 0:
            raise MemoryError("wl_gen_csv failed")
        k = int(t.count)
        return buf[:n], {"rec": arrs["rec"][:k], "col": arrs["col"][:k], "off": arrs["off"][:k],
                         "len": arrs["len"][:k], "n_fields": k, "n_records": int(t.records)}
    rc = lib().wl_gen_csv(ctypes.byref(params), buf.ctypes.data, None)
    if rc != 0:
        raise MemoryError("wl_gen_csv failed")
    return buf[:n]


def generate(cfg_id: int, n: int | None = None, seed: int | None = None, truth: bool = False):
    c = CONFIGS[cfg_id]
    if c["kind"] == "csv":
        return gen_csv(csv_params(cfg_id, n, seed), truth=truth)
    return gen_tokens(seed_of(cfg_id) if seed is None else seed, c["n"] if n is None else n, truth=truth)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(memoryview(np.ascontiguousarray(a))).hexdigest()


# ---------------------------------------------------------------- lexer workload

lexer_dfa = _lexgrammar.lexer_dfa
toy_dfa = _lexgrammar.toy_dfa
random_token_dfa = _lexgrammar.random_token_dfa
keyword_chain_dfa = _lexgrammar.keyword_chain_dfa
many_columns_dfa = _lexgrammar.many_columns_dfa

from . import numtext as _numtext  # noqa: E402

numeric_csv = _numtext.numeric_csv

_PATTERN_FIRST = {
    1: set(_lexgrammar.ALPHA),
    2: set(_lexgrammar.DIGIT),
    3: set(_lexgrammar.DIGIT),
    4: {ord('"')},
    5: set(b" \t\n\r"),
    6: {ord("/")},
}
_PATTERN_RULE = {1: "IDENT", 2: "INT", 3: "FLOAT", 4: "STRING", 5: "WS", 6: "COMMENT"}
_PATTERN_WEIGHT = {1: 22, 2: 6, 3: 3, 4: 3, 5: 18, 6: 1}
_OP_WEIGHT = {"(": 4, ")": 4, ";": 4, ",": 3, ".": 3, "=": 3, "{": 2, "}": 2, "[": 2, "]": 2, "+": 2,
              "-": 2, "*": 2, "==": 1, "->": 1, ":": 1}


def _run(d, s: bytes):
    q = d["q0"]
    for b in s:
        q = int(d["delta"][q][b])
        if q < 0:
            return None
    return q


def token_entries(d=None):
    """Generator entries for the 40-rule grammar, the byte pair table and the
    padding rule (see wl_gen_tokens). Derived from the grammar's DFA: an entry
    may follow another directly only if no state the first can end in continues
    on any byte the second can start with."""
    d = lexer_dfa() if d is None else d
    names = d["kind_names"]
    kind_of = {nm: i for i, nm in enumerate(names)}
    ents, lits = [], bytearray()
    for pat in range(1, 7):
        ents.append(dict(pattern=pat, kind=kind_of[_PATTERN_RULE[pat]], lit=b"", weight=_PATTERN_WEIGHT[pat]))
    for op in _lexgrammar.OPERATORS:
        ents.append(dict(pattern=0, kind=kind_of["OP" + op], lit=op.encode(), weight=_OP_WEIGHT.get(op, 1)))
    seps = []
    for s in (b" ", b"\n"):
        seps.append(len(ents))
        ents.append(dict(pattern=0, kind=kind_of["WS"], lit=s, weight=0))
    delta = d["delta"]

    def end_states(e):
        if e["pattern"] == 0:
            q = _run(d, e["lit"])
            assert q is not None and d["kind"][q] == e["kind"]
            return {q}
        return {q for q in range(d["n_states"]) if d["kind"][q] == e["kind"]}

    def first(e):
        return {e["lit"][0]} if e["pattern"] == 0 else _PATTERN_FIRST[e["pattern"]]

    ends = [end_states(e) for e in ents]
    firsts = [first(e) for e in ents]

    def fuse(a, b):
        return any(delta[q][c] >= 0 for q in ends[a] for c in firsts[b])

    ne = len(ents)
    pair = np.zeros((ne, ne), dtype=np.uint8)
    for a in range(ne):
        for b in range(ne):
            if not fuse(a, b):
                continue
            pair[a, b] = 255
            for s in seps:
                if not fuse(a, s) and not fuse(s, b):
                    pair[a, b] = s + 1
                    break
    absorbs = np.zeros(ne, dtype=np.uint8)
    for i in range(ne):
        cont = {bool(delta[q][ord(" ")] >= 0) for q in ends[i]}
        assert len(cont) == 1, "padding behaviour differs between end states"
        absorbs[i] = cont.pop()
    arr = (TokenEntry * ne)()
    for i, e in enumerate(ents):
        arr[i].pattern = e["pattern"]
        arr[i].kind = e["kind"]
        arr[i].lit_off = len(lits)
        arr[i].lit_len = len(e["lit"])
        arr[i].weight = e["weight"]
        lits += e["lit"]
    return dict(entries=arr, n=ne, lits=bytes(lits) + b"\0", pair=pair, absorbs=absorbs,
                pad_kind=kind_of["WS"], pad_byte=ord(" "))


_TOKEN_CACHE = {}


def gen_tokens(seed: int, n: int, truth: bool = False, out: np.ndarray | None = None):
    """n bytes of token stream from the 40-rule grammar; with truth=True also the
    token (kind, start, length) sequence the generator wrote."""
    if "t" not in _TOKEN_CACHE:
        _TOKEN_CACHE["t"] = token_entries()
    te = _TOKEN_CACHE["t"]
    buf = np.empty(n, dtype=np.uint8) if out is None else out
    pair = np.ascontiguousarray(te["pair"]).tobytes()
    absorbs = te["absorbs"].tobytes()
    if truth:
        t, arrs = _truth_arrays(n + 1)
        rc = lib().wl_gen_tokens(seed, n, te["entries"], te["n"], te["lits"], pair, absorbs, te["pad_kind"],
                                 te["pad_byte"], buf.ctypes.data, ctypes.byref(t))
        if rc != 0:
            raise RuntimeError("wl_gen_tokens failed")
        k = int(t.count)
        return buf[:n], {"kind": arrs["rec"][:k], "start": arrs["off"][:k], "length": arrs["len"][:k],
                         "n_tokens": k}
    rc = lib().wl_gen_tokens(seed, n, te["entries"], te["n"], te["lits"], pair, absorbs, te["pad_kind"],
                             te["pad_byte"], buf.ctypes.data, None)
    if rc != 0:
        raise RuntimeError("wl_gen_tokens failed")
    return buf[:n]


def long_field_csv(n: int, seed: int) -> np.ndarray:
    """n bytes of T5 CSV whose records mix short fields with quoted fields of
    1-6 KiB (commas, newlines and doubled quotes inside), so that chunks far
    into a quoted field are ambiguous (inside or outside quotes) for several
    KiB. Seeded; the last record may be cut at n bytes."""
    r = np.random.default_rng(seed)
    alnum = np.frombuffer(b"abcdefghijklmnopqrstuvwxyz0123456789", np.uint8)

    def text(k):
        return bytes(alnum[r.integers(0, alnum.size, k)])

    templates = []
    for _ in range(64):
        fields = []
        for _ in range(int(r.integers(2, 7))):
            u = r.random()
            if u < 0.3:
                body = bytearray(text(int(r.integers(1024, 6144))))
                for pos in r.integers(0, len(body), 6):
                    body[pos] = b",\n"[int(r.integers(0, 2))]
                if r.random() < 0.5:
                    body[len(body) // 2:len(body) // 2] = b'""'
                fields.append(b'"' + bytes(body) + b'"')
            elif u < 0.6:
                fields.append(b'"' + text(int(r.integers(0, 30))) + b'"')
            else:
                fields.append(text(int(r.integers(0, 30))))
        templates.append(b",".join(fields) + b"\n")
    out = bytearray()
    while len(out) < n:
        out += templates[int(r.integers(0, len(templates)))]
    return np.frombuffer(bytes(out[:n]), np.uint8).copy()
