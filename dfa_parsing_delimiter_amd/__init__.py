"""Data-parallel DFA parsing of delimiter-separated bytes and table-driven lexing
on AMD Instinct MI355X (gfx950).

Thin binding over the C ABI of ``libppr.so`` (``include/ppr.h``): it marshals
arguments and nothing else. Every step of the parse runs in the library's HIP
kernels; PyTorch only provides device memory and the stream. There is no CPU
fallback: if the library is missing, importing this package fails.

    import dfa_parsing_delimiter_amd as ppr
    res = ppr.parse(bytes_tensor_on_cuda, table)          # per-field arrays
    tables = ppr.LexTables.from_dfa(token_dfa)            # lexer tables (device)
    toks = ppr.lex(bytes_tensor_on_cuda, tables)          # (kind, start, length)

A DFA table is a dict with keys n_states, n_classes, next[s][c], tag[s][c]
(0 value, 1 field delimiter, 2 record delimiter, 3 invalid), start,
accept_mask and class_map (256 bytes). A token DFA is a dict with delta
(n_states x 256, -1 = undefined; the start state's row total), kind
(n_states), q0.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PPR_LIB_PATH") or os.path.join(_HERE, "libppr.so")

PPR_OK, PPR_EINVAL, PPR_ECAPACITY, PPR_ETOOBIG, PPR_EHIP, PPR_EWORKSPACE = 0, -1, -2, -3, -4, -5
PPR_PATH_STREAMING, PPR_PATH_SINGLE_PASS, PPR_PATH_FUSED = 1, 2, 3
PPR_PARSE_CONTINUE, PPR_PARSE_PARTIAL = 1, 2
PPR_CSS_INDEXED, PPR_CSS_INLINE, PPR_CSS_VECTOR = 0, 1, 2
PPR_NUM_EMPTY, PPR_NUM_INT8, PPR_NUM_INT16, PPR_NUM_INT32, PPR_NUM_INT64, PPR_NUM_FLOAT64, PPR_NUM_TEXT = range(7)
PPR_NUM_OK, PPR_NUM_DEFAULTED, PPR_NUM_MISMATCH, PPR_NUM_INEXACT, PPR_NUM_NOT_CONVERTED = range(5)
_ERRNAMES = {-1: "PPR_EINVAL", -2: "PPR_ECAPACITY", -3: "PPR_ETOOBIG", -4: "PPR_EHIP", -5: "PPR_EWORKSPACE"}
TAG_VALUE, TAG_FIELD, TAG_RECORD, TAG_INVALID = 0, 1, 2, 3


class PprError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__("%s failed: %s (%d)" % (where, _ERRNAMES.get(code, "?"), code))
        self.code = code


class Dfa(ctypes.Structure):
    _fields_ = [("n_states", ctypes.c_uint32), ("n_classes", ctypes.c_uint32), ("start_state", ctypes.c_uint32),
                ("accept_mask", ctypes.c_uint32), ("next", (ctypes.c_uint8 * 16) * 8),
                ("tag", (ctypes.c_uint8 * 16) * 8)]


class ParseOut(ctypes.Structure):
    _fields_ = [("record_idx", ctypes.c_void_p), ("column_ids", ctypes.c_void_p),
                ("field_offsets", ctypes.c_void_p), ("field_lengths", ctypes.c_void_p),
                ("cap_fields", ctypes.c_uint64), ("n_fields", ctypes.c_uint64), ("n_records", ctypes.c_uint64),
                ("error_pos", ctypes.c_int64), ("end_state", ctypes.c_uint32), ("path", ctypes.c_uint32),
                ("min_columns", ctypes.c_uint32), ("max_columns", ctypes.c_uint32),
                ("bad_records", ctypes.c_uint64), ("first_bad_record", ctypes.c_int64),
                ("tail_start", ctypes.c_uint32), ("tail_column", ctypes.c_uint32)]


class ParseOpts(ctypes.Structure):
    _fields_ = [("chunk_bytes", ctypes.c_uint32), ("n_stage_events", ctypes.c_uint32),
                ("stage_events", ctypes.c_void_p), ("path", ctypes.c_uint32),
                ("expected_columns", ctypes.c_uint32), ("flags", ctypes.c_uint32), ("start_state", ctypes.c_uint32),
                ("start_column", ctypes.c_uint32)]


class ColumnsOut(ctypes.Structure):
    _fields_ = [("css", ctypes.c_void_p), ("aux", ctypes.c_void_p), ("css_cap", ctypes.c_uint64),
                ("rec", ctypes.c_void_p), ("css_off", ctypes.c_void_p), ("length", ctypes.c_void_p),
                ("col_first_field", ctypes.c_void_p), ("col_first_byte", ctypes.c_void_p),
                ("css_bytes", ctypes.c_uint64)]


class FieldsC(ctypes.Structure):
    _fields_ = [("bytes", ctypes.c_void_p), ("n_bytes", ctypes.c_uint64), ("off", ctypes.c_void_p),
                ("len", ctypes.c_void_p), ("col", ctypes.c_void_p), ("col_first", ctypes.c_void_p),
                ("n_fields", ctypes.c_uint64), ("n_columns", ctypes.c_uint32)]


class StreamOut(ctypes.Structure):
    _fields_ = [("record_idx", ctypes.c_void_p), ("column_ids", ctypes.c_void_p), ("field_offsets", ctypes.c_void_p),
                ("field_lengths", ctypes.c_void_p), ("cap_fields", ctypes.c_uint64), ("n_fields", ctypes.c_uint64),
                ("n_records", ctypes.c_uint64), ("error_pos", ctypes.c_int64), ("end_state", ctypes.c_uint32),
                ("min_columns", ctypes.c_uint32), ("max_columns", ctypes.c_uint32), ("partitions", ctypes.c_uint32),
                ("bad_records", ctypes.c_uint64), ("first_bad_record", ctypes.c_int64)]


class LexTablesC(ctypes.Structure):
    _fields_ = [("initial_state", ctypes.c_void_p), ("merge_table", ctypes.c_void_p),
                ("final_states", ctypes.c_void_p), ("k", ctypes.c_uint32), ("identity", ctypes.c_uint16),
                ("flag_mask", ctypes.c_uint16)]


class LexPrepared(ctypes.Structure):
    _fields_ = [("d_fold", ctypes.c_void_p), ("k", ctypes.c_uint32), ("m", ctypes.c_uint32),
                ("identity", ctypes.c_uint16), ("flag_mask", ctypes.c_uint16), ("column_of", ctypes.c_uint8 * 256),
                ("n_states", ctypes.c_uint32), ("n_rows", ctypes.c_uint32), ("row0", ctypes.c_uint32)]


class TokensOut(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_void_p), ("start", ctypes.c_void_p), ("length", ctypes.c_void_p),
                ("cap_tokens", ctypes.c_uint64), ("n_tokens", ctypes.c_uint64), ("path", ctypes.c_uint32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libppr.so is not built (run: python dfa_parsing_delimiter_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    P, U64, U32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32
    L.ppr_parse_workspace_bytes.argtypes = [U64, ctypes.POINTER(ParseOpts)]
    L.ppr_parse_workspace_bytes.restype = ctypes.c_size_t
    for f in ("ppr_parse", "ppr_parse_async"):
        getattr(L, f).argtypes = [P, U64, ctypes.POINTER(Dfa), ctypes.c_char_p, ctypes.POINTER(ParseOut), P,
                                  ctypes.c_size_t, ctypes.POINTER(ParseOpts), P]
        getattr(L, f).restype = ctypes.c_int
    L.ppr_parse_noalloc.argtypes = [P, U64, ctypes.POINTER(Dfa), ctypes.c_char_p, ctypes.POINTER(ParseOut),
                                    ctypes.POINTER(ParseOpts), P]
    L.ppr_parse_noalloc.restype = ctypes.c_int
    L.ppr_parse_stream.argtypes = [P, U64, ctypes.POINTER(Dfa), ctypes.c_char_p, ctypes.POINTER(StreamOut), U64,
                                   ctypes.POINTER(ParseOpts)]
    L.ppr_parse_stream.restype = ctypes.c_int
    L.ppr_columns_workspace_bytes.argtypes = [U64, U32]
    L.ppr_columns_workspace_bytes.restype = ctypes.c_size_t
    L.ppr_columns.argtypes = [P, U64, P, P, P, P, U64, U32, U32, U32, ctypes.POINTER(ColumnsOut), P, ctypes.c_size_t,
                              ctypes.POINTER(ParseOpts), P]
    L.ppr_columns.restype = ctypes.c_int
    L.ppr_numbers_workspace_bytes.argtypes = [U32]
    L.ppr_numbers_workspace_bytes.restype = ctypes.c_size_t
    L.ppr_infer_types.argtypes = [ctypes.POINTER(FieldsC), P, P, P, ctypes.c_size_t, P]
    L.ppr_infer_types.restype = ctypes.c_int
    L.ppr_convert.argtypes = [ctypes.POINTER(FieldsC), P, ctypes.c_int64, ctypes.c_double, P, P, P, P, ctypes.c_size_t,
                              P]
    L.ppr_convert.restype = ctypes.c_int
    L.ppr_parse_results.argtypes = [P, U64, ctypes.POINTER(ParseOut), P]
    L.ppr_parse_results.restype = ctypes.c_int
    L.ppr_lex_fold_bytes.argtypes = [U32]
    L.ppr_lex_fold_bytes.restype = ctypes.c_size_t
    L.ppr_lex_prepare.argtypes = [ctypes.POINTER(LexTablesC), ctypes.POINTER(LexPrepared), P]
    L.ppr_lex_prepare.restype = ctypes.c_int
    L.ppr_lex_workspace_bytes.argtypes = [U64, ctypes.POINTER(ParseOpts)]
    L.ppr_lex_workspace_bytes.restype = ctypes.c_size_t
    for f in ("ppr_lex", "ppr_lex_async"):
        getattr(L, f).argtypes = [P, U64, ctypes.POINTER(LexTablesC), ctypes.POINTER(LexPrepared),
                                  ctypes.POINTER(TokensOut), P, ctypes.c_size_t, ctypes.POINTER(ParseOpts), P]
        getattr(L, f).restype = ctypes.c_int
    L.ppr_lex_results.argtypes = [P, U64, ctypes.POINTER(TokensOut), P]
    L.ppr_lex_results.restype = ctypes.c_int
    L.ppr_lex_build_tables.argtypes = [P, P, U32, U32, U32, ctypes.POINTER(U32), P, P, P, ctypes.POINTER(ctypes.c_uint16)]
    L.ppr_lex_build_tables.restype = ctypes.c_int
    L.ppr_version.argtypes = []
    L.ppr_version.restype = ctypes.c_char_p
    L.ppr_bandwidth_probe.argtypes = [U32, U32, P, P, U64, U32, P]
    L.ppr_bandwidth_probe.restype = ctypes.c_int
    return L


lib = _load()


def version() -> str:
    return lib.ppr_version().decode()


def bandwidth_probe(mode: int, pattern: int, src, dst, nbytes: int, grid: int, stream=None):
    """Enqueue one probe kernel (ppr_bandwidth_probe): mode 0 read, 1 write,
    2 copy; pattern 0 wave-contiguous 16-byte words, 1 64 bytes per lane."""
    _check(lib.ppr_bandwidth_probe(mode, pattern, ctypes.c_void_p(0 if src is None else src.data_ptr()),
                                   ctypes.c_void_p(dst.data_ptr()), nbytes, grid, _stream_handle(stream)),
           "ppr_bandwidth_probe")


def _check(code: int, where: str):
    if code != PPR_OK:
        raise PprError(code, where)


def _stream_handle(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _opts(chunk_bytes, path=None, expected_columns=0):
    o = ParseOpts()
    o.chunk_bytes = int(chunk_bytes or 0)
    o.path = int(path or 0)
    o.expected_columns = int(expected_columns or 0)
    return o


def _opts_with_events(opts, events):
    """A copy of opts that records the given (already created) torch.cuda.Event
    objects between the call's kernels; returns (opts, the handle array to keep alive)."""
    o = ParseOpts()
    o.chunk_bytes = opts.chunk_bytes
    o.path = opts.path
    o.expected_columns = opts.expected_columns
    o.flags, o.start_state, o.start_column = opts.flags, opts.start_state, opts.start_column
    if not events:
        return o, None
    handles = (ctypes.c_void_p * len(events))(*[int(e.cuda_event) for e in events])
    if not all(handles):
        raise ValueError("stage events must have been recorded once (created) before use")
    o.n_stage_events = len(events)
    o.stage_events = ctypes.cast(handles, ctypes.c_void_p)
    return o, handles


def make_dfa(table: dict):
    """(Dfa struct, class map bytes) from a DFA table dict."""
    d = Dfa()
    d.n_states = table["n_states"]
    d.n_classes = table["n_classes"]
    d.start_state = table["start"]
    d.accept_mask = table["accept_mask"]
    for s in range(table["n_states"]):
        for c in range(table["n_classes"]):
            d.next[s][c] = table["next"][s][c]
            d.tag[s][c] = table["tag"][s][c]
    cm = bytes(table["class_map"])
    assert len(cm) == 256
    return d, cm


def _check_input(data: torch.Tensor):
    if not (isinstance(data, torch.Tensor) and data.is_cuda and data.dtype == torch.uint8 and data.dim() == 1
            and data.is_contiguous()):
        raise TypeError("input must be a contiguous 1-D torch.uint8 tensor on a CUDA (HIP) device")


@dataclass
class ParseResult:
    record_idx: torch.Tensor     # int32 view of the uint32 arrays, length n_fields
    column_ids: torch.Tensor
    field_offsets: torch.Tensor
    field_lengths: torch.Tensor
    n_fields: int
    n_records: int
    error_pos: int
    end_state: int
    path: int                    # the kernels that ran: a PPR_PATH_* value
    min_columns: int             # fewest / most fields of a record (0 / 0 without records): the inferred
    max_columns: int             # number of columns is max_columns; all records conform iff the two are equal
    bad_records: int = 0         # with expected_columns: records with another number of fields,
    first_bad_record: int = -1   # and the first of them (-1: none)


class Parser:
    """Reusable workspace and output buffers for inputs of up to max_n bytes."""

    def __init__(self, table: dict, max_n: int, capacity: int | None = None, chunk_bytes: int | None = None,
                 device=None, path: int | None = None, expected_columns: int = 0):
        self.dfa, self.class_map = make_dfa(table)
        self.opts = _opts(chunk_bytes, path, expected_columns)
        self.device = torch.device("cuda") if device is None else torch.device(device)
        self.max_n = int(max_n)
        ws = lib.ppr_parse_workspace_bytes(self.max_n, ctypes.byref(self.opts))
        if ws == 0:
            raise PprError(PPR_EINVAL, "ppr_parse_workspace_bytes")
        self.ws = torch.empty(ws + 256, dtype=torch.uint8, device=self.device)
        self.ws_off = (-self.ws.data_ptr()) % 256
        self.ws_bytes = ws
        self._alloc(self.max_n + 1 if capacity is None else int(capacity))

    def _alloc(self, cap):
        self.cap = max(int(cap), 1)
        self.out_arrays = [torch.empty(self.cap, dtype=torch.int32, device=self.device) for _ in range(4)]

    def _out(self):
        o = ParseOut()
        o.record_idx, o.column_ids, o.field_offsets, o.field_lengths = [a.data_ptr() for a in self.out_arrays]
        o.cap_fields = self.cap
        return o

    def _ws_ptr(self):
        return ctypes.c_void_p(self.ws.data_ptr() + self.ws_off)

    def launch(self, data: torch.Tensor, stream=None, stage_events=None):
        """enqueue one parse without waiting (for timing loops); stage_events:
        optional torch.cuda.Event list recorded before/between/after the kernels"""
        _check_input(data)
        n = data.numel()
        if n > self.max_n:
            raise ValueError("input larger than the parser's max_n")
        o = self._out()
        opts, keep = _opts_with_events(self.opts, stage_events)
        _check(lib.ppr_parse_async(ctypes.c_void_p(data.data_ptr()), n, ctypes.byref(self.dfa), self.class_map,
                                   ctypes.byref(o), self._ws_ptr(), self.ws_bytes, ctypes.byref(opts),
                                   _stream_handle(stream)), "ppr_parse_async")
        del keep

    def results(self, n: int, stream=None) -> ParseOut:
        o = self._out()
        rc = lib.ppr_parse_results(self._ws_ptr(), n, ctypes.byref(o), _stream_handle(stream))
        if rc not in (PPR_OK, PPR_ECAPACITY):
            raise PprError(rc, "ppr_parse_results")
        return o

    def __call__(self, data: torch.Tensor, stream=None) -> ParseResult:
        _check_input(data)
        n = data.numel()
        if n > self.max_n:
            raise ValueError("input larger than the parser's max_n")
        for _ in range(2):
            o = self._out()
            rc = lib.ppr_parse(ctypes.c_void_p(data.data_ptr()), n, ctypes.byref(self.dfa), self.class_map,
                               ctypes.byref(o), self._ws_ptr(), self.ws_bytes, ctypes.byref(self.opts),
                               _stream_handle(stream))
            if rc == PPR_ECAPACITY:  # size, then fill
                self._alloc(o.n_fields)
                continue
            _check(rc, "ppr_parse")
            k = int(o.n_fields)
            return ParseResult(*[a[:k] for a in self.out_arrays], k, int(o.n_records), int(o.error_pos),
                               int(o.end_state), int(o.path), int(o.min_columns), int(o.max_columns),
                               int(o.bad_records), int(o.first_bad_record))
        raise PprError(PPR_ECAPACITY, "ppr_parse")


def parse(data: torch.Tensor, table: dict, chunk_bytes: int | None = None, capacity: int | None = None,
          stream=None, path: int | None = None, expected_columns: int = 0) -> ParseResult:
    """Parse one input (device uint8 tensor) with a DFA table; path: a
    PPR_PATH_* value to ask for (None: the library's automatic choice);
    expected_columns > 0: count the records with another number of fields."""
    _check_input(data)
    n = data.numel()
    cap = capacity if capacity is not None else min(n + 1, max(4096, n // 4))
    return Parser(table, n, cap, chunk_bytes, data.device, path, expected_columns)(data, stream)


@dataclass
class ColumnsResult:
    css: torch.Tensor              # uint8, css_bytes (device)
    aux: torch.Tensor | None       # uint8, css_bytes (vector-delimited mode)
    rec: torch.Tensor              # int32 views of uint32, one entry per field grouped by column
    css_off: torch.Tensor
    length: torch.Tensor
    col_first_field: torch.Tensor  # n_columns + 1
    col_first_byte: torch.Tensor
    css_bytes: int
    n_columns: int


class Columns:
    """Reusable workspace and outputs for the columnar partition (ppr_columns)
    of parses of up to max_fields fields and max_bytes input bytes."""

    def __init__(self, max_fields: int, n_columns: int, max_bytes: int, mode: int = PPR_CSS_INDEXED,
                 terminator: int = 0x1F, device=None, css_capacity: int | None = None):
        self.device = torch.device("cuda") if device is None else torch.device(device)
        self.mode, self.terminator, self.n_columns = int(mode), int(terminator), int(n_columns)
        ws = lib.ppr_columns_workspace_bytes(max_fields, self.n_columns)
        if ws == 0:
            raise PprError(PPR_EINVAL, "ppr_columns_workspace_bytes")
        self.ws = torch.empty(ws + 256, dtype=torch.uint8, device=self.device)
        self.ws_off = (-self.ws.data_ptr()) % 256
        self.ws_bytes = ws
        cap = css_capacity if css_capacity is not None else max_bytes + (max_fields if mode != PPR_CSS_INDEXED else 0)
        self.css_cap = max(1, int(cap))
        self.css = torch.empty(self.css_cap, dtype=torch.uint8, device=self.device)
        self.aux = torch.empty(self.css_cap, dtype=torch.uint8, device=self.device) if mode == PPR_CSS_VECTOR else None
        f = max(1, int(max_fields))
        self.ent = [torch.empty(f, dtype=torch.int32, device=self.device) for _ in range(3)]
        self.bounds = [torch.empty(self.n_columns + 1, dtype=torch.int32, device=self.device) for _ in range(2)]

    def __call__(self, data: torch.Tensor, res: "ParseResult", stream=None, stage_events=None) -> ColumnsResult:
        """stage_events: optional list of 7 torch.cuda.Event recorded before and after the call's kernels"""
        _check_input(data)
        opts, keep = _opts_with_events(_opts(None), stage_events)
        o = ColumnsOut()
        o.css, o.css_cap = self.css.data_ptr(), self.css_cap
        o.aux = self.aux.data_ptr() if self.aux is not None else None
        o.rec, o.css_off, o.length = [a.data_ptr() for a in self.ent]
        o.col_first_field, o.col_first_byte = [a.data_ptr() for a in self.bounds]
        nf = int(res.n_fields)
        rc = lib.ppr_columns(ctypes.c_void_p(data.data_ptr()), data.numel(), ctypes.c_void_p(res.record_idx.data_ptr()),
                             ctypes.c_void_p(res.column_ids.data_ptr()), ctypes.c_void_p(res.field_offsets.data_ptr()),
                             ctypes.c_void_p(res.field_lengths.data_ptr()), nf, self.n_columns, self.mode,
                             self.terminator, ctypes.byref(o), ctypes.c_void_p(self.ws.data_ptr() + self.ws_off),
                             self.ws_bytes, ctypes.byref(opts), _stream_handle(stream))
        del keep
        _check(rc, "ppr_columns")
        k = int(o.css_bytes)
        return ColumnsResult(self.css[:k], self.aux[:k] if self.aux is not None else None,
                             *[a[:nf] for a in self.ent], *self.bounds, k, self.n_columns)


def columns(data: torch.Tensor, res: "ParseResult", n_columns: int | None = None, mode: int = PPR_CSS_INDEXED,
            terminator: int = 0x1F, stream=None) -> ColumnsResult:
    """Partition a parse's fields by column into per-column symbol strings and
    their index (one call; n_columns defaults to the parse's max_columns)."""
    nc = int(res.max_columns if n_columns is None else n_columns)
    return Columns(res.n_fields, nc, data.numel(), mode, terminator, data.device)(data, res, stream)


class Fields:
    """Spans (off, len) of a device byte tensor, with their columns: col (per
    field) or col_first (fields grouped by column) or neither (one column)."""

    def __init__(self, data: torch.Tensor, off: torch.Tensor, length: torch.Tensor, n_columns: int = 1,
                 col: torch.Tensor | None = None, col_first: torch.Tensor | None = None):
        _check_input(data)
        self.keep = (data, off, length, col, col_first)
        self.c = FieldsC(data.data_ptr(), data.numel(), off.data_ptr() if off.numel() else None,
                         length.data_ptr() if length.numel() else None,
                         col.data_ptr() if col is not None and col.numel() else None,
                         col_first.data_ptr() if col_first is not None else None, off.numel(), int(n_columns))
        self.device = data.device

    @classmethod
    def of_parse(cls, data: torch.Tensor, res: "ParseResult", n_columns: int | None = None):
        return cls(data, res.field_offsets, res.field_lengths, max(1, res.max_columns if n_columns is None else n_columns),
                   col=res.column_ids)

    @classmethod
    def of_columns(cls, cols: "ColumnsResult"):
        return cls(cols.css, cols.css_off, cols.length, max(1, cols.n_columns), col_first=cols.col_first_field)


def _num_ws(n_columns, device):
    nbytes = lib.ppr_numbers_workspace_bytes(int(n_columns))
    if nbytes == 0:
        raise PprError(PPR_EINVAL, "ppr_numbers_workspace_bytes")
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    return ws, (-ws.data_ptr()) % 256, nbytes


def infer_types(fields: Fields, field_types: bool = False, stream=None):
    """(column types as a numpy uint32 array, per-field types as a device uint8 tensor or None)"""
    ws, off, nbytes = _num_ws(fields.c.n_columns, fields.device)
    ft = torch.empty(max(1, fields.c.n_fields), dtype=torch.uint8, device=fields.device) if field_types else None
    ct = np.zeros(fields.c.n_columns, dtype=np.uint32)
    _check(lib.ppr_infer_types(ctypes.byref(fields.c), ctypes.c_void_p(ft.data_ptr()) if ft is not None else None,
                               ct.ctypes.data, ctypes.c_void_p(ws.data_ptr() + off), nbytes, _stream_handle(stream)),
           "ppr_infer_types")
    return ct, (ft[:fields.c.n_fields] if ft is not None else None)


@dataclass
class Converted:
    values: torch.Tensor   # int64 per field (device): the value, or the double's bits for FLOAT64 columns
    status: torch.Tensor   # uint8 per field (device): PPR_NUM_OK ... PPR_NUM_NOT_CONVERTED
    counts: np.ndarray     # fields with status 1..4


def convert(fields: Fields, column_types, int_default: int = 0, float_default: float = 0.0, stream=None) -> Converted:
    ws, off, nbytes = _num_ws(fields.c.n_columns, fields.device)
    n = fields.c.n_fields
    vals = torch.empty(max(1, n), dtype=torch.int64, device=fields.device)
    st = torch.empty(max(1, n), dtype=torch.uint8, device=fields.device)
    ct = np.ascontiguousarray(column_types, dtype=np.uint32)
    if ct.size != fields.c.n_columns:
        raise ValueError("one type per column")
    counts = np.zeros(4, dtype=np.uint64)
    _check(lib.ppr_convert(ctypes.byref(fields.c), ct.ctypes.data, int(int_default), float(float_default),
                           ctypes.c_void_p(vals.data_ptr()), ctypes.c_void_p(st.data_ptr()), counts.ctypes.data,
                           ctypes.c_void_p(ws.data_ptr() + off), nbytes, _stream_handle(stream)), "ppr_convert")
    return Converted(vals[:n], st[:n], counts)


@dataclass
class StreamResult:
    record_idx: np.ndarray       # uint64, length n_fields (host)
    column_ids: np.ndarray       # uint32
    field_offsets: np.ndarray    # uint64
    field_lengths: np.ndarray    # uint64
    n_fields: int
    n_records: int
    error_pos: int
    end_state: int
    min_columns: int
    max_columns: int
    partitions: int
    bad_records: int = 0
    first_bad_record: int = -1


def parse_stream(data, table: dict, partition_bytes: int, capacity: int | None = None,
                 chunk_bytes: int | None = None, path: int | None = None, expected_columns: int = 0,
                 pinned: bool = True) -> StreamResult:
    """Parse host bytes (a uint8 numpy array or a CPU torch tensor, pinned for
    overlapped transfers) in partitions of partition_bytes through
    ppr_parse_stream; the results are those of one parse of the whole input,
    in host arrays (pinned torch memory when pinned)."""
    if isinstance(data, torch.Tensor):
        if data.is_cuda or data.dtype != torch.uint8 or not data.is_contiguous():
            raise TypeError("host input must be a contiguous CPU uint8 tensor or numpy array")
        ptr, n = data.data_ptr(), data.numel()
    else:
        data = np.ascontiguousarray(data, dtype=np.uint8)
        ptr, n = data.ctypes.data, data.size
    dfa, cm = make_dfa(table)
    opts = _opts(chunk_bytes, path, expected_columns)
    for _ in range(2):  # size, then fill
        cap = max(1, int(capacity if capacity is not None else min(n + 1, max(4096, n // 4))))
        arrs = [torch.empty(cap, dtype=dt, pin_memory=pinned) for dt in (torch.int64, torch.int32, torch.int64,
                                                                          torch.int64)]
        o = StreamOut()
        o.record_idx, o.column_ids, o.field_offsets, o.field_lengths = [a.data_ptr() for a in arrs]
        o.cap_fields = cap
        rc = lib.ppr_parse_stream(ctypes.c_void_p(ptr), n, ctypes.byref(dfa), cm, ctypes.byref(o), partition_bytes,
                                  ctypes.byref(opts))
        if rc == PPR_ECAPACITY and capacity is None:
            capacity = int(o.n_fields)
            continue
        _check(rc, "ppr_parse_stream")
        k = int(o.n_fields)
        return StreamResult(arrs[0][:k].numpy().view(np.uint64), arrs[1][:k].numpy().view(np.uint32),
                            arrs[2][:k].numpy().view(np.uint64), arrs[3][:k].numpy().view(np.uint64), k,
                            int(o.n_records), int(o.error_pos), int(o.end_state), int(o.min_columns),
                            int(o.max_columns), int(o.partitions), int(o.bad_records), int(o.first_bad_record))
    raise PprError(PPR_ECAPACITY, "ppr_parse_stream")


# ------------------------------------------------------------------ lexer

class LexTables:
    """Device-resident lexer tables plus their prepared fold table."""

    def __init__(self, initial_state: np.ndarray, merge_table: np.ndarray, final_states: np.ndarray, k: int,
                 identity: int = 0, device=None):
        dev = torch.device("cuda") if device is None else torch.device(device)
        self.k = int(k)
        self.identity = int(identity)
        self.h_initial = np.ascontiguousarray(initial_state, dtype=np.uint16).reshape(256)
        self.h_merge = np.ascontiguousarray(merge_table, dtype=np.uint16).reshape(self.k * self.k)
        self.h_final = np.ascontiguousarray(final_states, dtype=np.uint16).reshape(self.k)
        as_dev = lambda a: torch.from_numpy(a.view(np.int16)).to(dev)
        self.initial_state, self.merge_table, self.final_states = (as_dev(self.h_initial), as_dev(self.h_merge),
                                                                   as_dev(self.h_final))
        self.c = LexTablesC(self.initial_state.data_ptr(), self.merge_table.data_ptr(), self.final_states.data_ptr(),
                            self.k, self.identity, 0x8000)
        self.fold = torch.empty(lib.ppr_lex_fold_bytes(self.k) // 2, dtype=torch.int16, device=dev)
        self.prep = LexPrepared()
        self.prep.d_fold = self.fold.data_ptr()
        _check(lib.ppr_lex_prepare(ctypes.byref(self.c), ctypes.byref(self.prep), _stream_handle()),
               "ppr_lex_prepare")

    @staticmethod
    def build_host(dfa: dict, max_k: int = 32768):
        """(initial_state, merge_table, final_states, k, identity) built by the library's host builder."""
        delta = np.ascontiguousarray(dfa["delta"], dtype=np.int16)
        kind = np.ascontiguousarray(dfa["kind"], dtype=np.uint16)
        Q = delta.shape[0]
        k = ctypes.c_uint32()
        ident = ctypes.c_uint16()
        _check(lib.ppr_lex_build_tables(delta.ctypes.data, kind.ctypes.data, Q, dfa["q0"], max_k, ctypes.byref(k),
                                        None, None, None, None), "ppr_lex_build_tables")
        kk = int(k.value)
        init = np.zeros(256, dtype=np.uint16)
        merge = np.zeros(kk * kk, dtype=np.uint16)
        fin = np.zeros(kk, dtype=np.uint16)
        _check(lib.ppr_lex_build_tables(delta.ctypes.data, kind.ctypes.data, Q, dfa["q0"], max_k, ctypes.byref(k),
                                        init.ctypes.data, merge.ctypes.data, fin.ctypes.data, ctypes.byref(ident)),
               "ppr_lex_build_tables")
        return init, merge.reshape(kk, kk), fin, kk, int(ident.value)

    @classmethod
    def from_dfa(cls, dfa: dict, device=None):
        init, merge, fin, k, ident = cls.build_host(dfa)
        return cls(init, merge, fin, k, ident, device)


@dataclass
class LexResult:
    kind: torch.Tensor
    start: torch.Tensor
    length: torch.Tensor
    n_tokens: int
    path: int = 0                # the kernels that ran: PPR_PATH_STREAMING or PPR_PATH_SINGLE_PASS


class Lexer:
    """Reusable workspace and token buffers for inputs of up to max_n bytes."""

    def __init__(self, tables: LexTables, max_n: int, capacity: int | None = None, chunk_bytes: int | None = None,
                 path: int | None = None):
        self.t = tables
        self.opts = _opts(chunk_bytes, path)
        self.max_n = int(max_n)
        dev = tables.merge_table.device
        ws = lib.ppr_lex_workspace_bytes(self.max_n, ctypes.byref(self.opts))
        if ws == 0:
            raise PprError(PPR_EINVAL, "ppr_lex_workspace_bytes")
        self.ws = torch.empty(ws + 256, dtype=torch.uint8, device=dev)
        self.ws_off = (-self.ws.data_ptr()) % 256
        self.ws_bytes = ws
        self.device = dev
        self._alloc(self.max_n + 1 if capacity is None else int(capacity))

    def _alloc(self, cap):
        self.cap = max(int(cap), 1)
        self.out_arrays = [torch.empty(self.cap, dtype=torch.int32, device=self.device) for _ in range(3)]

    def _out(self):
        o = TokensOut()
        o.kind, o.start, o.length = [a.data_ptr() for a in self.out_arrays]
        o.cap_tokens = self.cap
        return o

    def _ws_ptr(self):
        return ctypes.c_void_p(self.ws.data_ptr() + self.ws_off)

    def launch(self, data: torch.Tensor, stream=None, stage_events=None):
        _check_input(data)
        o = self._out()
        opts, keep = _opts_with_events(self.opts, stage_events)
        _check(lib.ppr_lex_async(ctypes.c_void_p(data.data_ptr()), data.numel(), ctypes.byref(self.t.c),
                                 ctypes.byref(self.t.prep), ctypes.byref(o), self._ws_ptr(), self.ws_bytes,
                                 ctypes.byref(opts), _stream_handle(stream)), "ppr_lex_async")
        del keep

    def results(self, n: int, stream=None) -> TokensOut:
        o = self._out()
        rc = lib.ppr_lex_results(self._ws_ptr(), n, ctypes.byref(o), _stream_handle(stream))
        if rc not in (PPR_OK, PPR_ECAPACITY):
            raise PprError(rc, "ppr_lex_results")
        return o

    def __call__(self, data: torch.Tensor, stream=None) -> LexResult:
        _check_input(data)
        n = data.numel()
        if n > self.max_n:
            raise ValueError("input larger than the lexer's max_n")
        for _ in range(2):
            o = self._out()
            rc = lib.ppr_lex(ctypes.c_void_p(data.data_ptr()), n, ctypes.byref(self.t.c), ctypes.byref(self.t.prep),
                             ctypes.byref(o), self._ws_ptr(), self.ws_bytes, ctypes.byref(self.opts),
                             _stream_handle(stream))
            if rc == PPR_ECAPACITY:
                self._alloc(o.n_tokens)
                continue
            _check(rc, "ppr_lex")
            k = int(o.n_tokens)
            return LexResult(*[a[:k] for a in self.out_arrays], k, int(o.path))
        raise PprError(PPR_ECAPACITY, "ppr_lex")


def lex(data: torch.Tensor, tables: LexTables, chunk_bytes: int | None = None, capacity: int | None = None,
        stream=None, path: int | None = None) -> LexResult:
    """Lex one input (device uint8 tensor); path: a PPR_PATH_* value to ask for
    (None: automatic)."""
    _check_input(data)
    n = data.numel()
    cap = capacity if capacity is not None else min(n + 1, max(4096, n // 3))
    return Lexer(tables, n, cap, chunk_bytes, path)(data, stream)
