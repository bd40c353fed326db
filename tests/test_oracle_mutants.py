"""The pins must catch plausible mistakes in the oracle.

Each mutant is a copy of the oracle's C source with one planted mistake
(a dropped term, a wrong index, an inverted test, a transposed operand),
compiled into a temporary library. The pins used here (hand-worked examples
and exhaustive comparison with the independent readers) must reject every one.
The oracle's own source is never modified.
"""
import ctypes
import itertools
import json
import multiprocessing
import os
import subprocess
import tempfile

import numpy as np
import pytest

import workloads as W
from oracle import lex_closure
from tests.rd_reader import read_t5, read_t6

HERE = os.path.dirname(__file__)
ORACLE_DIR = os.path.join(os.path.dirname(HERE), "oracle")

CSV_MUTANTS = {
    "length_plus_one": ("len_out[nf] = (uint32_t)(i - field_start);", "len_out[nf] = (uint32_t)(i - field_start + 1);"),
    "start_at_terminator": ("field_start = i + 1;", "field_start = i;"),
    "no_column_advance": ("                col++;\n", "\n"),
    "no_column_reset": ("                col = 0;\n", "\n"),
    "final_rule_field": ("last_tag != TAG_RECORD", "last_tag != TAG_FIELD"),
    "error_at_n_minus_1": ("err = (int64_t)n;", "err = (int64_t)n - 1;"),
    "last_invalid_not_first": ("if (t == TAG_INVALID && err < 0)", "if (t == TAG_INVALID)"),
    "accept_inverted": ("if (err < 0 && !((accept_mask >> s) & 1u))", "if (err < 0 && ((accept_mask >> s) & 1u))"),
    "final_record_not_counted": ("        nf++;\n        rec++;\n    }\n    if (err", "        nf++;\n    }\n    if (err"),
    "table_transposed": ("uint32_t t = tag[s * n_classes + c];", "uint32_t t = tag[c * n_classes + s];"),
    "next_from_old_state": ("        s = s_next;\n", "        s = next[s_next * n_classes + c];\n"),
    "record_index_after_bump": ("rec_out[nf] = (uint32_t)rec;\n                col_out", "rec_out[nf] = (uint32_t)(rec + (t == TAG_RECORD));\n                col_out"),
}

LEX_MUTANTS = {
    "restart_from_current": ("q = (uint32_t)delta[(uint64_t)q0 * 256 + b];", "q = (uint32_t)delta[(uint64_t)q * 256 + b] < 0 ? q0 : q;"),
    "kind_of_new_state": ("put(kind, start, len, cap, &nt, kind_of[q], tok_start, i - tok_start);\n            tok_start = i;",
                          "tok_start = i;\n            put(kind, start, len, cap, &nt, kind_of[delta[(uint64_t)q0 * 256 + b]], tok_start, i - tok_start);"),
    "no_final_token": ("    if (n > 0) put(kind, start, len, cap, &nt, kind_of[q], tok_start, n - tok_start);\n", "\n"),
    "fold_operands_swapped": ("uint16_t m = merge[(uint64_t)prev * k + x];", "uint16_t m = merge[(uint64_t)x * k + prev];"),
    "fold_kind_of_current": ("put(kind, start, len, cap, &nt, final_[prev], tok_start, i - tok_start);",
                             "put(kind, start, len, cap, &nt, final_[m & id_mask], tok_start, i - tok_start);"),
    "fold_flag_not_masked": ("        prev = m & id_mask;", "        prev = m;"),
}


def _compile_so(src_name, subst, tmp):
    src = open(os.path.join(ORACLE_DIR, src_name)).read()
    old, new = subst
    assert src.count(old) == 1, (src_name, old)
    path = os.path.join(tmp, "m.c")
    open(path, "w").write(src.replace(old, new))
    so = os.path.join(tmp, "m%d.so" % abs(hash(old + new)))
    subprocess.run(["gcc", "-O1", "-shared", "-fPIC", "-o", so, path], check=True, capture_output=True)
    return so


def _compile(src_name, subst, tmp):
    return ctypes.CDLL(_compile_so(src_name, subst, tmp))


def _pins_reject(src_name, subst, pins_pass):
    """Compiles a mutant and runs the pins on it in a forked child process. A
    mutant is caught when the pins reject it, and also when its mistake makes
    it crash or hang (an identifier with its flag bit left on indexes far past
    the merge table) instead of returning a wrong answer."""
    with tempfile.TemporaryDirectory() as tmp:
        so = _compile_so(src_name, subst, tmp)

        def child():
            os._exit(0 if pins_pass(ctypes.CDLL(so)) else 1)

        proc = multiprocessing.get_context("fork").Process(target=child)
        proc.start()
        proc.join(300)
        if proc.exitcode is None:
            proc.kill()
            proc.join()
            return True
        return proc.exitcode != 0


def _csv_run(L, t, b):
    n = len(b)
    cap = n + 2
    arr = np.frombuffer(b + b"\0", dtype=np.uint8)
    nxt = np.array(t["next"], dtype=np.uint8)
    tag = np.array(t["tag"], dtype=np.uint8)
    cm = np.frombuffer(t["class_map"], dtype=np.uint8)
    out = [np.zeros(cap, dtype=np.uint32) for _ in range(4)]
    nf, nr, err, es = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_int64(), ctypes.c_uint32()
    P = ctypes.c_void_p
    L.oracle_csv_parse.argtypes = [P, ctypes.c_uint64] + [ctypes.c_uint32] * 4 + [P] * 7 + [ctypes.c_uint64] + [P] * 4
    L.oracle_csv_parse(arr.ctypes.data, n, t["n_states"], t["n_classes"], t["start"], t["accept_mask"],
                       nxt.ctypes.data, tag.ctypes.data, cm.ctypes.data, *[o.ctypes.data for o in out], cap,
                       ctypes.byref(nf), ctypes.byref(nr), ctypes.byref(err), ctypes.byref(es))
    k = min(int(nf.value), cap)
    return [tuple(int(o[i]) for o in out) for i in range(k)], int(nr.value), int(err.value)


def _csv_pins_pass(L):
    """golden examples + exhaustive comparison with the readers (short inputs)"""
    for line in open(os.path.join(HERE, "golden", "csv_examples.jsonl")):
        c = json.loads(line)
        got = _csv_run(L, W.table(c["table"]), c["input"].encode("latin-1"))
        if got != ([tuple(f) for f in c["fields"]], c["n_records"], c["error_pos"]):
            return False
    for name, alpha, reader, max_len in (("T5", b',\n"a', read_t5, 5), ("T6", b'\t\n"#a', read_t6, 4)):
        t = W.table(name)
        for L_ in range(max_len + 1):
            for s in itertools.product(alpha, repeat=L_):
                s = bytes(s)
                if _csv_run(L, t, s) != reader(s):
                    return False
    return True


@pytest.mark.parametrize("mutant", sorted(CSV_MUTANTS))
def test_csv_mutant_is_caught(mutant):
    assert _pins_reject("csv_oracle.c", CSV_MUTANTS[mutant], _csv_pins_pass), "pins did not catch mutant %s" % mutant


def test_unmutated_csv_source_passes_same_pins():
    with tempfile.TemporaryDirectory() as tmp:
        L = _compile("csv_oracle.c", ("int oracle_csv_parse(", "int oracle_csv_parse("), tmp)
        assert _csv_pins_pass(L)


def _lex_tokens(L, fn, d, tables, b):
    n = len(b)
    cap = n + 2
    arr = np.frombuffer(b + b"\0", dtype=np.uint8)
    out = [np.zeros(cap, dtype=np.uint32) for _ in range(3)]
    nt = ctypes.c_uint64()
    P = ctypes.c_void_p
    if fn == "restart":
        delta = np.ascontiguousarray(d["delta"], dtype=np.int16)
        kind = np.ascontiguousarray(d["kind"], dtype=np.uint16)
        L.oracle_lex_restart.argtypes = [P, ctypes.c_uint64, ctypes.c_uint32, P, P, P, P, P, ctypes.c_uint64, P]
        L.oracle_lex_restart(arr.ctypes.data, n, d["q0"], delta.ctypes.data, kind.ctypes.data,
                             *[o.ctypes.data for o in out], cap, ctypes.byref(nt))
    else:
        init, merge, fin, k = tables
        L.oracle_lex_fold.argtypes = [P, ctypes.c_uint64, P, P, P, ctypes.c_uint32, ctypes.c_uint16, P, P, P,
                                      ctypes.c_uint64, P]
        L.oracle_lex_fold(arr.ctypes.data, n, init.ctypes.data, merge.ctypes.data, fin.ctypes.data, k, 0x8000,
                          *[o.ctypes.data for o in out], cap, ctypes.byref(nt))
    m = min(int(nt.value), cap)
    return [(int(out[0][i]), int(out[1][i]), int(out[2][i])) for i in range(m)]


def _lex_pins_pass(L):
    d = W.toy_dfa()
    t = lex_closure.build_tables(d)
    tables = (np.array(t["initial_state"], dtype=np.uint16), np.array(t["merge_table"], dtype=np.uint16),
              np.array(t["final_states"], dtype=np.uint16), t["k"])
    names = {nm: i for i, nm in enumerate(d["kind_names"])}
    for line in open(os.path.join(HERE, "golden", "lex_examples.jsonl")):
        c = json.loads(line)
        if c["grammar"] != "toy":
            continue
        want = [(names[k], s, ln) for k, s, ln in c["tokens"]]
        if _lex_tokens(L, "restart", d, None, c["input"].encode()) != want:
            return False
    for L_ in range(6):
        for s in itertools.product(b"a1 #", repeat=L_):
            s = bytes(s)
            if _lex_tokens(L, "restart", d, None, s) != _lex_tokens(L, "fold", d, tables, s):
                return False
    return True


@pytest.mark.parametrize("mutant", sorted(LEX_MUTANTS))
def test_lex_mutant_is_caught(mutant):
    assert _pins_reject("lex_oracle.c", LEX_MUTANTS[mutant], _lex_pins_pass), "pins did not catch mutant %s" % mutant


def test_unmutated_lex_source_passes_same_pins():
    with tempfile.TemporaryDirectory() as tmp:
        L = _compile("lex_oracle.c", ("int oracle_lex_fold(", "int oracle_lex_fold("), tmp)
        assert _lex_pins_pass(L)


# Planted mistakes in the oracle's count of records that do not have the
# expected number of fields (oracle._conformance): each must fail the
# hand-worked or exhaustive pins of tests/test_oracle_csv.py.
CONFORMANCE_MUTANTS = {
    "count_fields_not_records": lambda rec, n, e: (int(np.count_nonzero(np.bincount(rec.astype(np.int64), minlength=n)
                                                                         != e)) if e and n else 0,
                                                    -1),
    "first_off_by_one": lambda rec, n, e: _conf_with(rec, n, e, lambda bad: int(bad[0]) + 1),
    "last_not_first": lambda rec, n, e: _conf_with(rec, n, e, lambda bad: int(bad[-1])),
    "fewer_only": lambda rec, n, e: _conf_with(rec, n, e, None, cmp=lambda per: per < e),
    "columns_not_fields": lambda rec, n, e: _conf_with(rec, n, e, None, shift=1),
}


def _conf_with(rec, n, e, first=None, cmp=None, shift=0):
    if not e or n == 0:
        return 0, -1
    per = np.bincount(rec.astype(np.int64), minlength=n) - shift
    bad = np.nonzero(cmp(per) if cmp else per != e)[0]
    return int(bad.size), ((first or (lambda b: int(b[0])))(bad) if bad.size else -1)


def _conformance_pins_pass():
    from tests import test_oracle_csv as T
    try:
        T.test_conformance_examples()
        T.test_conformance_exhaustive_vs_recursive_descent("T5", b',\n"a', 5, read_t5)
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("mutant", sorted(CONFORMANCE_MUTANTS))
def test_conformance_mutant_is_caught(mutant, monkeypatch):
    import oracle
    monkeypatch.setattr(oracle, "_conformance", CONFORMANCE_MUTANTS[mutant])
    assert not _conformance_pins_pass(), mutant


def test_unmutated_conformance_passes_same_pins():
    assert _conformance_pins_pass()


# Planted mistakes in the columnar-partition oracle (oracle/columns.py): each
# copy of its source with one change must fail the pins of
# tests/test_oracle_columns.py.
COLUMNS_MUTANTS = {
    "unstable_within_column": ('order = np.argsort(col, kind="stable")', 'order = np.argsort(-col, kind="stable")[::-1]'),
    "slot_not_counted": ("pos += int(lens[j]) + slot", "pos += int(lens[j])"),
    "empty_fields_dropped": ("    for j in range(nf):\n", "    for j in [i for i in range(nf) if lens[i] > 0]:\n"),
    "aux_one_late": ("aux += bytes(int(lens[j]))", "aux += bytes(int(lens[j]) + 1)"),
    "column_bound_off_by_one": ("css_off[f] if f < nf else pos", "css_off[f] + 1 if f < nf else pos"),
    "terminator_before_field": ("        css += b[offs[j]:offs[j] + lens[j]].tobytes()\n        aux += bytes(int(lens[j]))\n        if slot:\n            css.append(terminator if mode == MODE_INLINE else 0)\n            aux.append(1)\n",
                                "        if slot:\n            css.append(terminator if mode == MODE_INLINE else 0)\n            aux.append(1)\n        css += b[offs[j]:offs[j] + lens[j]].tobytes()\n        aux += bytes(int(lens[j]))\n"),
}


def _columns_mutant(name):
    import types
    src = open(os.path.join(ORACLE_DIR, "columns.py")).read()
    old, new = COLUMNS_MUTANTS[name]
    assert src.count(old) == 1, (name, old)
    mod = types.ModuleType("columns_mutant")
    exec(compile(src.replace(old, new), "columns_mutant.py", "exec"), mod.__dict__)
    return mod.partition


def _columns_pins_pass():
    from tests import test_oracle_columns as T
    try:
        T.test_hand_worked()
        T.test_exhaustive_vs_recursive_descent()
        T.test_variant_invariants()
    except (AssertionError, IndexError, ValueError):
        return False
    return True


@pytest.mark.parametrize("mutant", sorted(COLUMNS_MUTANTS))
def test_columns_mutant_is_caught(mutant, monkeypatch):
    from oracle import columns
    monkeypatch.setattr(columns, "partition", _columns_mutant(mutant))
    assert not _columns_pins_pass(), mutant


def test_unmutated_columns_passes_same_pins():
    assert _columns_pins_pass()


NUMBERS_MUTANTS = {
    "width_top_inclusive": ("-(1 << (bits - 1)) <= v < (1 << (bits - 1))", "-(1 << (bits - 1)) <= v <= (1 << (bits - 1))"),
    "fraction_digits_added": ("- len(fp) +", "+ len(fp) +"),
    "trailing_zeros_kept": ('stripped = digits.rstrip(b"0")', "stripped = digits"),
    "column_minimum": ("ct[c] = max(ct[c], t)", "ct[c] = min(ct[c], t)"),
    "exponent_bound_23": ("    if -22 <= e10 <= 22:\n", "    if -23 <= e10 <= 23:\n"),
    "mantissa_bound_2_54": ("if w > 1 << 53:", "if w > 1 << 54:"),
    "int64_overflow_text": ("        return FLOAT64\n    if _FLOAT", "        return TEXT\n    if _FLOAT"),
    "mismatch_only_text": ("        elif t > ct:", "        elif t > ct and t == TEXT:"),
}


def _numbers_mutant(name):
    import types
    src = open(os.path.join(ORACLE_DIR, "numbers.py")).read()
    old, new = NUMBERS_MUTANTS[name]
    assert src.count(old) == 1, (name, old)
    mod = types.ModuleType("numbers_mutant")
    exec(compile(src.replace(old, new), "numbers_mutant.py", "exec"), mod.__dict__)
    return mod


def _numbers_pins_pass(mod, monkeypatch):
    from tests import test_oracle_numbers as T
    monkeypatch.setattr(T, "N", mod)
    try:
        for text, want in T.HAND_TYPES:
            T.test_hand_worked_types(text, want)
        T.test_width_boundaries()
        T.test_decompose_against_fractions()
        T.test_exact_class_one_rounding()
        T.test_infer_reduction()
        T.test_convert_hand_worked()
    except (AssertionError, IndexError, ValueError):
        return False
    return True


@pytest.mark.parametrize("mutant", sorted(NUMBERS_MUTANTS))
def test_numbers_mutant_is_caught(mutant, monkeypatch):
    assert not _numbers_pins_pass(_numbers_mutant(mutant), monkeypatch), mutant


def test_unmutated_numbers_passes_same_pins(monkeypatch):
    from oracle import numbers
    assert _numbers_pins_pass(numbers, monkeypatch)
