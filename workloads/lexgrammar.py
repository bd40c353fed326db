"""Token grammar for the lexer workload, compiled to a DFA (pure input data).

"Lexing on the GPU: the scan is the easy part" (section "A lexer is a prefix
scan") starts from a lexer DFA with transition function delta and start state
q0. The pages do not print a grammar; this module defines one of 40 token rules
(identifiers, integers, floats, strings with escapes, whitespace, line comments
and 34 operators) and compiles it with Thompson's construction followed by the
subset construction. The result is the DFA every lexer in this project reads:

  delta[q][b]  next state, or -1 where the rule set has no continuation,
  kind[q]      token kind accepted in q (0 = ERROR for non-accepting states),
  q0           start state, whose row is total: a byte that starts no token
               leads to the dead state E (kind ERROR, no transitions).

Rule priority breaks ties between rules accepting the same spelling (the
earlier rule wins). No lexing happens here.
"""
from __future__ import annotations

import numpy as np

# ---- regular expressions over byte sets (combinators) ----


class _R:
    pass


class Set(_R):
    def __init__(self, chars):
        self.chars = frozenset(chars if not isinstance(chars, (bytes, str)) else
                               (chars.encode() if isinstance(chars, str) else chars))


class Cat(_R):
    def __init__(self, *parts):
        self.parts = parts


class Alt(_R):
    def __init__(self, *parts):
        self.parts = parts


class Star(_R):
    def __init__(self, inner):
        self.inner = inner


def lit(s: str) -> _R:
    return Cat(*[Set([b]) for b in s.encode()])


def plus(r: _R) -> _R:
    return Cat(r, Star(r))


def opt(r: _R) -> _R:
    return Alt(r, Cat())


def rng(a: str, b: str) -> set:
    return set(range(ord(a), ord(b) + 1))


def anybut(chars: str) -> Set:
    ex = set(chars.encode())
    return Set([b for b in range(256) if b not in ex])


DIGIT = rng("0", "9")
HEX = DIGIT | rng("a", "f") | rng("A", "F")
ALPHA = rng("a", "z") | rng("A", "Z") | {ord("_")}

OPERATORS = ["+", "-", "*", "/", "%", "=", "==", "!=", "<", "<=", ">", ">=", "&&", "||", "!",
             "&", "|", "^", "~", "<<", ">>", "(", ")", "{", "}", "[", "]", ";", ",", ".",
             ":", "+=", "-=", "->"]


def token_rules():
    """The 40 rules, in priority order. Kind ids are 1 + index; 0 is ERROR.

    INT     decimal digits, or 0x/0X + hex digits, or 0b/0B + binary digits
    FLOAT   digits '.' digits [exponent], or digits exponent; exponent = [eE][+-]?digits
    STRING  '"' ... '"' with no raw quote, backslash or newline inside;
            escapes \\" \\\\ \\n \\t and \\x followed by two hex digits
    COMMENT '//' up to (not including) the next newline
    """
    exponent = Cat(Set(b"eE"), opt(Set(b"+-")), plus(Set(DIGIT)))
    escape = Alt(Cat(lit("\\"), Set(b'"\\nt')), Cat(lit("\\x"), Set(HEX), Set(HEX)))
    rules = [
        ("WS", plus(Set(b" \t\r\n"))),
        ("COMMENT", Cat(lit("//"), Star(anybut("\n")))),
        ("IDENT", Cat(Set(ALPHA), Star(Set(ALPHA | DIGIT)))),
        ("INT", Alt(plus(Set(DIGIT)),
                    Cat(lit("0"), Set(b"xX"), plus(Set(HEX))),
                    Cat(lit("0"), Set(b"bB"), plus(Set(b"01"))))),
        ("FLOAT", Alt(Cat(plus(Set(DIGIT)), lit("."), plus(Set(DIGIT)), opt(exponent)),
                      Cat(plus(Set(DIGIT)), exponent))),
        ("STRING", Cat(lit('"'), Star(Alt(anybut('"\\\n'), escape)), lit('"'))),
    ]
    rules += [("OP" + op, lit(op)) for op in OPERATORS]
    assert len(rules) == 40
    return rules


# ---- Thompson NFA ----


class _NFA:
    def __init__(self):
        self.eps = []   # list of lists of targets
        self.edges = []  # list of lists of (frozenset bytes, target)

    def new(self):
        self.eps.append([])
        self.edges.append([])
        return len(self.eps) - 1

    def build(self, r):
        """returns (start, end) fragment"""
        if isinstance(r, Set):
            a, b = self.new(), self.new()
            self.edges[a].append((r.chars, b))
            return a, b
        if isinstance(r, Cat):
            a = self.new()
            cur = a
            for p in r.parts:
                s, e = self.build(p)
                self.eps[cur].append(s)
                cur = e
            return a, cur
        if isinstance(r, Alt):
            a, b = self.new(), self.new()
            for p in r.parts:
                s, e = self.build(p)
                self.eps[a].append(s)
                self.eps[e].append(b)
            return a, b
        if isinstance(r, Star):
            a, b = self.new(), self.new()
            s, e = self.build(r.inner)
            self.eps[a] += [s, b]
            self.eps[e] += [s, b]
            return a, b
        raise TypeError(r)


def _closure(nfa, states):
    stack, seen = list(states), set(states)
    while stack:
        s = stack.pop()
        for t in nfa.eps[s]:
            if t not in seen:
                seen.add(t)
                stack.append(t)
    return frozenset(seen)


def compile_rules(rules):
    nfa = _NFA()
    root = nfa.new()
    accept = {}  # nfa end state -> kind id
    for i, (_, r) in enumerate(rules):
        s, e = nfa.build(r)
        nfa.eps[root].append(s)
        accept[e] = i + 1
    start = _closure(nfa, [root])
    index = {start: 0}
    order = [start]
    trans = []
    i = 0
    while i < len(order):
        cur = order[i]
        i += 1
        row = [-1] * 256
        for b in range(256):
            tgt = set()
            for s in cur:
                for chars, t in nfa.edges[s]:
                    if b in chars:
                        tgt.add(t)
            if tgt:
                nxt = _closure(nfa, tgt)
                if nxt not in index:
                    index[nxt] = len(order)
                    order.append(nxt)
                row[b] = index[nxt]
        trans.append(row)
    # dead state E, and a total start row
    E = len(order)
    trans.append([-1] * 256)
    for b in range(256):
        if trans[0][b] < 0:
            trans[0][b] = E
    kinds = []
    for st in order:
        ks = [accept[s] for s in st if s in accept]
        kinds.append(min(ks) if ks else 0)
    kinds.append(0)
    trans, kinds, E = _minimize(trans, kinds, E)
    return {
        "n_states": len(trans),
        "q0": 0,
        "err": E,
        "delta": np.array(trans, dtype=np.int16),
        "kind": np.array(kinds, dtype=np.uint16),
        "kind_names": ("ERROR",) + tuple(name for name, _ in rules),
    }


def _minimize(trans, kinds, E):
    """Moore partition refinement. Two states merge only if they accept the same
    kind and, for every byte, both lack a continuation or both continue into
    merged states (a missing continuation is observable: the lexer restarts).
    The start state and the dead state keep classes of their own."""
    n = len(trans)
    cls = [(0 if q == 0 else 1 if q == E else 2, kinds[q]) for q in range(n)]
    while True:
        ids = {}
        block = [ids.setdefault(c, len(ids)) for c in cls]
        sig = [(block[q],) + tuple(block[t] if t >= 0 else -1 for t in trans[q]) for q in range(n)]
        ids2 = {}
        block2 = [ids2.setdefault(s, len(ids2)) for s in sig]
        if len(ids2) == len(ids):
            break
        cls = sig
    # renumber blocks in order of their first member (the start state keeps id 0)
    new_id, order = {}, []
    for q in range(n):
        b = block2[q]
        if b not in new_id:
            new_id[b] = len(order)
            order.append(q)
    out = [[new_id[block2[t]] if t >= 0 else -1 for t in trans[q]] for q in order]
    return out, [kinds[q] for q in order], new_id[block2[E]]


def lexer_dfa():
    """DFA of the 40-rule grammar."""
    return compile_rules(token_rules())


def toy_dfa():
    """Three rules: ID=[a-z]+, NUM=[0-9]+, WS=' '+ (a small hand-checkable grammar)."""
    rules = [("ID", plus(Set(rng("a", "z")))), ("NUM", plus(Set(DIGIT))), ("WS", plus(Set(b" ")))]
    return compile_rules(rules)


def random_token_dfa(seed: int, n_states: int, n_cols: int, p_undefined: float = 0.3, n_kinds: int = 6):
    """A seeded random token DFA (same dict format as compile_rules): the 256
    bytes fall into n_cols byte classes (every class used), each state has a
    random successor or none (-1) per class, the start state 0 has a successor
    for every class, and every state a random kind in [0, n_kinds)."""
    r = np.random.default_rng(seed)
    col_of = np.concatenate([np.arange(n_cols), r.integers(0, n_cols, 256 - n_cols)])
    r.shuffle(col_of)
    table = r.integers(0, n_states, (n_states, n_cols))
    undefined = r.random((n_states, n_cols)) < p_undefined
    undefined[0, :] = False
    table[undefined] = -1
    return {
        "n_states": n_states,
        "q0": 0,
        "delta": table[:, col_of].astype(np.int16),
        "kind": r.integers(0, n_kinds, n_states).astype(np.uint16),
        "kind_names": tuple("K%d" % i for i in range(n_kinds)),
    }


def keyword_chain_dfa(length: int, seed: int):
    """A token DFA for one keyword of `length` distinct bytes (a seeded
    permutation of 1..255): state i has read the keyword's first i bytes, the
    keyword's next byte moves on, anything else ends the token; the start row
    sends every other byte to the dead state E. Kinds: KEYWORD for the whole
    keyword, PART for a proper prefix, ERROR for E. Returns (dfa, keyword)."""
    r = np.random.default_rng(seed)
    word = r.permutation(np.arange(1, 256))[:length]
    Q, E = length + 2, length + 1
    delta = np.full((Q, 256), -1, dtype=np.int16)
    delta[0, :] = E
    delta[0, word[0]] = 1
    for i in range(1, length):
        delta[i, word[i]] = i + 1
    kind = np.full(Q, 2, dtype=np.uint16)
    kind[length], kind[E], kind[0] = 1, 0, 0
    return ({"n_states": Q, "q0": 0, "delta": delta, "kind": kind, "kind_names": ("ERROR", "KEYWORD", "PART")},
            bytes(word.astype(np.uint8)))


def many_columns_dfa(n_cols: int, seed: int = 5):
    """A token DFA of 4 states whose 256 bytes fall into n_cols classes (byte b
    in class b mod n_cols, 2 <= n_cols <= 192) with pairwise different columns,
    so that the byte columns of its closure number exactly n_cols. Each class
    is one of the 192 columns (successor of the start state in {1, 2, 3}, of
    states 1-3 in {none, 1, 2, 3}), drawn without repetition; kinds 0-3."""
    import itertools
    combos = list(itertools.product([1, 2, 3], [-1, 1, 2, 3], [-1, 1, 2, 3], [-1, 1, 2, 3]))
    if not 2 <= n_cols <= len(combos):
        raise ValueError("n_cols out of range")
    pick = np.random.default_rng(seed).permutation(len(combos))[:n_cols]
    delta = np.empty((4, 256), dtype=np.int16)
    for b in range(256):
        delta[:, b] = combos[pick[b % n_cols]]
    return {"n_states": 4, "q0": 0, "delta": delta, "kind": np.arange(4, dtype=np.uint16),
            "kind_names": ("K0", "K1", "K2", "K3")}
