"""Merge tables written out from their definition, for small grammars.

TEST INFRASTRUCTURE ONLY (see the package docstring). Plain Python tuples; it
shares nothing with the library's own table builder.

"Lexing on the GPU: the scan is the easy part", section "A lexer is a prefix
scan": partially apply the transition function to each symbol, delta_a(q) =
delta(q, a); composition is associative; precompute every composition that is
reachable, number it, and store composition as a k x k table so that merging
two prefix states is one lookup. The page's lexer masks a "produces a token"
flag off both operands (lexer.fut excerpt), so an element carries, besides the
state map f, a map p telling from which states its last byte ends a token:

  element of byte c:  f_c(q) = delta(q, c)           if defined,
                              delta(q0, c)           otherwise (restart),
                      p_c(q) = 1 if delta(q, c) is undefined, else 0;
  product (earlier a, later b):  (f_b o f_a,  p_b o f_a)  for non-empty a, b;
  identity: the empty string's element, neutral on both sides: a.e = a,
  e.b = b. It is an element of its own, apart from every non-empty element,
  even one whose maps are (id, 0): the product rule turns a.(id, 0) into
  (f_a, 0), clearing a's flag (a byte that keeps every state and ends no
  token), while a.e keeps it.

Table entries: merge[a][b] = id(a.b), with the flag bit set when p_{a.b}(q0)
is 1; initial_state[c] = id(element of c) (with the same flag rule);
final_states[x] = kind accepted in f_x(q0). Identifiers are handed out in
breadth-first order from the identity.
"""
from __future__ import annotations


def element_of_byte(d, c):
    Q, q0, delta = d["n_states"], d["q0"], d["delta"]
    f = tuple(int(delta[q][c]) if delta[q][c] >= 0 else int(delta[q0][c]) for q in range(Q))
    p = tuple(1 if delta[q][c] < 0 else 0 for q in range(Q))
    return f, p


EMPTY = ()  # the empty string's element (non-empty elements are (f, p) pairs)


def identity(Q):
    return EMPTY


def product(a, b):
    if b == EMPTY:
        return a
    if a == EMPTY:
        return b
    (fa, pa), (fb, pb) = a, b
    return tuple(fb[x] for x in fa), tuple(pb[x] for x in fa)


def build_tables(d, flag=0x8000, max_k=20000):
    Q, q0 = d["n_states"], d["q0"]
    ident = identity(Q)
    gens = {}
    byte_elem = []
    for c in range(256):
        e = element_of_byte(d, c)
        gens.setdefault(e, None)
        byte_elem.append(e)
    ids = {ident: 0}
    order = [ident]
    i = 0
    while i < len(order):
        x = order[i]
        i += 1
        for g in gens:
            y = product(x, g)
            if y not in ids:
                ids[y] = len(order)
                order.append(y)
                if len(order) > max_k:
                    raise ValueError("closure exceeds max_k")
    k = len(order)

    def entry(e):
        return ids[e] | (flag if e != EMPTY and e[1][q0] else 0)

    merge = [[entry(product(a, b)) for b in order] for a in order]
    init = [entry(e) for e in byte_elem]
    final = [int(d["kind"][q0 if e == EMPTY else e[0][q0]]) for e in order]
    return {"k": k, "identity": 0, "initial_state": init, "merge_table": merge, "final_states": final,
            "elements": order}
