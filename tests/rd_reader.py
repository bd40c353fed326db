"""Independent readers for the delimiter-separated formats (test pins).

Written from the format rules, not from any DFA table: a recursive-descent walk
over fields and records. They pin the oracle's sequential DFA loop: for every
input, the four per-field arrays, the record count and the error position must
agree. Rules (the readings the project fixes for ParPaRaw, Sec. 3 and
"validating format"):

* a field's span is raw: from the byte after the previous terminator (or 0) to
  its terminator (or the end), quotes included;
* every record delimiter closes a field and a record; a final record exists iff
  the input is non-empty and does not end with a record delimiter;
* RFC 4180 quoting in the five-state format: a quote at a field start opens a
  quoted field, "" inside it is a literal quote, the closing quote must be
  followed by a delimiter or the end; a quote inside an unquoted field, or any
  other byte after a closing quote, makes the input invalid at that byte, and
  from there to the end nothing more is delimited;
* an input that ends inside quotes is invalid at n;
* tab-separated format with comments: a record starting with '#' is one field
  up to the next newline, uninterpreted; elsewhere a quote opens a quoted
  section wherever it appears in a field (not only at its start).
"""


def read_t5(b: bytes, fd=ord(","), rd=ord("\n"), q=ord('"')):
    n = len(b)
    fields, rec, col, err = [], 0, 0, -1
    pos = 0  # start of the current field
    i = 0
    while True:
        # at a field start
        if i < n and b[i] == q:
            j = i + 1
            closed = None
            while j < n:
                if b[j] == q:
                    if j + 1 < n and b[j + 1] == q:
                        j += 2
                        continue
                    closed = j
                    break
                j += 1
            if closed is None:  # ran off the end inside quotes
                err = n
                fields.append((rec, col, pos, n - pos))
                return fields, rec + 1, err
            k = closed + 1
            if k == n:
                fields.append((rec, col, pos, n - pos))
                return fields, rec + 1, err
            if b[k] == fd or b[k] == rd:
                i = k
            else:  # stray byte after the closing quote
                err = k
                fields.append((rec, col, pos, n - pos))
                return fields, rec + 1, err
        else:
            j = i
            while j < n and b[j] not in (fd, rd, q):
                j += 1
            if j == n:
                if n == 0:
                    return fields, 0, -1
                fields.append((rec, col, pos, n - pos))
                return fields, rec + 1, err
            if b[j] == q:  # quote inside an unquoted field
                err = j
                fields.append((rec, col, pos, n - pos))
                return fields, rec + 1, err
            i = j
        # b[i] is a delimiter ending the current field
        fields.append((rec, col, pos, i - pos))
        if b[i] == fd:
            col += 1
        else:
            rec += 1
            col = 0
        pos = i = i + 1
        if i == n:
            # input ends right after a delimiter: a field delimiter leaves an empty final field
            if b[n - 1] == fd:
                fields.append((rec, col, pos, 0))
                return fields, rec + 1, err
            return fields, rec, err


def read_t6(b: bytes, fd=ord("\t"), rd=ord("\n"), q=ord('"'), cm=ord("#")):
    n = len(b)
    fields, rec, col, err = [], 0, 0, -1
    pos = i = 0
    at_record_start = True
    while True:
        if at_record_start and i < n and b[i] == cm:
            j = i
            while j < n and b[j] != rd:
                j += 1
            if j == n:
                fields.append((rec, 0, pos, n - pos))
                return fields, rec + 1, err
            i = j
        else:
            # a field: runs of plain bytes and quoted sections
            j = i
            while True:
                while j < n and b[j] not in (fd, rd, q):
                    j += 1
                if j == n or b[j] != q:
                    break
                # quoted section from j
                k = j + 1
                closed = None
                while k < n:
                    if b[k] == q:
                        if k + 1 < n and b[k + 1] == q:
                            k += 2
                            continue
                        closed = k
                        break
                    k += 1
                if closed is None:
                    err = n
                    fields.append((rec, col, pos, n - pos))
                    return fields, rec + 1, err
                k = closed + 1
                if k == n or b[k] in (fd, rd):
                    j = k
                    break
                # byte after a closing quote that is neither a delimiter nor a quote
                err = k
                fields.append((rec, col, pos, n - pos))
                return fields, rec + 1, err
            if j == n:
                if n == 0:
                    return fields, 0, -1
                fields.append((rec, col, pos, n - pos))
                return fields, rec + 1, err
            i = j
        fields.append((rec, col, pos, i - pos))
        if b[i] == fd:
            col += 1
            at_record_start = False
        else:
            rec += 1
            col = 0
            at_record_start = True
        pos = i = i + 1
        if i == n:
            if b[n - 1] == fd:
                fields.append((rec, col, pos, 0))
                return fields, rec + 1, err
            return fields, rec, err
