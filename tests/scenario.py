"""Parser/runner for the hand-worked page-table scenario fixtures.

The runner drives any object with the page-table operations
(seq_create, seq_fork, reserve, truncate, seq_free, export, stats) and
raises AssertionError on the first mismatch.  Errors are reported by the
driven object as an exception carrying ``.kind``.
"""

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    ops = []
    cfg = None
    order = None
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("config"):
                cfg = [int(x) for x in line.split()[1:]]
                continue
            if line.startswith("free_order"):
                order = [int(x) for x in line.split()[1:]]
                continue
            lhs, rhs = [x.strip() for x in line.split("->")]
            ops.append((lhs.split(), rhs))
    return cfg, order, ops


def run(pt, ops, error_type):
    for args, expect in ops:
        op = args[0]
        a = [int(x) for x in args[1:]]
        try:
            if op == "create":
                got = str(pt.seq_create())
            elif op == "fork":
                got = str(pt.seq_fork(a[0], a[1]))
            elif op == "reserve":
                r = pt.reserve(a[0], a[1])
                got = "none" if r is None else "cow %d %d %d" % tuple(r)
            elif op == "truncate":
                pt.truncate(a[0], a[1])
                got = "ok"
            elif op == "free":
                pt.seq_free(a[0])
                got = "ok"
            elif op == "export":
                table, lens = pt.export(a[1:], a[0])
                rows = " | ".join(" ".join(str(int(x)) for x in row) for row in table)
                got = rows + " ; " + " ".join(str(int(x)) for x in lens)
            elif op == "stats":
                got = "%d %d" % tuple(pt.stats())
            else:
                raise ValueError(op)
        except error_type as e:
            got = "error " + e.kind
        norm = " ".join(expect.split())
        assert " ".join(got.split()) == norm, "%s: expected %r, got %r" % (" ".join(args), norm, got)
