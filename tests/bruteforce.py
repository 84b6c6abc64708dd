"""Exact rational brute force for tiny cases (a pin for the oracle, not the oracle).

Works on *logical* values (Python ``Fraction`` / ``int``) chosen by the test, never on
the stored bit patterns, so that the oracle's decoding (fp16, bf16, packed int4) is
checked too.  Scalar loops only; the per-element parameter lookup is written from the
pages' description of the granularities, independently of the oracle's expansion.
"""
from fractions import Fraction


def param_at(p, mode, i, j, g):
    """Parameter value applying to weight element (i, j)."""
    if mode == "tensor":
        return p[0]
    if mode == "channel":
        return p[j]
    return p[i // g][j]          # per-group: rows [r*g, (r+1)*g) share parameter row r


def antiquant(x1, codes, scale, offset, bias, x3, mode, g):
    """x1: list of m rows of k Fractions; codes: k rows of n ints."""
    m, k = len(x1), len(codes)
    n = len(codes[0]) if k else len(bias if bias is not None else x3[0])
    out = []
    for r in range(m):
        row = []
        for j in range(n):
            acc = Fraction(0)
            for i in range(k):
                off = param_at(offset, mode, i, j, g) if offset is not None else 0
                w = (codes[i][j] + off) * param_at(scale, mode, i, j, g)
                acc += x1[r][i] * w
            if bias is not None:
                acc += bias[j]
            if x3 is not None:
                acc += x3[r][j]
            row.append(acc)
        out.append(row)
    return out


def w8a8(x1, x2, bias, dq, pt, x3):
    m, k, n = len(x1), len(x2), len(x2[0])
    accs, outs = [], []
    for r in range(m):
        arow, orow = [], []
        for j in range(n):
            acc = sum(int(x1[r][i]) * int(x2[i][j]) for i in range(k))
            if bias is not None:
                acc += int(bias[j])
            d = dq[0] if len(dq) == 1 else dq[j]
            y = Fraction(d) * (Fraction(pt[r]) if pt is not None else 1) * acc
            if x3 is not None:
                y += x3[r][j]
            arow.append(acc)
            orow.append(y)
        accs.append(arow)
        outs.append(orow)
    return accs, outs
