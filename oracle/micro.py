"""Exact-rational micro oracle for tiny vocabularies (test infrastructure only).

A second, independent statement of steps 3-4 of alg. 2 (wikillm.com card for
arXiv 2302.01318, Method: "Modified rejection sampling", paper sec. 4.2, and
"Algorithm: Speculative Sampling (SpS)"), written with ``fractions.Fraction``
so that every comparison is exact.  It works on probability vectors given as
rationals and shares no code with ``spec_oracle.c``.  Used to cross-check the
fp64 oracle on small cases whose decision boundaries are exact rationals.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Sequence


def accept(q: Fraction, p: Fraction, u: Fraction) -> bool:
    """u < min(1, q/p); with p == 0 accept exactly when q > 0."""
    if p == 0:
        return q > 0
    return u < min(Fraction(1), q / p)


def residual(q: Sequence[Fraction], p: Sequence[Fraction]) -> list[Fraction]:
    """max(0, q - p), or q itself when that has no mass."""
    w = [max(Fraction(0), a - b) for a, b in zip(q, p)]
    if sum(w) == 0:
        return list(q)
    return w


def draw(w: Sequence[Fraction], u: Fraction) -> int:
    """Smallest x whose cumulative weight exceeds u * total (strict)."""
    total = sum(w)
    target = u * total
    acc = Fraction(0)
    for x, wx in enumerate(w):
        acc += wx
        if acc > target:
            return x
    raise ValueError("no token: total weight is zero or u >= 1")


def verify(q: Sequence[Sequence[Fraction]], p: Sequence[Sequence[Fraction]],
           tokens: Sequence[int], uniforms: Sequence[Fraction]) -> tuple[int, list[int]]:
    """Return (accepted count n, emitted tokens of length n+1)."""
    K = len(p)
    out: list[int] = []
    n = 0
    while n < K:
        x = tokens[n]
        if not accept(q[n][x], p[n][x], uniforms[n]):
            break
        out.append(x)
        n += 1
    w = residual(q[n], p[n]) if n < K else list(q[K])
    out.append(draw(w, uniforms[K]))
    return n, out
