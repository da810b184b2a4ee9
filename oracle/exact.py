"""Exact rational brute force for tiny shapes (fractions + forward-mode dual numbers).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The forward is the definition on "Fractus-1B training optimization", section 1,
Bottleneck #1, evaluated literally: for every token t the state S_t is rebuilt
from scratch as S_in + sum_{j<=t} k_j v_j^T (no running recurrence, no
reordering), then o_t = S_t^T q_t / (q_t . z_t).  Gradients are not derived by
hand: each is the exact derivative of the scalar loss
    L = sum_t <dO_t, o_t> + <dS_out, S_out> + dz_out . z_out
along one input coordinate, obtained by evaluating the same forward on dual
numbers.  All arithmetic is exact (``fractions.Fraction``).
"""
from __future__ import annotations

from fractions import Fraction


class Dual:
    """a + b*eps with eps^2 = 0, over Fractions."""

    __slots__ = ("a", "b")

    def __init__(self, a, b=0):
        self.a = Fraction(a)
        self.b = Fraction(b)

    def _lift(self, o):
        return o if isinstance(o, Dual) else Dual(o)

    def __add__(self, o):
        o = self._lift(o)
        return Dual(self.a + o.a, self.b + o.b)

    __radd__ = __add__

    def __sub__(self, o):
        o = self._lift(o)
        return Dual(self.a - o.a, self.b - o.b)

    def __mul__(self, o):
        o = self._lift(o)
        return Dual(self.a * o.a, self.a * o.b + self.b * o.a)

    __rmul__ = __mul__

    def __truediv__(self, o):
        o = self._lift(o)
        return Dual(self.a / o.a, (self.b * o.a - self.a * o.b) / (o.a * o.a))


def forward(q, k, v, S_in, z_in):
    """q, k, v: T x D nested lists; S_in: D x D; z_in: D (Fractions or Duals).

    Returns o (T x D), S_out (D x D), z_out (D)."""
    T = len(q)
    D = len(S_in)
    o = []
    S_t = [row[:] for row in S_in]
    z_t = list(z_in)
    for t in range(T):
        S_t = [[S_in[p][c] + sum((k[j][p] * v[j][c] for j in range(t + 1)), Fraction(0))
                for c in range(D)] for p in range(D)]
        z_t = [z_in[p] + sum((k[j][p] for j in range(t + 1)), Fraction(0)) for p in range(D)]
        den = sum((q[t][p] * z_t[p] for p in range(D)), Fraction(0))
        o.append([sum((q[t][p] * S_t[p][c] for p in range(D)), Fraction(0)) / den for c in range(D)])
    return o, S_t, z_t


def loss(q, k, v, S_in, z_in, dO, dS_out, dz_out):
    o, S, z = forward(q, k, v, S_in, z_in)
    T, D = len(q), len(S_in)
    L = Fraction(0)
    for t in range(T):
        for c in range(D):
            L = dO[t][c] * o[t][c] + L
    for p in range(D):
        for c in range(D):
            L = dS_out[p][c] * S[p][c] + L
        L = dz_out[p] * z[p] + L
    return L


def gradients(q, k, v, S_in, z_in, dO, dS_out, dz_out):
    """Exact dL/d(q, k, v, S_in, z_in) by one dual-number forward per input coordinate."""
    T, D = len(q), len(S_in)
    names = ("q", "k", "v", "S_in", "z_in")
    base = {"q": q, "k": k, "v": v, "S_in": S_in, "z_in": z_in}
    shapes = {"q": (T, D), "k": (T, D), "v": (T, D), "S_in": (D, D), "z_in": (D,)}
    grads = {}
    for name in names:
        shp = shapes[name]
        idxs = [(i,) for i in range(shp[0])] if len(shp) == 1 else \
            [(i, j) for i in range(shp[0]) for j in range(shp[1])]
        g = [[None] * shp[1] for _ in range(shp[0])] if len(shp) == 2 else [None] * shp[0]
        for idx in idxs:
            args = {}
            for n in names:
                src = base[n]
                if len(shapes[n]) == 1:
                    args[n] = [Dual(x) for x in src]
                else:
                    args[n] = [[Dual(x) for x in row] for row in src]
            if len(idx) == 1:
                args[name][idx[0]] = Dual(base[name][idx[0]], 1)
            else:
                args[name][idx[0]][idx[1]] = Dual(base[name][idx[0]][idx[1]], 1)
            L = loss(args["q"], args["k"], args["v"], args["S_in"], args["z_in"], dO, dS_out, dz_out)
            if len(idx) == 1:
                g[idx[0]] = L.b
            else:
                g[idx[0]][idx[1]] = L.b
        grads[name] = g
    return grads
