"""Writes tests/golden/tiny_exact.json from the exact rational oracle (oracle.exact) only.

Each case is a tiny chunk with small rational inputs: q and k strictly positive
(the positive feature map that "Fractus-1B training optimization" assumes for
its linear attention), v, dO and the upstream carry gradient small integers.
Its expected values are exact fractions: the forward from the literal prefix-sum
definition (section 1, Bottleneck #1) and the gradients as exact derivatives of
the scalar loss, so no floating-point code is involved in writing them.

Run:  python tests/golden/make_golden.py
"""
import json
import os
import random
import sys
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import exact  # noqa: E402

POS = [Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(5, 2), Fraction(3)]
INTS = [Fraction(i) for i in range(-3, 4)]


def case(name, T, D, seed, carry, upstream):
    rnd = random.Random(seed)
    q = [[rnd.choice(POS) for _ in range(D)] for _ in range(T)]
    k = [[rnd.choice(POS) for _ in range(D)] for _ in range(T)]
    v = [[rnd.choice(INTS) for _ in range(D)] for _ in range(T)]
    dO = [[rnd.choice(INTS) for _ in range(D)] for _ in range(T)]
    if carry:
        # a carry built as if from two earlier tokens: z_in > 0, S_in = sum kp vp^T
        kp = [[rnd.choice(POS) for _ in range(D)] for _ in range(2)]
        vp = [[rnd.choice(INTS) for _ in range(D)] for _ in range(2)]
        S_in = [[sum((kp[j][p] * vp[j][c] for j in range(2)), Fraction(0)) for c in range(D)]
                for p in range(D)]
        z_in = [sum((kp[j][p] for j in range(2)), Fraction(0)) for p in range(D)]
    else:
        S_in = [[Fraction(0)] * D for _ in range(D)]
        z_in = [Fraction(0)] * D
    if upstream:
        dS_out = [[rnd.choice(INTS) for _ in range(D)] for _ in range(D)]
        dz_out = [rnd.choice(INTS) for _ in range(D)]
    else:
        dS_out = [[Fraction(0)] * D for _ in range(D)]
        dz_out = [Fraction(0)] * D
    o, S_out, z_out = exact.forward(q, k, v, S_in, z_in)
    g = exact.gradients(q, k, v, S_in, z_in, dO, dS_out, dz_out)

    def enc(x):
        if isinstance(x, list):
            return [enc(y) for y in x]
        return str(x)

    return {
        "name": name, "T": T, "D": D, "carry": carry, "upstream": upstream,
        "inputs": {"q": enc(q), "k": enc(k), "v": enc(v), "S_in": enc(S_in), "z_in": enc(z_in),
                   "dO": enc(dO), "dS_out": enc(dS_out), "dz_out": enc(dz_out)},
        "expected": {"o": enc(o), "S_out": enc(S_out), "z_out": enc(z_out),
                     "dq": enc(g["q"]), "dk": enc(g["k"]), "dv": enc(g["v"]),
                     "dS_in": enc(g["S_in"]), "dz_in": enc(g["z_in"])},
    }


def main():
    cases = [
        case("t3_d2_carry_upstream", 3, 2, seed=1, carry=True, upstream=True),
        case("t4_d3_zero_carry", 4, 3, seed=2, carry=False, upstream=False),
        case("t5_d2_carry", 5, 2, seed=3, carry=True, upstream=False),
    ]
    doc = {
        "source": "exact rational evaluation of the prefix-sum definition and of the exact "
                  "derivatives of L = sum <dO,o> + <dS_out,S_out> + dz_out.z_out "
                  "(oracle/exact.py); written by tests/golden/make_golden.py",
        "cases": cases,
    }
    with open(os.path.join(HERE, "tiny_exact.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
