"""Exact rational brute force for tiny cases (pure Python, fractions.Fraction).

TEST INFRASTRUCTURE ONLY. It takes the codes q(n,k) themselves (not packed
words), so a test that builds the words with an independent packer checks the
float64 oracle's unpack and its arithmetic at once.

It evaluates the definition y(m,n) = sum_k x(m,k) * (scale(n,k/gs)*q(n,k) +
bias(n,k/gs)) with no rounding at all [P1 "@mlx-bun/inference 0.0.0-stage ->
1.0.0", affine3-mma.ts: weight = fma(scale, q, bias); affine-split-mma.ts
header: y = x . W^T].
"""
from __future__ import annotations

from fractions import Fraction


def exact_matmul(x_rows, codes_rows, scales_rows, biases_rows, group_size=64):
    """All arguments are nested lists of Python floats/ints (floats are exact
    binary values, so Fraction(v) is exact). Returns [M][N] Fractions."""
    out = []
    for xr in x_rows:
        xf = [Fraction(v) for v in xr]
        row = []
        for qr, sr, br in zip(codes_rows, scales_rows, biases_rows):
            acc = Fraction(0)
            for k, q in enumerate(qr):
                g = k // group_size
                acc += xf[k] * (Fraction(sr[g]) * q + Fraction(br[g]))
            row.append(acc)
        out.append(row)
    return out
