"""Exact rational brute force for tiny weight-quantized GEMMs.

TEST INFRASTRUCTURE ONLY. Every value is a ``fractions.Fraction`` built from
the exact binary value of the stored fp16/fp32 number, so the sums carry no
rounding at all. Used to pin the fp64 oracle on tiny shapes: the oracle must
agree to ~1e-12 relative, which a dropped term, a wrong index, a transposed
operand or a wrong nibble order would break by many orders of magnitude.

The definitions are those of the MNN GemmSpeed benchmark page, section "Why
Conv1x1 is used to measure GEMM" (C = A x B, w = offset + scale*q, pairs
[offset, scale]); codes are decoded here from the canonical storage by
integer arithmetic on the page's "low nibble first" reading.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def exact(x) -> Fraction:
    """Exact rational value of a finite binary float (fp16/fp32/fp64)."""
    return Fraction(float(x))


def code(q: np.ndarray, bits: int, n: int, k: int) -> int:
    if bits == 8:
        return int(q[n, k])
    byte = int(q[n, k // 2])
    return (byte >> 4) if (k % 2) else (byte & 0xF)


def gemm_f32(A: np.ndarray, B: np.ndarray):
    M, K = A.shape
    N = B.shape[1]
    return [[sum((exact(A[m, k]) * exact(B[k, n]) for k in range(K)), Fraction(0))
             for n in range(N)] for m in range(M)]


def gemm_blockq(A: np.ndarray, q: np.ndarray, pairs: np.ndarray, bits: int, block: int):
    M, K = A.shape
    N = q.shape[0]
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                b = k // block
                w = exact(pairs[n, b, 0]) + exact(pairs[n, b, 1]) * code(q, bits, n, k)
                s += exact(A[m, k]) * w
            row.append(s)
        out.append(row)
    return out


def to_array(rows) -> np.ndarray:
    return np.array([[float(v) for v in r] for r in rows], dtype=np.float64)
