"""Exact rational brute force of the quantized projections (test infrastructure).

Pure Python ``fractions.Fraction`` arithmetic for tiny shapes: every bf16 is
decoded from its bit pattern into an exact rational, every code is read from
its packed word, and the sums carry no rounding at all.  Used to pin the
float64 oracle (which must agree to float64 rounding) and to check the
per-group decomposition identity exactly.

Same definition as the C oracle (affine weights ``w = s*q + b`` per group of
``gs`` codes along K; codes least significant first in each uint32 word), but
written independently of it.
"""
from __future__ import annotations

from fractions import Fraction


def bf16_exact(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern."""
    bits = int(bits) & 0xFFFF
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    if exp == 0xFF:
        raise ValueError("non-finite bf16")
    if exp == 0:                       # subnormal: man * 2^(-126-7)
        return sign * Fraction(man, 1 << 133)
    return sign * Fraction(128 + man, 128) * (Fraction(2) ** (exp - 127))


def f16_exact(bits: int) -> Fraction:
    """Exact value of a finite IEEE binary16 bit pattern (1 sign, 5 exponent
    bits with bias 15, 10 fraction bits)."""
    bits = int(bits) & 0xFFFF
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 10) & 0x1F
    man = bits & 0x3FF
    if exp == 0x1F:
        raise ValueError("non-finite binary16")
    if exp == 0:                       # subnormal: man * 2^(-14-10)
        return sign * Fraction(man, 1 << 24)
    return sign * Fraction(1024 + man, 1024) * (Fraction(2) ** (exp - 15))


_DECODE = {"bf16": bf16_exact, "f16": f16_exact}


def code_at(words_row, k: int, bits: int) -> int:
    per = 32 // bits
    w = int(words_row[k // per])
    return (w >> (bits * (k % per))) & ((1 << bits) - 1)


def dequant_row(words_row, s_row, b_row, H: int, bits: int, gs: int, act: str = "bf16"):
    """Exact weights of one output feature (scales and biases of type ``act``)."""
    dec = _DECODE[act]
    return [dec(s_row[k // gs]) * code_at(words_row, k, bits) + dec(b_row[k // gs]) for k in range(H)]


def qmm_exact(x, W, S, B, M: int, H: int, N: int, bits: int, gs: int, act: str = "bf16"):
    """Exact ``y[m][n] = sum_k x[m,k] w[n,k]`` as a list of lists of Fractions
    (x, scales and biases of type ``act``: "bf16" or "f16")."""
    dec = _DECODE[act]
    xs = [[dec(x[m][k]) for k in range(H)] for m in range(M)]
    ws = [dequant_row(W[n], S[n], B[n], H, bits, gs, act) for n in range(N)]
    return [[sum((xs[m][k] * ws[n][k] for k in range(H)), Fraction(0)) for n in range(N)]
            for m in range(M)]


def qmm_grouped_exact(x, W, S, B, M: int, H: int, N: int, bits: int, gs: int):
    """The same projection through the per-group decomposition
    ``sum_g ( s_g * sum_{k in g} x_k q_k  +  b_g * sum_{k in g} x_k )``."""
    out = []
    for m in range(M):
        xs = [bf16_exact(x[m][k]) for k in range(H)]
        row = []
        for n in range(N):
            tot = Fraction(0)
            for g in range(H // gs):
                ks = range(g * gs, (g + 1) * gs)
                p = sum((xs[k] * code_at(W[n], k, bits) for k in ks), Fraction(0))
                sx = sum((xs[k] for k in ks), Fraction(0))
                tot += bf16_exact(S[n][g]) * p + bf16_exact(B[n][g]) * sx
            row.append(tot)
        out.append(row)
    return out


def qmm_sq_exact(x, W, S, B, M: int, H: int, N: int, bits: int, gs: int):
    """Exact ``sum_k (x[m,k] w[n,k])^2`` as a list of lists of Fractions: the
    square of the oracle's cancellation-free scale nu of each dot product."""
    xs = [[bf16_exact(x[m][k]) for k in range(H)] for m in range(M)]
    ws = [dequant_row(W[n], S[n], B[n], H, bits, gs) for n in range(N)]
    return [[sum(((xs[m][k] * ws[n][k]) ** 2 for k in range(H)), Fraction(0)) for n in range(N)]
            for m in range(M)]
