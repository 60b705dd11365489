"""Exact-arithmetic scalar reference used to pin the oracle on tiny inputs.

Everything here works element by element with Python ``Fraction`` and ints:
the exact result of one hop is rounded to the target format by the textbook
definition of round-to-nearest-even (significand of p bits, minimum exponent
emin, gradual underflow). It shares nothing with ``oracle/ring.py``: the
partition is computed per element in closed form and the arithmetic never
touches NumPy float kernels.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

FORMATS = {
    # name: (precision p incl. hidden bit, emin, emax)
    "float32": (24, -126, 127),
    "bfloat16": (8, -126, 127),
}
INT_BITS = {"int32": 32, "int64": 64}


class XVal:
    """A finite float as (exact value, sign bit); the sign bit keeps -0."""

    __slots__ = ("q", "neg")

    def __init__(self, q: Fraction, neg: bool):
        self.q = q
        self.neg = neg

    def __repr__(self):
        return f"XVal({self.q}, neg={self.neg})"


INF = "inf"


def decode(bits: int, dtype: str) -> XVal:
    if dtype == "float32":
        f = struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0]
    elif dtype == "bfloat16":
        f = struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]
    else:
        raise ValueError(dtype)
    if math.isinf(f) or math.isnan(f):
        raise ValueError("finite values only")
    return XVal(Fraction(f), math.copysign(1.0, f) < 0)


def round_exact(q: Fraction, dtype: str):
    """Round an exact value to the format, nearest-even. Returns a Fraction or
    the string ``"inf"`` / ``"-inf"`` on overflow."""
    p, emin, emax = FORMATS[dtype]
    if q == 0:
        return Fraction(0)
    neg = q < 0
    a = -q if neg else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    e = max(e, emin)
    ulp = Fraction(2) ** (e - p + 1)
    m = a / ulp
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    res = n * ulp
    if res >= Fraction(2) ** (emax + 1):
        return "-inf" if neg else "inf"
    return -res if neg else res


def encode(q, neg_zero: bool, dtype: str) -> int:
    if q == "inf" or q == "-inf":
        f = math.inf if q == "inf" else -math.inf
    elif q == 0:
        f = -0.0 if neg_zero else 0.0
    else:
        f = float(q)  # exact: q is representable in float32
    u = struct.unpack("<I", struct.pack("<f", f))[0]
    if dtype == "float32":
        return u
    assert u & 0xFFFF == 0
    return u >> 16


def hop_float(a_bits: int, b_bits: int, op: str, dtype: str) -> int:
    """Exact op(a, b) rounded once to ``dtype`` (IEEE semantics, finite inputs)."""
    a = decode(a_bits, dtype)
    b = decode(b_bits, dtype)
    if op in ("max", "min"):
        if a.q != b.q:
            pick_a = (a.q > b.q) == (op == "max")
            return a_bits if pick_a else b_bits
        if a.q == 0:
            # -0 < +0: max is -0 only if both are -0; min is -0 if either is
            neg = (a.neg and b.neg) if op == "max" else (a.neg or b.neg)
            return encode(Fraction(0), neg, dtype)
        return a_bits
    if op == "sum":
        q = a.q + b.q
        if q == 0:
            # exact zero: -0 only when both operands are -0 (round-to-nearest)
            return encode(Fraction(0), a.neg and b.neg and a.q == 0 and b.q == 0, dtype)
        r = round_exact(q, dtype)
        return encode(r, False, dtype)
    if op == "prod":
        neg = a.neg != b.neg
        q = a.q * b.q
        r = round_exact(q, dtype)
        if r == 0:
            return encode(Fraction(0), neg, dtype)
        return encode(r, False, dtype)
    raise ValueError(op)


def hop_int(a: int, b: int, op: str, dtype: str) -> int:
    bits = INT_BITS[dtype]
    if op == "sum":
        v = a + b
    elif op == "prod":
        v = a * b
    elif op == "max":
        v = max(a, b)
    elif op == "min":
        v = min(a, b)
    else:
        raise ValueError(op)
    half = 1 << (bits - 1)
    return ((v + half) % (1 << bits)) - half


def to_scalar_list(arr, dtype: str) -> list[int]:
    """Host array -> list of Python ints (bit patterns for floats)."""
    import numpy as np

    if dtype == "float32":
        return [int(v) for v in np.asarray(arr, dtype=np.float32).view(np.uint32)]
    if dtype == "bfloat16":
        return [int(v) for v in np.asarray(arr, dtype=np.uint16)]
    return [int(v) for v in arr]


def hop(a: int, b: int, op: str, dtype: str) -> int:
    if dtype in INT_BITS:
        return hop_int(a, b, op, dtype)
    return hop_float(a, b, op, dtype)


# Per-element closed form of the partition -----------------------------------

def ceil_div(x: int, y: int) -> int:
    return (x + y - 1) // y


def ar_chunk_id(e: int, count: int, nranks: int, nchannels: int, chunk: int, align: int) -> int:
    """Chunk id of element e: channel by e // per, loop by position // (N*chunk),
    chunk by offset // (chunk size of that loop), written per element."""
    per = ceil_div(ceil_div(count, nchannels), align) * align
    c = e // per
    local = e - c * per
    length = min(per, count - c * per)
    loop = nranks * chunk
    l = local // loop
    rem = length - l * loop
    cur = chunk if rem >= loop else ceil_div(ceil_div(rem, nranks), align) * align
    return (local - l * loop) // cur


def brute_allreduce(values: list[list[int]], op: str, dtype: str, nchannels: int, chunk: int,
                    align: int) -> list[int]:
    """Result (same on every rank) of the ring all-reduce, one element at a time:
    chunk k is folded in rank order k+1, k+2, ..., k."""
    n = len(values)
    count = len(values[0])
    if n == 1:
        return list(values[0])
    res = []
    for e in range(count):
        k = ar_chunk_id(e, count, n, nchannels, chunk, align)
        acc = values[(k + 1) % n][e]
        for t in range(2, n + 1):
            acc = hop(acc, values[(k + t) % n][e], op, dtype)
        res.append(acc)
    return res


def brute_reduce_block(values: list[list[int]], block: int, blocklen: int, op: str, dtype: str) -> list[int]:
    """Block ``block`` folded in rank order block+1, ..., block."""
    n = len(values)
    out = []
    for i in range(blocklen):
        e = block * blocklen + i
        acc = values[(block + 1) % n][e]
        for t in range(2, n + 1):
            acc = hop(acc, values[(block + t) % n][e], op, dtype)
        out.append(acc)
    return out
