"""CPU oracle for K-means codebook calibration -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; it shares no code with the HIP library.

What it computes (VeloxQuant-MLX blog, "I Wrote a Metal Kernel to Stop My Mac
From OOMing", section "What Even Is a KV Cache And Why Should You Care", step
2: the codebook is a set of K-means centroids pre-trained on calibration data;
blog index, "Where KIVI fits": VecInfer needs a short codebook calibration).
The pages name K-means and nothing more; the reading taken is Lloyd's
algorithm from a given initial codebook, for a given number of iterations,
every codebook slot trained on the sub-vectors of its own groups:

    repeat `iterations` times:
        assignment: idx = the encode of every sub-vector against the current
                    codebook (nearest centroid, fp32 distance, lowest index on
                    ties -- the pinned ``oracle.encode``)
        update:     centroid c of slot s = the exact mean of the sub-vectors
                    of slot s assigned to c, rounded once to the element type
                    (fp16 or bf16; round to nearest, ties to even); a centroid
                    with no member keeps its value

The mean is exact: every finite fp16 value is an integer multiple of 2^-24
and every finite bf16 value one of 2^-133, so the sum of the members is an
exact integer multiple of that unit (Python integers), and the one rounding
of sum / count is done on that exact rational.  A non-finite component
(infinity, NaN) adds 0 to its sum; its row still counts as a member.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import oracle

F16 = 0
BF16 = 1
# the smallest subnormal of each element type, as a power of two: the unit of
# the exact integer sums
UNIT_LOG2 = {F16: 24, BF16: 133}


def f16_round(q: Fraction) -> int:
    """fp16 bits of the exact rational q rounded to nearest, ties to even
    (written from the binary16 format: 1 sign, 5 exponent, 10 fraction bits,
    subnormal spacing 2^-24, largest finite 65504, beyond which +-inf)."""
    sign = 0x8000 if q < 0 else 0
    a = -q if q < 0 else q
    if a == 0:
        return sign
    # exponent e with 2^e <= a < 2^(e+1), clamped to the subnormal range
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -14)
    ulp = Fraction(2) ** (e - 10)
    m_floor = int(a / ulp)            # a / ulp >= 0
    rem = a / ulp - m_floor
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m_floor % 2 == 1):
        m_floor += 1
    if m_floor == 2048:               # rounding carried into the next binade
        m_floor = 1024
        e += 1
    if e > 15:
        return sign | 0x7C00          # overflow to infinity
    if m_floor < 1024:                # subnormal (e == -14)
        return sign | m_floor
    return sign | ((e + 15) << 10) | (m_floor - 1024)


def bf16_round(q: Fraction) -> int:
    """bf16 bits of the exact rational q rounded to nearest, ties to even
    (written from the bfloat16 format: 1 sign, 8 exponent bits with bias 127,
    7 fraction bits, subnormal spacing 2^-133, largest finite (2 - 2^-7) 2^127,
    beyond which +-inf)."""
    sign = 0x8000 if q < 0 else 0
    a = -q if q < 0 else q
    if a == 0:
        return sign
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 7)
    m_floor = int(a / ulp)
    rem = a / ulp - m_floor
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m_floor % 2 == 1):
        m_floor += 1
    if m_floor == 256:                # rounding carried into the next binade
        m_floor = 128
        e += 1
    if e > 127:
        return sign | 0x7F80          # overflow to infinity
    if m_floor < 128:                 # subnormal (e == -126)
        return sign | m_floor
    return sign | ((e + 127) << 7) | (m_floor - 128)


def f16_units(bits: np.ndarray) -> np.ndarray:
    """Exact integer value of fp16 elements in units of 2^-24 (int64; a
    non-finite element gives 0)."""
    bits = np.asarray(bits, dtype=np.uint16)
    v = bits.view(np.float16).astype(np.float64)
    v = np.where(np.isfinite(v), v, 0.0) * float(2 ** 24)
    return v.astype(np.int64)          # exact: |v| < 2^40


def bf16_terms(bits: np.ndarray):
    """Exact value of bf16 elements as m * 2^p in units of 2^-133: the signed
    significand m (int64) and the shift p (a normal element with exponent
    field E and fraction F is (128 + F) 2^(E - 134) = (128 + F) 2^(E - 1)
    units; a subnormal is F units; a non-finite element gives m = 0)."""
    bits = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    E = (bits >> 7) & 0xFF
    F = bits & 0x7F
    m = np.where(E == 0, F, 128 + F)
    m = np.where(E == 255, 0, m)
    p = np.where(E == 0, 0, E - 1)
    m = np.where(bits & 0x8000, -m, m)
    return m, p


def exact_sum(bits: np.ndarray, dtype: int) -> int:
    """Exact sum of elements in units of 2^-UNIT_LOG2[dtype] (Python int)."""
    if dtype == F16:
        return int(f16_units(bits).sum(dtype=np.int64))   # |sum| < 2^63 for <= 2^23 members
    m, p = bf16_terms(bits)
    total = 0
    for sh in np.unique(p):            # the terms grouped by their power of two
        total += int(m[p == sh].sum(dtype=np.int64)) << int(sh)
    return total


def update(x, idx, codebook, sub_dim, n_centroids, dtype=F16, *, codebook_stride=None,
           n_codebooks=1, group_len=None, group_map=None):
    """One Lloyd update from assignments `idx` (returns new codebook bits,
    and the member count of every (slot, centroid))."""
    x = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1, sub_dim)
    n = x.shape[0]
    stride = n_centroids * sub_dim if codebook_stride is None else codebook_stride
    glen = max(n, 1) if group_len is None else group_len
    cb = np.array(codebook, dtype=np.uint16, copy=True).reshape(-1)
    g = np.arange(n) // glen
    slots = (np.asarray(group_map)[g] if group_map is not None else g).astype(np.int64)
    idx = np.asarray(idx).astype(np.int64)
    unit = 2 ** UNIT_LOG2[dtype]
    rounding = f16_round if dtype == F16 else bf16_round
    counts = np.zeros((n_codebooks, n_centroids), dtype=np.int64)
    for s in range(n_codebooks):
        rows = np.nonzero((slots == s) & (idx < n_centroids))[0]
        rows = rows[np.argsort(idx[rows], kind="stable")]       # members grouped by centroid
        cents, first = np.unique(idx[rows], return_index=True)
        last = np.append(first[1:], rows.size)
        for c, a, b in zip(cents, first, last):                 # empty clusters keep theirs
            members = rows[a:b]
            cnt = int(b - a)
            counts[s, c] = cnt
            for i in range(sub_dim):
                total = exact_sum(x[members, i], dtype)
                q = Fraction(total, cnt * unit)
                cb[s * stride + c * sub_dim + i] = rounding(q)
    return cb, counts


def kmeans(x, codebook, sub_dim, n_centroids, iterations, *, dtype=F16, codebook_stride=None,
           n_codebooks=1, group_len=None, group_map=None, threads=1):
    """Lloyd iterations; returns (codebook bits, final assignment, counts of
    the last update).  The assignment returned is that of the last codebook
    used for an update (the encode at the start of the last iteration)."""
    cb = np.array(codebook, dtype=np.uint16, copy=True).reshape(-1)
    kw = dict(codebook_stride=codebook_stride, n_codebooks=n_codebooks, group_len=group_len,
              group_map=group_map)
    idx = None
    counts = None
    for _ in range(iterations):
        idx = oracle.encode(x, cb, sub_dim, n_centroids, dtype, threads=threads, **kw)
        cb, counts = update(x, idx, cb, sub_dim, n_centroids, dtype, **kw)
    return cb, idx, counts


def widen(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Element bits -> float64 (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def inertia(x, codebook, idx, sub_dim, n_centroids, *, dtype=F16, codebook_stride=None,
            group_len=None, group_map=None):
    """sum_n |x_n - c_idx(n)|^2 in float64 (for reports and monotonicity)."""
    x = widen(x, dtype).reshape(-1, sub_dim)
    n = x.shape[0]
    stride = n_centroids * sub_dim if codebook_stride is None else codebook_stride
    glen = max(n, 1) if group_len is None else group_len
    g = np.arange(n) // glen
    slots = (np.asarray(group_map)[g] if group_map is not None else g).astype(np.int64)
    cb = widen(codebook, dtype)
    rows = cb[(slots * stride)[:, None] + (idx.astype(np.int64) * sub_dim)[:, None]
              + np.arange(sub_dim)[None, :]]
    return float(((x - rows) ** 2).sum())
