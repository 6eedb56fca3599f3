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
                    of slot s assigned to c, rounded once to fp16 (round to
                    nearest, ties to even); a centroid with no member keeps
                    its value

The mean is exact: fp16 values are integer multiples of 2^-24, so the sum of
the members is an exact integer multiple of 2^-24 (Python integers), and the
one rounding of sum / count to fp16 is done on that exact rational.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import oracle

F16 = 0


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


def f16_units(bits: np.ndarray) -> np.ndarray:
    """Exact integer value of fp16 elements in units of 2^-24 (int64)."""
    bits = np.asarray(bits, dtype=np.uint16)
    v = bits.view(np.float16).astype(np.float64) * float(2 ** 24)
    return v.astype(np.int64)          # exact: |v| < 2^40


def update(x, idx, codebook, sub_dim, n_centroids, *, codebook_stride=None, n_codebooks=1,
           group_len=None, group_map=None):
    """One Lloyd update from assignments `idx` (returns new codebook bits,
    and the member count of every (slot, centroid))."""
    x = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1, sub_dim)
    n = x.shape[0]
    stride = n_centroids * sub_dim if codebook_stride is None else codebook_stride
    glen = max(n, 1) if group_len is None else group_len
    cb = np.array(codebook, dtype=np.uint16, copy=True).reshape(-1)
    g = np.arange(n) // glen
    slots = (np.asarray(group_map)[g] if group_map is not None else g).astype(np.int64)
    units = f16_units(x)
    counts = np.zeros((n_codebooks, n_centroids), dtype=np.int64)
    for s in range(n_codebooks):
        rows = (slots == s) & (idx.astype(np.int64) < n_centroids)
        for c in range(n_centroids):
            members = rows & (idx == c)
            cnt = int(members.sum())
            counts[s, c] = cnt
            if cnt == 0:
                continue                # empty cluster keeps its centroid
            total = units[members].sum(axis=0, dtype=np.int64)   # exact
            for i in range(sub_dim):
                q = Fraction(int(total[i]), cnt * 2 ** 24)
                cb[s * stride + c * sub_dim + i] = f16_round(q)
    return cb, counts


def kmeans(x, codebook, sub_dim, n_centroids, iterations, *, codebook_stride=None, n_codebooks=1,
           group_len=None, group_map=None, threads=1):
    """Lloyd iterations; returns (codebook bits, final assignment, counts of
    the last update).  The assignment returned is that of the last codebook
    used for an update (the encode at the start of the last iteration)."""
    cb = np.array(codebook, dtype=np.uint16, copy=True).reshape(-1)
    kw = dict(codebook_stride=codebook_stride, n_codebooks=n_codebooks, group_len=group_len,
              group_map=group_map)
    idx = None
    counts = None
    for _ in range(iterations):
        idx = oracle.encode(x, cb, sub_dim, n_centroids, F16, threads=threads, **kw)
        cb, counts = update(x, idx, cb, sub_dim, n_centroids, **kw)
    return cb, idx, counts


def inertia(x, codebook, idx, sub_dim, n_centroids, *, codebook_stride=None, group_len=None,
            group_map=None):
    """sum_n |x_n - c_idx(n)|^2 in float64 (for reports and monotonicity)."""
    x = np.asarray(x, dtype=np.uint16).reshape(-1, sub_dim).view(np.float16).astype(np.float64)
    n = x.shape[0]
    stride = n_centroids * sub_dim if codebook_stride is None else codebook_stride
    glen = max(n, 1) if group_len is None else group_len
    g = np.arange(n) // glen
    slots = (np.asarray(group_map)[g] if group_map is not None else g).astype(np.int64)
    cb = np.asarray(codebook, dtype=np.uint16).view(np.float16).astype(np.float64)
    rows = cb[(slots * stride)[:, None] + (idx.astype(np.int64) * sub_dim)[:, None]
              + np.arange(sub_dim)[None, :]]
    return float(((x - rows) ** 2).sum())
