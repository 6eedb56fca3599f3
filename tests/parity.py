"""Comparison of GPU indices with the CPU oracle (test infrastructure).

Acceptance rule for a row (stated with the encode contract): the GPU index
must equal the oracle's, except where the oracle's best and second-best fp32
distances differ by at most 1e-6 * max(1, best) (a near-tie); there the
oracle's distance to the GPU's choice must be within 1e-6 * max(1, best) of
the best.  Stricter self-check: when best and second-best are bit-equal (an
exact tie) the GPU must return the oracle's (lowest) index.  Sentinel
indices for bad codebook slots must match exactly.
"""
from __future__ import annotations

import dataclasses
import os

import numpy as np

import oracle

NEAR_TIE_REL = 1e-6


def oracle_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


@dataclasses.dataclass
class ParityReport:
    rows: int
    equal: int
    near_tie_ok: int
    failures: list

    @property
    def ok(self) -> bool:
        return not self.failures

    def summary(self) -> str:
        return (f"rows={self.rows} equal={self.equal} near_tie_accepted={self.near_tie_ok} "
                f"failures={len(self.failures)} {self.failures[:5]}")


def oracle_indices(wl, rows=None, threads=None):
    kw = wl.kwargs()
    if rows is None:
        return oracle.encode(wl.x, wl.codebook, wl.sub_dim, wl.n_centroids, wl.dtype,
                             threads=threads or oracle_threads(), **kw)
    return _rows_threaded(wl, np.asarray(rows, np.int64), threads or oracle_threads())


def _rows_threaded(wl, rows, threads):
    import threading
    out = np.empty(rows.size, np.uint32)
    parts = np.array_split(np.arange(rows.size), max(1, min(threads, rows.size)))

    def work(p):
        out[p] = oracle.encode_rows(wl.x, wl.codebook, rows[p], wl.sub_dim, wl.n_centroids,
                                    wl.dtype, **wl.kwargs())

    ts = [threading.Thread(target=work, args=(p,)) for p in parts if p.size]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    return out


def compare(wl, gpu_idx, rows=None, ref_idx=None) -> ParityReport:
    """Check GPU indices (for ``rows`` of the workload, or all rows)."""
    gpu_idx = np.asarray(gpu_idx, np.uint32).reshape(-1)
    sel = np.arange(wl.n) if rows is None else np.asarray(rows, np.int64)
    got = gpu_idx if rows is None else gpu_idx[sel]
    ref = oracle_indices(wl, None if rows is None else sel) if ref_idx is None else ref_idx
    bad = np.nonzero(got != ref)[0]
    failures = []
    near = 0
    if bad.size:
        brow = sel[bad]
        ridx, best, second = oracle.encode_rows(wl.x, wl.codebook, brow, wl.sub_dim,
                                                wl.n_centroids, wl.dtype, want_top2=True,
                                                **wl.kwargs())
        for k, r in enumerate(brow):
            g = int(got[bad[k]])
            if ref[bad[k]] == oracle.BAD_SLOT or g == oracle.BAD_SLOT or g >= wl.n_centroids:
                failures.append((int(r), "sentinel/range", int(ref[bad[k]]), g))
                continue
            b, s = float(best[k]), float(second[k])
            tol = NEAR_TIE_REL * max(1.0, b)
            if s == b:
                failures.append((int(r), "exact tie not resolved to lowest index",
                                 int(ref[bad[k]]), g))
                continue
            if not (s - b <= tol):
                failures.append((int(r), "not a near-tie", int(ref[bad[k]]), g, b, s))
                continue
            dg = float(oracle.sqdist_rows(wl.x, wl.codebook, [r], [g], wl.sub_dim, wl.dtype,
                                          codebook_stride=wl.codebook_stride,
                                          group_len=wl.group_len, group_map=wl.group_map,
                                          n_centroids=wl.n_centroids)[0])
            if abs(dg - b) <= tol:
                near += 1
            else:
                failures.append((int(r), "near-tie choice too far", int(ref[bad[k]]), g, b, dg))
    return ParityReport(int(sel.size), int(sel.size - bad.size), near, failures)
