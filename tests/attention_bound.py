"""The acceptance bound of decode attention against the float64 oracle, and
inputs that make it bite.  Test infrastructure: the GPU parity tests and the
CPU sensitivity tests use the same bound.

The pages give no tolerance for attention over VQ codes (post "I Wrote a
Metal Kernel to Stop My Mac From OOMing", section "What's Next: Phase 2"), so
the bound is derived from the fp32 arithmetic of any evaluation order:

  score error (natural-log units)  Delta <= 1.5 (sd_k + n_sub_k + 4) u A
      A = scale * max_t sum_i |q_i k_ti|: the lookup entry is an sd_k-term
      fp32 dot product, the score a sum of n_sub_k entries, plus q / f, the
      scale * log2(e) multiply and the base change (4 roundings);
  |out - ref|  <=  (2 Delta + (3 T + 32) u) * M_d  (+ 1e-30)
      M_d = sum_t p_t |v_td|; T attended tokens: exp2 and its input
      roundings, the fp32 sums of weights and of weighted values in any
      order, the chunk rescales.

A, T and M come from ``oracle.attention.tolerance_terms``.
"""
from __future__ import annotations

import numpy as np

U = 2.0 ** -24


def relative_bound(A, T, sdk: int, n_sub_k: int):
    """Per (b, hq): the bound on |out - ref| in units of M_d."""
    delta = 1.5 * (sdk + n_sub_k + 4) * U * np.asarray(A, dtype=np.float64)
    return 2 * delta + (3 * np.asarray(T, dtype=np.float64) + 32) * U


def bound(A, T, M, sdk: int, n_sub_k: int):
    """Per (b, hq, d): the largest |out - ref| the fp32 arithmetic allows."""
    return relative_bound(A, T, sdk, n_sub_k)[:, :, None] * M + 1e-30


def chunk_boundaries(L: int, chunk: int = 256):
    """Token positions on either side of every chunk boundary of a length-L
    sequence, plus its first and last token."""
    pos = {0, L - 1}
    for c in range(chunk, L, chunk):
        pos.update((c - 1, c))
    return sorted(p for p in pos if 0 <= p < L)


def make_boundary_tokens_heavy(wl, chunk: int = 256):
    """Give the tokens next to every chunk boundary the key that scores
    highest for the first query head of each group, so that they carry most
    of that head's attention: a kernel that drops, repeats or misweights a
    boundary token then moves the output far past the bound.  Works in place
    on the workload's key codes; returns the positions per sequence."""
    from oracle.attention import widen
    B, Hq, Hkv, D, S = wl.shape
    g = Hq // Hkv
    n_sub = wl.k_codes.shape[3]
    sd = D // n_sub
    q = widen(wl.q, wl.dtype)
    out = []
    for b in range(B):
        L = int(wl.kv_len[b])
        t0 = max(0, L - wl.window) if wl.window else 0
        pos = [t0 + p for p in chunk_boundaries(L - t0, chunk)] if L > t0 else []
        for h in range(Hkv):
            cb = widen(wl.k_codebook[h], wl.dtype)                  # [n_c, sd]
            qt = q[b, h * g].copy()
            if wl.k_scale is not None:
                qt = qt / wl.k_scale[h].astype(np.float64)
            best = [int(np.argmax(cb @ qt[s * sd:(s + 1) * sd])) for s in range(n_sub)]
            for t in pos:
                wl.k_codes[b, h, t] = best
        out.append(pos)
    return out
