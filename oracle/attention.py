"""CPU oracle for decode attention over VQ-coded keys and values.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; the product path
never does, and it shares no code with the HIP library.

What it computes (VeloxQuant-MLX blog, post A "I Wrote a Metal Kernel to Stop
My Mac From OOMing", section "What's Next: Phase 2": attention computed from
the codebook indices of keys and values and the per-query transformed query,
never materializing fp16 keys, with the softmax-weighted value sum in the same
pass; blog index page, "The Kernel's Hot Path": the scores come from a lookup
table LUT[sub, centroid] = q_sub . codebook_row[centroid]).  Those passages
describe a way of computing ordinary attention over the quantized cache; the
oracle computes that attention from its plain definition, in float64:

  for sequence b and query head hq (key/value head h = hq // (Hq / Hkv), the
  grouped-query mapping), with L = kv_len[b] and the attended tokens
  t in [max(0, L - window), L) (window 0 = all L):
      k_t = codebook_k[h][k_codes[b, h, t, s]] for every sub-space s,
            concatenated (D = n_sub * sub_dim), then divided channel-wise by
            the smoothing factors f[h] (keys were stored smoothed, k~ = k * f)
      v_t = codebook_v[h][v_codes[b, h, t, s]] concatenated
      score_t = softmax_scale * (q[b, hq] . k_t)
      out[b, hq] = sum_t softmax(score)_t * v_t      (0 when no token)
  (a code >= n_centroids decodes to a zero row)

Every step is one library primitive (numpy gather, float64 matmul, exp) over
the definition; no blocking, chunking or reordering.  ``tolerance_terms``
returns the quantities the GPU comparison's error bound is built from.

Pinned by ``tests/test_oracle_attention.py`` against torch's float64
scaled-dot-product attention, closed forms (one token, equal keys, zero
query), the LUT identity, grouped-query and window brute force, and planted
mistakes.  ``tolerance_terms`` is pinned by
``tests/test_oracle_attention_bound.py``: hand-worked A, T and M (one token,
a window over a grouped-query group with closed-form weights, equal keys)
and planted mistakes in each of the three.
"""
from __future__ import annotations

import numpy as np

F16 = 0
BF16 = 1


def widen(bits: np.ndarray, dtype: int) -> np.ndarray:
    """fp16/bf16 element bits -> float64 (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _attended(L: int, window: int):
    start = max(0, L - window) if window > 0 else 0
    return start, L


def dequantize(codes: np.ndarray, codebook: np.ndarray, dtype: int) -> np.ndarray:
    """[T, n_sub] codes -> [T, n_sub * sub_dim] float64 rows of `codebook` [n_c, sd].
    A code >= n_c decodes to a row of zeros (as the encode library's gather
    does for an out-of-range index)."""
    cb = widen(codebook, dtype)
    codes = np.asarray(codes, dtype=np.int64)
    if codes.size and codes.max() >= cb.shape[0]:
        cb = np.vstack([cb, np.zeros((int(codes.max()) + 1 - cb.shape[0], cb.shape[1]))])
    return cb[codes].reshape(codes.shape[0], -1)


def decode_attention(q, k_codes, v_codes, k_codebook, v_codebook, dtype, *, k_scale=None,
                     kv_len=None, window=0, softmax_scale=None):
    """Attention output float64 [B, Hq, D].

    q           element bits [B, Hq, D]
    k_codes     uint8 [B, Hkv, S, D / k_sub_dim]
    v_codes     uint8 [B, Hkv, S, D / v_sub_dim]
    k_codebook  element bits [Hkv, n_c, k_sub_dim]; v_codebook likewise
    k_scale     float32 [Hkv, D] smoothing factors of the stored keys, or None
    kv_len      int [B] attended prefix length per sequence (None = S)
    """
    B, Hq, D = q.shape
    Hkv, S = k_codes.shape[1], k_codes.shape[2]
    g = Hq // Hkv
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(D)
    lens = np.full(B, S) if kv_len is None else np.asarray(kv_len)
    qf = widen(q, dtype)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        t0, t1 = _attended(int(lens[b]), window)
        if t1 <= t0:
            continue
        for h in range(Hkv):
            K = dequantize(k_codes[b, h, t0:t1], k_codebook[h], dtype)
            if k_scale is not None:
                K = K / np.asarray(k_scale[h], dtype=np.float64)[None, :]
            V = dequantize(v_codes[b, h, t0:t1], v_codebook[h], dtype)
            for j in range(g):
                hq = h * g + j
                s = (K @ qf[b, hq]) * softmax_scale
                p = np.exp(s - s.max())
                p = p / p.sum()
                out[b, hq] = p @ V
    return out


def tolerance_terms(q, k_codes, v_codes, k_codebook, v_codebook, dtype, *, k_scale=None,
                    kv_len=None, window=0, softmax_scale=None):
    """Per (b, hq): the largest score magnitude bound A = scale * max_t
    sum_i |q_i k_ti| and the number of attended tokens T; per (b, hq, d):
    M = sum_t p_t |v_td|.  The GPU error bound is built from these."""
    B, Hq, D = q.shape
    Hkv, S = k_codes.shape[1], k_codes.shape[2]
    g = Hq // Hkv
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(D)
    lens = np.full(B, S) if kv_len is None else np.asarray(kv_len)
    qf = widen(q, dtype)
    A = np.zeros((B, Hq))
    T = np.zeros((B, Hq), dtype=np.int64)
    M = np.zeros((B, Hq, D))
    for b in range(B):
        t0, t1 = _attended(int(lens[b]), window)
        if t1 <= t0:
            continue
        for h in range(Hkv):
            K = dequantize(k_codes[b, h, t0:t1], k_codebook[h], dtype)
            if k_scale is not None:
                K = K / np.asarray(k_scale[h], dtype=np.float64)[None, :]
            V = dequantize(v_codes[b, h, t0:t1], v_codebook[h], dtype)
            for j in range(g):
                hq = h * g + j
                s = (K @ qf[b, hq]) * softmax_scale
                p = np.exp(s - s.max())
                p = p / p.sum()
                A[b, hq] = abs(softmax_scale) * (np.abs(K) @ np.abs(qf[b, hq])).max()
                T[b, hq] = t1 - t0
                M[b, hq] = p @ np.abs(V)
    return A, T, M
