"""Pins of ``oracle.attention.tolerance_terms`` and of the acceptance bound
built from it (tests/attention_bound.py), CPU only.

The decode-attention parity tests accept the GPU output when every element
is within (2 Delta + (3T + 32) u) * M_d of the float64 oracle, with
Delta = 1.5 (sd_k + n_sub_k + 4) u A.  A (the largest score magnitude bound),
T (attended tokens) and M_d (sum_t p_t |v_td|) come from tolerance_terms; a
mistake there would silently widen the bound.  So:

  * hand-worked cases fix A, T and M exactly: one attended token (T = 1,
    M_d = |v_d|, A = scale * sum_i |q_i k_i| with smoothing undone); two
    distinct keys in a window over a grouped-query group, whose softmax
    weights are closed forms in e; equal keys (M_d = mean_t |v_td|);
  * planted mistakes in copies of the oracle (M without the weights or with
    |.| outside the sum, T off by one, A without the scale, with signed
    products, averaged instead of maximal, without undoing the smoothing, a
    modulo head mapping) must fail these pins;
  * the bound bites: on the Falcon3-7B decode workload, a 10% error in the
    weight of any 256-token chunk, and a dropped token or a 10% error in one
    token's weight at every chunk boundary when those tokens carry the
    attention, exceed it (a chunk carrying >= 5% of the mass; a rescale
    error of 10% moves the output by 0.1 w (v_chunk - out), past the bound
    once w > ~10 x its relative size).  (A 10% error in the weight of a token that
    carries ~1/T of the mass changes the output by ~1e-5 of M_d, inside what
    fp32 rounding of any summation order may do, so no sound bound can see
    it; the GPU tests make the boundary tokens heavy instead.)
"""
import math
import os
import types

import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from tests import attention_bound as AB


def f16(vals):
    return np.asarray(vals, dtype=np.float64).astype(np.float16).view(np.uint16)


def terms(wl, mod=A):
    return mod.tolerance_terms(wl.q, wl.k_codes, wl.v_codes, wl.k_codebook, wl.v_codebook,
                               wl.dtype, **wl.kwargs())


def one_token_case():
    """D = 8, two sub-spaces of 4, one sequence with one token, scale 0.5."""
    kcb = f16([[[1, -2, 0.5, 0], [0.25, 1, -1, 2], [0, 0, 0, 0], [7, 7, 7, 7]]])
    vcb = f16([[[9, 9, 9, 9], [0, 0, 0, 0], [3, -0.5, 1, -2], [-1.5, 2, 0, 0.125]]])
    k_codes = np.array([[[[0, 1], [3, 3]]]], np.uint8)          # [B=1, Hkv=1, S=2, 2]
    v_codes = np.array([[[[3, 2], [0, 0]]]], np.uint8)
    f = np.array([[1, 2, 1, 0.5, 1, 1, 4, 1]], np.float32)
    q = f16([[[2, 1, -4, 3, 8, -1, 2, 0.5]]])
    wl = W.AttnWorkload("one token", q, k_codes, v_codes, kcb, vcb, f, np.array([1], np.int32),
                        W.F16)
    wl.softmax_scale = 0.5
    return wl


def test_one_attended_token_by_hand():
    Aq, T, M = terms(one_token_case())
    # k / f = [1, -1, 0.5, 0, 0.25, 1, -0.25, 2]; sum |q||k/f| = 9.5; times 0.5
    assert Aq[0, 0] == 4.75
    assert T[0, 0] == 1
    assert np.array_equal(M[0, 0], [1.5, 2, 0, 0.125, 3, 0.5, 1, 2])


def window_gqa_case():
    """Two kv heads, two query heads each; D = 4 (one sub-space), default
    scale 1/sqrt(4) = 0.5; six tokens, window 4 -> tokens 2..5 attended.
    Key row 0 scores s0 for the query, row 1 (all zero) scores 0."""
    kcb = f16([[[1, -0.5, 0, 0], [0, 0, 0, 0]],
               [[0, 0, 2, 0], [0, 0, 0, 0]]])
    vcb = f16([[[1, -1, 2, 0], [-3, 0.5, 0, 1]],
               [[0.5, 0.5, -4, 8], [2, 0, 0, -1]]])
    k_codes = np.zeros((1, 2, 6, 1), np.uint8)
    v_codes = np.zeros((1, 2, 6, 1), np.uint8)
    k_codes[0, 0, :, 0] = [1, 1, 0, 1, 1, 0]
    v_codes[0, 0, :, 0] = [1, 1, 0, 0, 0, 1]
    k_codes[0, 1, :, 0] = [0, 0, 1, 1, 1, 0]
    v_codes[0, 1, :, 0] = [0, 0, 0, 1, 1, 1]
    q = f16([[[1, 1, 0, 0], [-2, 0, 0, 5], [0, 3, 1, 0], [0, 0, -3, 0]]])
    wl = W.AttnWorkload("window gqa", q, k_codes, v_codes, kcb, vcb, None,
                        np.array([6], np.int32), W.F16)
    wl.window = 4
    return wl


def test_window_over_a_grouped_query_group_by_hand():
    Aq, T, M = terms(window_gqa_case())
    assert np.array_equal(T, [[4, 4, 4, 4]])
    av = lambda *r: np.abs(np.array(r, dtype=np.float64))
    v00, v01 = av(1, -1, 2, 0), av(-3, 0.5, 0, 1)
    v10, v11 = av(0.5, 0.5, -4, 8), av(2, 0, 0, -1)
    # head 0 (kv 0): q.k0 = 1 - 0.5 = 0.5, times 0.5 -> s0 = 0.25; sum |q||k0| = 1.5
    # attended (key, value) rows: t2 (0, 0), t3 (1, 0), t4 (1, 0), t5 (0, 1)
    e = math.exp(0.25)
    want0 = (e * v00 + v00 + v00 + e * v01) / (2 * e + 2)
    assert Aq[0, 0] == 0.75
    np.testing.assert_allclose(M[0, 0], want0, rtol=1e-14)
    # head 1 (kv 0): q.k0 = -2 -> s0 = -1; sum |q||k0| = 2
    e = math.exp(-1.0)
    want1 = (e * v00 + v00 + v00 + e * v01) / (2 * e + 2)
    assert Aq[0, 1] == 1.0
    np.testing.assert_allclose(M[0, 1], want1, rtol=1e-14)
    # heads 2, 3 (kv 1): key row 0 = [0, 0, 2, 0]; attended t2 (1, 0),
    # t3 (1, 1), t4 (1, 1), t5 (0, 1); row 1 scores 0
    for hq, qk in ((2, 2.0), (3, -6.0)):
        e = math.exp(0.5 * qk)
        want = (v10 + v11 + v11 + e * v11) / (3 + e)
        assert Aq[0, hq] == 0.5 * abs(qk)
        np.testing.assert_allclose(M[0, hq], want, rtol=1e-14)


def test_equal_keys_give_the_mean_of_the_value_magnitudes():
    wl = W.attention_case(31, 3, 4, 2, 32, 60, 4, 8, 64, lens="mixed")
    wl.k_codes[:] = wl.k_codes[:, :, :1, :]
    Aq, T, M = terms(wl)
    q = wl.q.view(np.float16).astype(np.float64)
    kcb = wl.k_codebook.view(np.float16).astype(np.float64)
    vcb = wl.v_codebook.view(np.float16).astype(np.float64)
    for b in range(3):
        L = int(wl.kv_len[b])
        for hq in range(4):
            h = hq // 2
            k = np.concatenate([kcb[h][c] for c in wl.k_codes[b, h, 0]]) / wl.k_scale[h]
            V = np.stack([np.concatenate([vcb[h][c] for c in wl.v_codes[b, h, t]])
                          for t in range(L)])
            assert T[b, hq] == L
            np.testing.assert_allclose(Aq[b, hq], np.sum(np.abs(q[b, hq] * k)) / math.sqrt(32),
                                       rtol=1e-14)
            np.testing.assert_allclose(M[b, hq], np.abs(V).mean(axis=0), rtol=1e-13)


def test_empty_sequence_has_no_terms():
    wl = W.attention_case(32, 3, 2, 1, 16, 10, 4, 4, 16, lens="ragged")
    Aq, T, M = terms(wl)
    assert T[0, 0] == 0 and Aq[0, 0] == 0 and np.all(M[0] == 0)
    assert T[1, 0] == 1


def _pin(mod, check):
    """Run one of the pins above with a (mutated) module's tolerance_terms."""
    saved = A.tolerance_terms
    try:
        A.tolerance_terms = mod.tolerance_terms
        check()
    finally:
        A.tolerance_terms = saved


PINS = [
    lambda m: _pin(m, test_one_attended_token_by_hand),
    lambda m: _pin(m, test_window_over_a_grouped_query_group_by_hand),
    lambda m: _pin(m, test_equal_keys_give_the_mean_of_the_value_magnitudes),
]


# mutation sites inside tolerance_terms only
MUTANTS = {
    "M_unweighted": ("M[b, hq] = p @ np.abs(V)", "M[b, hq] = np.abs(V).sum(axis=0)"),
    "M_abs_outside": ("M[b, hq] = p @ np.abs(V)", "M[b, hq] = np.abs(p @ V)"),
    "T_off_by_one": ("T[b, hq] = t1 - t0", "T[b, hq] = t1 - t0 + 1"),
    "A_no_scale": ("A[b, hq] = abs(softmax_scale) * ", "A[b, hq] = "),
    "A_signed": ("(np.abs(K) @ np.abs(qf[b, hq])).max()", "np.abs(K @ qf[b, hq]).max()"),
    "A_mean": ("(np.abs(K) @ np.abs(qf[b, hq])).max()", "(np.abs(K) @ np.abs(qf[b, hq])).mean()"),
    "A_smoothing_kept": ("(np.abs(K) @ np.abs(qf[b, hq])).max()",
                         "(np.abs(K * (1.0 if k_scale is None else np.asarray(k_scale[h], "
                         "dtype=np.float64))) @ np.abs(qf[b, hq])).max()"),
    "gqa_modulo": ("A[b, hq] = abs", "hq = j * Hkv + h\n                A[b, hq] = abs"),
}


def test_mutation_sites_are_in_tolerance_terms_only():
    src = open(A.__file__).read()
    body = src[src.index("def tolerance_terms"):]
    for name, (old, _) in MUTANTS.items():
        assert body.count(old) == 1 and src.count(old) == 1, name


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_tolerance_mistake(name):
    src = open(A.__file__).read()
    old, new = MUTANTS[name]
    mod = types.ModuleType("mutant_attention_terms")
    exec(compile(src.replace(old, new, 1), os.path.basename(A.__file__), "exec"), mod.__dict__)
    caught = False
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            caught = True
            break
    assert caught, f"no pin caught {name!r}"


# ---------------------------------------------------------------- the bound bites

def _falcon_sample(nb=4):
    wl = W.falcon_decode_attention()
    return W.AttnWorkload("falcon sample", wl.q[:nb].copy(), wl.k_codes[:nb].copy(),
                          wl.v_codes[:nb].copy(), wl.k_codebook, wl.v_codebook, wl.k_scale,
                          wl.kv_len[:nb].copy(), wl.dtype)


def _weights_and_values(wl, b, hq):
    """p_t and V for one (sequence, query head), from the plain definition."""
    B, Hq, Hkv, D, S = wl.shape
    h = hq // (Hq // Hkv)
    L = int(wl.kv_len[b])
    q = A.widen(wl.q[b, hq], wl.dtype)
    K = A.dequantize(wl.k_codes[b, h, :L], wl.k_codebook[h], wl.dtype) / wl.k_scale[h]
    V = A.dequantize(wl.v_codes[b, h, :L], wl.v_codebook[h], wl.dtype)
    s = (K @ q) / math.sqrt(D)
    p = np.exp(s - s.max())
    return p / p.sum(), V


def _exceeds(wl, b, hq, delta_out, Aq, T, M):
    D = wl.shape[3]
    n_sub_k = wl.k_codes.shape[3]
    rel = AB.relative_bound(Aq[b, hq], T[b, hq], D // n_sub_k, n_sub_k)
    return float(np.max(np.abs(delta_out) / (rel * M[b, hq] + 1e-30)))


def test_ten_percent_error_in_any_chunk_weight_exceeds_the_bound():
    wl = _falcon_sample()
    Aq, T, M = terms(wl)
    worst = np.inf
    for b in range(wl.shape[0]):
        L = int(wl.kv_len[b])
        for hq in range(wl.shape[1]):
            p, V = _weights_and_values(wl, b, hq)
            for c0 in range(0, L, 256):
                # the chunk's weights scaled by 1.1, then renormalized
                w = p.copy()
                w[c0:c0 + 256] *= 1.1
                w /= w.sum()
                r = _exceeds(wl, b, hq, (w - p) @ V, Aq, T, M)
                if p[c0:c0 + 256].sum() >= 0.05:
                    worst = min(worst, r)
    print(f"[bound] smallest excess of a 10% error in a chunk carrying >= 5% of the mass: "
          f"{worst:.1f}x")
    assert worst > 1.0


def test_boundary_token_errors_exceed_the_bound_when_they_carry_the_attention():
    wl = _falcon_sample()
    positions = AB.make_boundary_tokens_heavy(wl)
    Aq, T, M = terms(wl)
    Hq, Hkv = wl.shape[1], wl.shape[2]
    worst_drop = worst_ten = np.inf
    for b in range(wl.shape[0]):
        for hq in range(0, Hq, Hq // Hkv):           # the heads the keys were chosen for
            p, V = _weights_and_values(wl, b, hq)
            assert p[positions[b]].sum() > 0.9
            for t in positions[b]:
                w = p.copy()
                w[t] = 0.0
                w /= w.sum()
                worst_drop = min(worst_drop, _exceeds(wl, b, hq, (w - p) @ V, Aq, T, M))
                w = p.copy()
                w[t] *= 1.1
                w /= w.sum()
                worst_ten = min(worst_ten, _exceeds(wl, b, hq, (w - p) @ V, Aq, T, M))
    print(f"[bound] smallest excess at chunk boundaries: dropped token {worst_drop:.1f}x, "
          f"10% weight error {worst_ten:.1f}x")
    assert worst_drop > 1.0 and worst_ten > 1.0


def test_light_token_errors_are_below_fp32_rounding_of_the_sum():
    """Why the unmodified workload cannot pin a single light token: a 10%
    error in a weight of ~1/T is smaller than (T - 1) u, the worst-case
    relative rounding error of an fp32 sum of T terms in any order."""
    wl = _falcon_sample(1)
    p, _ = _weights_and_values(wl, 0, 0)
    T = p.size
    light = np.median(p)
    assert 0.1 * light < (T - 1) * AB.U
