"""Pins of the K-means oracle (oracle/kmeans.py), CPU only.

Against what:
  * the exact fp16 rounding against numpy's float64 -> float16 conversion
    (a library routine, one rounding of an exactly representable value),
    including subnormals, exact ties and overflow;
  * hand-built clusters whose means are exactly representable: one update
    gives numpy's float64 means;
  * properties of a Lloyd update that hold whatever the data: every updated
    centroid is the fp16 value nearest the exact member mean (checked against
    its fp16 neighbours), a centroid of an empty cluster keeps its value, the
    objective does not grow past the rounding slack, a codebook of exact
    cell means is a fixed point;
  * per-slot training equals training every slot on its own;
  * planted mistakes in copies of the oracle fail these pins.
"""
import os
import types
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W
from oracle import kmeans as K


def test_f16_round_matches_numpy_on_representable_values():
    r = np.random.default_rng(1)
    vals = np.concatenate([
        r.standard_normal(3000) * np.exp(r.uniform(-20, 12, 3000)),
        np.ldexp(r.integers(1, 2 ** 20, 500).astype(np.float64), -35),     # subnormal range
        np.array([0.0, 65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -25, 3 * 2.0 ** -26,
                  1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, -(1.0 + 2.0 ** -11), 2.0 ** -24]),
    ])
    for v in vals:
        with np.errstate(over="ignore"):
            want = int(np.array(v).astype(np.float16).view(np.uint16))
        got = K.f16_round(Fraction(float(v)))
        assert got == want, (v, hex(got), hex(want))


def test_f16_round_of_rationals_is_the_nearest_fp16():
    r = np.random.default_rng(2)
    for _ in range(2000):
        den = int(r.integers(1, 10 ** 6))
        q = Fraction(int(r.integers(-60000 * den, 60000 * den)), den)      # finite in fp16
        if _ % 3 == 0:
            q /= 2 ** int(r.integers(0, 30))                               # down to subnormals
        b = K.f16_round(q)
        v = Fraction(float(np.array(b, np.uint16).view(np.float16)))
        for nb in (b - 1, b + 1):
            if 0 <= nb <= 0xFFFF and (nb & 0x7C00) != 0x7C00:
                w = Fraction(float(np.array(nb, np.uint16).view(np.float16)))
                assert abs(v - q) <= abs(w - q)


def _cluster_case():
    """Three exact clusters (integer points); codebook rows start inside them."""
    pts = np.array([[0, 0, 0, 0], [2, 0, 0, 2], [0, 2, 2, 0], [2, 2, 2, 2],      # mean 1,1,1,1
                    [10, 10, 10, 10], [12, 12, 12, 12],                          # mean 11
                    [-8, 4, -8, 4], [-6, 6, -6, 6], [-7, 5, -7, 5]], np.float64)  # mean -7,5,-7,5
    init = np.array([[0.5, 0.5, 0.5, 0.5], [10.5, 10, 10, 10], [-7, 4, -7, 4], [100, 100, 100, 100]])
    return W.to_f16_bits(pts).reshape(-1, 4), W.to_f16_bits(init).reshape(-1)


def test_one_update_gives_exact_means_and_keeps_empty_clusters():
    x, cb = _cluster_case()
    new, idx, counts = K.kmeans(x, cb, 4, 4, 1)
    got = new.view(np.float16).astype(np.float64).reshape(4, 4)
    np.testing.assert_array_equal(got[0], [1, 1, 1, 1])
    np.testing.assert_array_equal(got[1], [11, 11, 11, 11])
    np.testing.assert_array_equal(got[2], [-7, 5, -7, 5])
    np.testing.assert_array_equal(new.reshape(4, 4)[3], cb.reshape(4, 4)[3])   # empty keeps
    assert counts.tolist() == [[4, 2, 3, 0]]
    again, _, _ = K.kmeans(x, new, 4, 4, 1)                                     # fixed point
    np.testing.assert_array_equal(again, new)


def test_updates_are_nearest_fp16_of_member_means_and_objective_does_not_grow():
    wl = W.random_case(5, 3000, 8, 40)
    cb = wl.codebook.copy()
    for _ in range(3):
        idx = oracle.encode(wl.x, cb, 8, 40, W.F16)
        before = K.inertia(wl.x, cb, idx, 8, 40)
        new, counts = K.update(wl.x, idx, cb, 8, 40)
        after = K.inertia(wl.x, new, idx, 8, 40)
        slack = 0.0
        for c in range(40):
            m = idx == c
            if not m.any():
                assert np.array_equal(new[c * 8:(c + 1) * 8], cb[c * 8:(c + 1) * 8])
                continue
            mean = [Fraction(int(t), int(m.sum()) * 2 ** 24) for t in K.f16_units(wl.x[m]).sum(0)]
            for i in range(8):
                b = int(new[c * 8 + i])
                v = Fraction(float(np.array(b, np.uint16).view(np.float16)))
                for nb in (b - 1, b + 1):
                    if (nb & 0x7C00) != 0x7C00 and 0 <= nb <= 0xFFFF:
                        w = Fraction(float(np.array(nb, np.uint16).view(np.float16)))
                        assert abs(v - mean[i]) <= abs(w - mean[i])
                slack += int(m.sum()) * float(v - mean[i]) ** 2
        # the mean minimizes the members' squared distance; rounding adds
        # exactly count * (rounding offset)^2 per coordinate
        assert after <= before + slack * (1 + 1e-9) + 1e-12
        cb = new


def test_slots_train_independently():
    wl = W.random_case(6, 4000, 4, 16, n_codebooks=3, group_len=500, use_map=True)
    new, idx, _ = K.kmeans(wl.x, wl.codebook, 4, 16, 2, codebook_stride=wl.codebook_stride,
                           n_codebooks=3, group_len=500, group_map=wl.group_map)
    g = np.arange(wl.n) // 500
    for s in range(3):
        rows = wl.group_map[g] == s
        sub = wl.codebook[s * wl.codebook_stride: s * wl.codebook_stride + 64]
        alone, aidx, _ = K.kmeans(wl.x[rows], sub, 4, 16, 2)
        np.testing.assert_array_equal(new[s * wl.codebook_stride: s * wl.codebook_stride + 64], alone)
        np.testing.assert_array_equal(idx[rows], aidx)


PINS = [
    lambda: test_f16_round_matches_numpy_on_representable_values(),
    lambda: test_one_update_gives_exact_means_and_keeps_empty_clusters(),
    lambda: test_slots_train_independently(),
]

MUTANTS = {
    "count_plus_one": ("q = Fraction(int(total[i]), cnt * 2 ** 24)",
                       "q = Fraction(int(total[i]), (cnt + 1) * 2 ** 24)"),
    "empty_to_zero": ("if cnt == 0:\n                continue",
                      "if cnt == 0:\n                cb[s * stride + c * sub_dim: s * stride + (c + 1) * sub_dim] = 0\n                continue"),
    "ties_away": ("if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m_floor % 2 == 1):",
                  "if rem >= Fraction(1, 2):"),
    "subnormal_floor": ("e = max(e, -14)", "e = max(e, -15)"),
    "slot_by_group_modulo": ("g = np.arange(n) // glen\n    slots = (np.asarray(group_map)[g] if group_map is not None else g).astype(np.int64)\n    units",
                             "g = np.arange(n) % glen\n    slots = (np.asarray(group_map)[g % len(group_map)] if group_map is not None else g).astype(np.int64)\n    units"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_kmeans_mistake(name):
    src = open(K.__file__).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mod = types.ModuleType("mutant_kmeans")
    exec(compile(src.replace(old, new, 1), os.path.basename(K.__file__), "exec"), mod.__dict__)
    real = K.__dict__.copy()
    caught = False
    try:
        K.__dict__.update({k: v for k, v in mod.__dict__.items() if callable(v)})
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError, IndexError):
                caught = True
                break
    finally:
        K.__dict__.update(real)
    assert caught, f"no pin caught {name!r}"
