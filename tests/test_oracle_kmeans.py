"""Pins of the K-means oracle (oracle/kmeans.py), CPU only.

Against what:
  * the exact fp16 rounding against numpy's float64 -> float16 conversion
    (a library routine, one rounding of an exactly representable value),
    including subnormals, exact ties and overflow; the exact bf16 rounding
    against torch's float32 -> bfloat16 conversion (one rounding of a float32
    value), and both against brute-force neighbour checks of random rationals;
  * the exact bf16 member sums against sums of Python fractions of the
    values (every exponent, subnormals, signs, non-finite elements);
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


# ---------------------------------------------------------------- bf16

def _bf16_value(b: int) -> Fraction:
    """Exact value of finite bf16 bits (via float32, which holds it exactly)."""
    return Fraction(float(np.array([b << 16], np.uint32).view(np.float32)[0]))


def test_bf16_round_matches_torch_on_float32_values():
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(11)
    f32 = np.concatenate([
        (r.standard_normal(4000) * np.exp(r.uniform(-80, 80, 4000))).astype(np.float32),
        r.integers(1, 2 ** 23, 800).astype(np.uint32).view(np.float32),          # fp32 subnormals
        np.array([0x3F808000, 0x3F818000, 0x00008000, 0x00018000, 0x7F7FFFFF, 0x7F7F8000,
                  0x7F7F7FFF, 0x80008000, 0x00000001], np.uint32).view(np.float32),
    ])
    want = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for v, w in zip(f32, want):
        got = K.bf16_round(Fraction(float(v)))
        assert got == int(w), (float(v), hex(got), hex(int(w)))


def test_bf16_round_of_rationals_is_the_nearest_bf16():
    r = np.random.default_rng(12)
    for k in range(2000):
        den = int(r.integers(1, 10 ** 6))
        q = Fraction(int(r.integers(-10 ** 7 * den, 10 ** 7 * den)), den)
        q *= Fraction(2) ** int(r.integers(-150, 110))
        b = K.bf16_round(q)
        if (b & 0x7F80) == 0x7F80:
            assert (b & 0x7FFF) == 0x7F80                 # infinity, never a NaN pattern
            assert abs(q) >= _bf16_value(0x7F7F)
            continue
        v = _bf16_value(b)
        for nb in (b - 1, b + 1):
            if 0 <= nb <= 0xFFFF and (nb & 0x7F80) != 0x7F80:
                w = _bf16_value(nb)
                assert abs(v - q) <= abs(w - q)
                if abs(v - q) == abs(w - q):
                    assert (b & 1) == 0                                     # ties to even


def test_bf16_exact_sums_equal_fraction_sums():
    r = np.random.default_rng(13)
    for k in range(300):
        n = int(r.integers(1, 40))
        bits = r.integers(0, 0x10000, n).astype(np.uint16)
        if k % 3 == 0:                                  # a narrow exponent band
            bits = ((bits & 0x807F) | (int(r.integers(1, 254)) << 7)).astype(np.uint16)
        if k % 5 == 0:                                  # subnormals
            bits = (bits & 0x807F).astype(np.uint16)
        want = sum((_bf16_value(int(b)) for b in bits if (b & 0x7F80) != 0x7F80), Fraction(0))
        got = K.exact_sum(bits, K.BF16)
        assert Fraction(got, 2 ** 133) == want


def test_non_finite_components_add_zero_but_their_rows_count():
    for dt, inf, nan, one in ((K.F16, 0x7C00, 0x7E00, 0x3C00), (K.BF16, 0x7F80, 0x7FC0, 0x3F80)):
        x = np.array([[one, one, one, one], [inf, nan, one, 0x8000 | inf]], np.uint16)
        cb = np.zeros(4, np.uint16)
        new, counts = K.update(x, np.array([0, 0], np.uint32), cb, 4, 1, dt)
        assert counts.tolist() == [[2]]
        half = 0x3800 if dt == K.F16 else 0x3F00
        assert new.tolist() == [half, half, one, half]        # (1 + 0) / 2 and (1 + 1) / 2


def _cluster_case_bf16():
    """Exact clusters over a wide exponent range (bf16 keeps 8 significant bits)."""
    pts = np.array([[2.0 ** 100, 2.0 ** -120, -3.0, 0.0], [3 * 2.0 ** 100, 3 * 2.0 ** -120, -5.0, 0.0],
                    [1.0, 1.0, 1.0, 1.0], [1.0, 1.0, 1.0, 1.0], [1.0, 1.0, 1.0, 4.0],
                    [1.0, 1.0, 1.0, 2.0],
                    [2.0 ** -130, -(2.0 ** -131), 2.0 ** 127, -(2.0 ** 127)],
                    [3 * 2.0 ** -130, -(3 * 2.0 ** -131), 2.0 ** 126, -(2.0 ** 126)]], np.float64)
    init = np.array([[2.0 ** 101, 0, -4, 0], [1, 1, 1, 2], [2.0 ** -129, 0, 2.0 ** 126, -(2.0 ** 126)],
                     [-100, -100, -100, -100]])
    return W.to_bf16_bits(pts).reshape(-1, 4), W.to_bf16_bits(init).reshape(-1)


def test_bf16_one_update_gives_exact_means():
    x, cb = _cluster_case_bf16()
    idx = np.array([0, 0, 1, 1, 1, 1, 2, 2], np.uint32)
    new, counts = K.update(x, idx, cb, 4, 4, K.BF16)
    got = K.widen(new, K.BF16).reshape(4, 4)
    np.testing.assert_array_equal(got[0], [2.0 ** 101, 2.0 ** -119, -4.0, 0.0])
    np.testing.assert_array_equal(got[1], [1.0, 1.0, 1.0, 2.0])
    # (2^-130 + 3 2^-130) / 2 = 2^-129; (2^127 + 2^126) / 2 = 1.5 2^126
    np.testing.assert_array_equal(got[2], [2.0 ** -129, -(2.0 ** -130), 1.5 * 2.0 ** 126,
                                           -1.5 * 2.0 ** 126])
    np.testing.assert_array_equal(new.reshape(4, 4)[3], cb.reshape(4, 4)[3])
    assert counts.tolist() == [[2, 4, 2, 0]]


def test_bf16_updates_are_nearest_bf16_of_member_means():
    wl = W.random_case(15, 2000, 8, 30, W.BF16)
    cb = wl.codebook.copy()
    for _ in range(2):
        idx = oracle.encode(wl.x, cb, 8, 30, W.BF16)
        before = K.inertia(wl.x, cb, idx, 8, 30, dtype=K.BF16)
        new, counts = K.update(wl.x, idx, cb, 8, 30, K.BF16)
        after = K.inertia(wl.x, new, idx, 8, 30, dtype=K.BF16)
        slack = 0.0
        xv = K.widen(wl.x, K.BF16).reshape(-1, 8)
        for c in range(30):
            m = idx == c
            if not m.any():
                assert np.array_equal(new[c * 8:(c + 1) * 8], cb[c * 8:(c + 1) * 8])
                continue
            for i in range(8):
                mean = sum((Fraction(float(v)) for v in xv[m, i]), Fraction(0)) / int(m.sum())
                b = int(new[c * 8 + i])
                v = _bf16_value(b)
                for nb in (b - 1, b + 1):
                    if (nb & 0x7F80) != 0x7F80 and 0 <= nb <= 0xFFFF:
                        assert abs(v - mean) <= abs(_bf16_value(nb) - mean)
                slack += int(m.sum()) * float(v - mean) ** 2
        assert after <= before + slack * (1 + 1e-9) + 1e-12
        cb = new


PINS = [
    lambda: test_f16_round_matches_numpy_on_representable_values(),
    lambda: test_one_update_gives_exact_means_and_keeps_empty_clusters(),
    lambda: test_slots_train_independently(),
    lambda: test_bf16_round_matches_torch_on_float32_values(),
    lambda: test_bf16_round_of_rationals_is_the_nearest_bf16(),
    lambda: test_bf16_exact_sums_equal_fraction_sums(),
    lambda: test_bf16_one_update_gives_exact_means(),
    lambda: test_non_finite_components_add_zero_but_their_rows_count(),
]

_F16_ROUND_TIES = ("ulp = Fraction(2) ** (e - 10)\n    m_floor = int(a / ulp)            # a / ulp >= 0\n"
                   "    rem = a / ulp - m_floor\n"
                   "    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m_floor % 2 == 1):")
_BF16_ROUND_TIES = ("ulp = Fraction(2) ** (e - 7)\n    m_floor = int(a / ulp)\n    rem = a / ulp - m_floor\n"
                    "    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m_floor % 2 == 1):")
MUTANTS = {
    "count_plus_one": ("q = Fraction(total, cnt * unit)", "q = Fraction(total, (cnt + 1) * unit)"),
    "empty_to_zero": ("for s in range(n_codebooks):\n        rows = ",
                      "for s in range(n_codebooks):\n        cb[s * stride: s * stride + n_centroids * sub_dim] = 0\n        rows = "),
    "ties_away": (_F16_ROUND_TIES, _F16_ROUND_TIES.split("    if rem")[0] + "    if rem >= Fraction(1, 2):"),
    "subnormal_floor": ("e = max(e, -14)", "e = max(e, -15)"),
    "slot_by_group_modulo": ("g = np.arange(n) // glen\n    slots = (np.asarray(group_map)[g] if group_map is not None else g).astype(np.int64)\n    idx",
                             "g = np.arange(n) % glen\n    slots = (np.asarray(group_map)[g % len(group_map)] if group_map is not None else g).astype(np.int64)\n    idx"),
    "bf16_ties_away": (_BF16_ROUND_TIES, _BF16_ROUND_TIES.split("    if rem")[0] + "    if rem >= Fraction(1, 2):"),
    "bf16_subnormal_floor": ("e = max(e, -126)", "e = max(e, -127)"),
    "bf16_overflow_late": ("if e > 127:", "if e > 128:"),
    "bf16_shift_off_by_one": ("p = np.where(E == 0, 0, E - 1)", "p = np.where(E == 0, 0, E)"),
    "bf16_subnormal_implicit_bit": ("m = np.where(E == 0, F, 128 + F)", "m = 128 + F"),
    "bf16_sign_dropped": ("m = np.where(bits & 0x8000, -m, m)", "m = m"),
    "bf16_wrong_unit": ("UNIT_LOG2 = {F16: 24, BF16: 133}", "UNIT_LOG2 = {F16: 24, BF16: 134}"),
    "non_finite_counted": ("v = np.where(np.isfinite(v), v, 0.0) * float(2 ** 24)",
                           "v = np.where(np.isfinite(v), v, 65504.0) * float(2 ** 24)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_kmeans_mistake(name):
    src = open(K.__file__).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found or not unique"
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
