"""Pins for the CPU oracle, against things other than itself.

The oracle (oracle/vq_oracle.c) computes, per sub-vector, the index of the
nearest codebook centroid by summed squared difference in fp32 (one rounded
subtraction and one fused multiply-add per component, components in order),
strict-< running argmin so ties keep the lowest index (VeloxQuant-MLX blog,
"I Wrote a Metal Kernel to Stop My Mac From OOMing", sections "What quantize_vq
Was Doing Wrong" and "The Kernel: 18 Lines of MSL").

What pins it here:
  * exact integer brute force: fp16/bf16 values are integer multiples of a
    power of two, so every distance is an exact int64; the oracle must equal
    the exact argmin (lowest index on exact ties) everywhere on a grid where
    fp32 arithmetic is exact, and everywhere else except where the exact gap
    is inside the fp32 rounding bound;
  * hand-built inputs with known answers;
  * sub_dim = 1 with a sorted codebook, which reduces to boundary-sum scalar
    quantization (index = number of midpoints the value exceeds);
  * the element widening against numpy's and torch's own conversions.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W

U = 2.0 ** -24


# --------------------------------------------------------------------------
# helpers: exact arithmetic, independent of the oracle
# --------------------------------------------------------------------------

def f16_exact_int(bits):
    """fp16 value * 2^24 as int64 (exact for every finite fp16)."""
    v = np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)
    return np.rint(v * 2.0 ** 24).astype(np.int64)


def bf16_exact_int(bits, shift):
    """bf16 value * 2^shift as int64 (exact when every ulp >= 2^-shift)."""
    v = (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    k = v * 2.0 ** shift
    assert np.all(k == np.rint(k)), "value not on the integer grid"
    return k.astype(np.int64)


def exact_argmin(kx, kc):
    """Exact squared distances (int64) and the lowest-index argmin."""
    diff = kx[:, None, :] - kc[None, :, :]
    d = np.sum(diff * diff, axis=-1)
    return d, np.argmin(d, axis=1)   # np.argmin returns the first minimum


def gamma(sd):
    # |fp32 distance - exact| <= ((1+u)^(sd+2) - 1) * exact  (all terms >= 0)
    return (1.0 + U) ** (sd + 2) - 1.0


def random_f16_bits(r, shape, max_exp_field):
    """Random finite fp16 bit patterns with exponent field <= max_exp_field
    (magnitude < 2^(max_exp_field-14)), subnormals and zeros included."""
    sign = r.integers(0, 2, size=shape).astype(np.uint16) << 15
    expo = r.integers(0, max_exp_field + 1, size=shape).astype(np.uint16) << 10
    frac = r.integers(0, 1024, size=shape).astype(np.uint16)
    return sign | expo | frac


def random_bf16_bits(r, shape, lo_exp, hi_exp):
    sign = r.integers(0, 2, size=shape).astype(np.uint16) << 15
    expo = r.integers(127 + lo_exp, 127 + hi_exp + 1, size=shape).astype(np.uint16) << 7
    frac = r.integers(0, 128, size=shape).astype(np.uint16)
    bits = sign | expo | frac
    zero = r.random(shape) < 0.05
    bits[zero] = 0
    return bits


# --------------------------------------------------------------------------
# element widening
# --------------------------------------------------------------------------

def test_f16_widening_matches_numpy_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.to_f32(int(b), oracle.F16) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_widening_matches_torch_every_pattern():
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint32).astype(np.int32)
    t = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).float().numpy()
    got = np.array([oracle.to_f32(int(b), oracle.BF16) for b in bits], dtype=np.float32)
    nan = np.isnan(t)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), t[~nan].view(np.uint32))


# --------------------------------------------------------------------------
# exact brute force
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_exact_grid_no_exemptions(dtype):
    """Values k/64, |k| <= 255: every fp32 step of the distance is exact, so
    the oracle must reproduce the exact argmin and its lowest-index tie rule
    on every row, with no exemption.  The coarse grid makes exact ties common."""
    r = np.random.default_rng(11 + dtype)
    n_ties = 0
    for case in range(600):
        sd = int(r.choice([1, 2, 3, 4, 5, 8]))
        n = int(r.integers(1, 48))
        n_c = int(r.integers(1, 48))
        kx = r.integers(-255, 256, size=(n, sd))
        kc = r.integers(-255, 256, size=(n_c, sd))
        if r.random() < 0.5:                      # a very coarse grid: many ties
            kx = 64 * r.integers(-3, 4, size=(n, sd))
            kc = 64 * r.integers(-3, 4, size=(n_c, sd))
        to_bits = W.to_f16_bits if dtype == oracle.F16 else W.to_bf16_bits
        xb = to_bits(kx / 64.0)
        cb = to_bits(kc / 64.0)
        d, want = exact_argmin(kx.astype(np.int64), kc.astype(np.int64))
        got = oracle.encode(xb, cb, sd, n_c, dtype)
        assert np.array_equal(got, want.astype(np.uint32)), f"case {case}"
        srt = np.sort(d, axis=1)
        if n_c > 1:
            n_ties += int(np.sum(srt[:, 0] == srt[:, 1]))
    assert n_ties > 1000, "the grid should exercise the tie rule heavily"


def _check_with_exemptions(kx, kc, got, sd):
    d, want = exact_argmin(kx, kc)
    rows = np.arange(kx.shape[0])
    bad = got != want
    if not np.any(bad):
        return 0
    best = d[rows, want].astype(np.float64)
    chosen = d[rows, got.astype(np.int64)].astype(np.float64)
    gap = chosen - best
    bound = 2.0 * gamma(sd) / (1.0 - gamma(sd)) * best
    assert np.all(gap[bad] <= bound[bad] * 1.000001 + 0), (
        f"oracle outside the fp32 bound: rows {np.nonzero(bad & (gap > bound))[0][:5]}")
    return int(np.sum(bad))


def test_exact_fp16_full_range():
    """Random fp16 with |v| < 32 (subnormals included): exact int64 distances."""
    r = np.random.default_rng(5)
    exempt = 0
    total = 0
    for case in range(400):
        sd = int(r.choice([1, 2, 4, 8]))
        n = int(r.integers(1, 64))
        n_c = int(r.integers(1, 64))
        xb = random_f16_bits(r, (n, sd), 19)
        cb = random_f16_bits(r, (n_c, sd), 19)
        if n_c > 2 and r.random() < 0.3:
            cb[r.integers(0, n_c)] = cb[r.integers(0, n_c)]   # an exact duplicate row
        if r.random() < 0.2:
            xb[0] = cb[r.integers(0, n_c)]                      # x equal to a centroid
        got = oracle.encode(xb, cb, sd, n_c, oracle.F16)
        exempt += _check_with_exemptions(f16_exact_int(xb), f16_exact_int(cb), got, sd)
        total += n
    assert exempt <= max(2, total // 1000), f"{exempt} exemptions out of {total}"


def test_exact_bf16_range():
    """bf16 with exponents in [-12, 3] (values on a 2^-19 grid): exact int64."""
    r = np.random.default_rng(6)
    exempt = 0
    total = 0
    for case in range(400):
        sd = int(r.choice([1, 4, 8]))
        n = int(r.integers(1, 64))
        n_c = int(r.integers(1, 64))
        xb = random_bf16_bits(r, (n, sd), -12, 3)
        cb = random_bf16_bits(r, (n_c, sd), -12, 3)
        if n_c > 2 and r.random() < 0.3:
            cb[r.integers(0, n_c)] = cb[r.integers(0, n_c)]
        got = oracle.encode(xb, cb, sd, n_c, oracle.BF16)
        exempt += _check_with_exemptions(bf16_exact_int(xb, 19), bf16_exact_int(cb, 19), got, sd)
        total += n
    assert exempt <= max(2, total // 1000), f"{exempt} exemptions out of {total}"


def test_exact_rational_extreme_magnitudes():
    """Huge and tiny fp16/bf16 values with exact rational distances (Python
    Fractions), where int64 would overflow."""
    r = np.random.default_rng(7)
    for case in range(60):
        dtype = oracle.F16 if case % 2 == 0 else oracle.BF16
        sd = int(r.choice([4, 8]))
        n, n_c = 3, 12
        if dtype == oracle.F16:
            xb = random_f16_bits(r, (n, sd), 30)
            cb = random_f16_bits(r, (n_c, sd), 30)
            xv = xb.view(np.float16).astype(np.float64)
            cv = cb.view(np.float16).astype(np.float64)
        else:
            xb = random_bf16_bits(r, (n, sd), -60, 30)
            cb = random_bf16_bits(r, (n_c, sd), -60, 30)
            xv = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            cv = (cb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        got = oracle.encode(xb, cb, sd, n_c, dtype)
        for i in range(n):
            ex = [sum((Fraction(xv[i, k]) - Fraction(cv[c, k])) ** 2 for k in range(sd))
                  for c in range(n_c)]
            f32max = Fraction(float(np.finfo(np.float32).max))
            finite = [c for c in range(n_c) if ex[c] <= f32max * Fraction(1, 2)]
            if not finite:
                continue
            best = min(ex[c] for c in finite)
            want = min(c for c in finite if ex[c] == best)
            if int(got[i]) != want:
                g = ex[int(got[i])]
                bound = Fraction(2.0 * gamma(sd) / (1 - gamma(sd)) * 1.000001) * best
                assert g - best <= bound, f"case {case} row {i}"


# --------------------------------------------------------------------------
# hand-built known answers
# --------------------------------------------------------------------------

def _f16(a):
    return W.to_f16_bits(np.asarray(a, dtype=np.float64))


def test_x_equal_to_a_centroid_gives_that_index():
    r = np.random.default_rng(3)
    cb = _f16(r.standard_normal((64, 8)))
    for c in [0, 1, 17, 63]:
        xb = cb.reshape(64, 8)[c:c + 1].copy()
        idx, best, _ = oracle.encode_top2(xb, cb, 8, 64, oracle.F16)
        assert idx[0] == c and best[0] == 0.0


def test_x_equal_to_a_duplicated_centroid_gives_the_first_copy():
    r = np.random.default_rng(4)
    cb = _f16(r.standard_normal((32, 4))).reshape(32, 4)
    cb[5] = cb[20]
    cb[29] = cb[20]
    for row in (5, 20, 29):
        got = oracle.encode(cb[row:row + 1], cb, 4, 32, oracle.F16)
        assert got[0] == 5


def test_equidistant_axis_rows_resolve_to_lowest_index():
    # x = 0 and rows +-s*e_i are all at distance s^2.
    sd = 4
    rows = []
    for i in range(sd):
        for sgn in (+1, -1):
            e = np.zeros(sd)
            e[i] = 0.75 * sgn
            rows.append(e)
    rows = np.array(rows)
    for perm_seed in range(5):
        perm = np.random.default_rng(perm_seed).permutation(len(rows))
        cb = _f16(rows[perm])
        got = oracle.encode(_f16(np.zeros((1, sd))), cb, sd, len(rows), oracle.F16)
        assert got[0] == 0
    # a farther row placed first must lose, the first nearer row must win
    cb = _f16(np.vstack([[[2, 0, 0, 0]], rows]))
    assert oracle.encode(_f16(np.zeros((1, sd))), cb, sd, len(rows) + 1, oracle.F16)[0] == 1


def test_identical_rows_and_single_centroid_give_zero():
    r = np.random.default_rng(9)
    xb = _f16(r.standard_normal((100, 8)))
    same = np.tile(_f16(r.standard_normal((1, 8))), (50, 1))
    assert np.all(oracle.encode(xb, same, 8, 50, oracle.F16) == 0)
    assert np.all(oracle.encode(xb, same[:1], 8, 1, oracle.F16) == 0)


def test_reversed_codebook_reverses_indices():
    r = np.random.default_rng(10)
    xb = _f16(r.standard_normal((500, 4)))
    cb = _f16(r.standard_normal((97, 4))).reshape(97, 4)
    a = oracle.encode(xb, cb, 4, 97, oracle.F16)
    b = oracle.encode(xb, cb[::-1].copy(), 4, 97, oracle.F16)
    _, best, second = oracle.encode_top2(xb, cb, 4, 97, oracle.F16)
    distinct = best < second
    assert np.all(b[distinct] == 96 - a[distinct])


def test_non_finite_inputs():
    nan, inf = np.nan, np.inf
    cb = _f16([[0, 0, 0, 0], [1, 1, 1, 1], [2, 2, 2, 2]])
    # NaN in x: every distance is NaN, nothing beats +inf -> index 0
    assert oracle.encode(_f16([[1, nan, 1, 1]]), cb, 4, 3, oracle.F16)[0] == 0
    # +inf in x: every distance is +inf -> index 0
    assert oracle.encode(_f16([[2, 2, inf, 2]]), cb, 4, 3, oracle.F16)[0] == 0
    # a NaN row never wins, even when it comes first
    cbn = _f16([[nan, 0, 0, 0], [5, 5, 5, 5], [1, 1, 1, 1]])
    assert oracle.encode(_f16([[1, 1, 1, 1]]), cbn, 4, 3, oracle.F16)[0] == 2
    # an infinite row never wins either
    cbi = _f16([[inf, 0, 0, 0], [3, 3, 3, 3]])
    assert oracle.encode(_f16([[0, 0, 0, 0]]), cbi, 4, 2, oracle.F16)[0] == 1
    # squared differences that overflow fp32 (bf16 has fp32's range)
    big = W.to_bf16_bits(np.array([[3e38, 0, 0, 0], [-3e38, 0, 0, 0], [1e19, 0, 0, 0]]))
    x0 = W.to_bf16_bits(np.zeros((1, 4)))
    # distances: inf, inf, 1e38 -> index 2
    assert oracle.encode(x0, big, 4, 3, oracle.BF16)[0] == 2


def test_subnormal_differences_are_kept():
    # bf16 values around 1e-20: squares are fp32 subnormal or zero; with
    # subnormals kept the nearer row still wins.
    x = W.to_bf16_bits(np.array([[1e-20, 0, 0, 0]]))
    cb = W.to_bf16_bits(np.array([[4e-20, 0, 0, 0], [2e-20, 0, 0, 0]]))
    d0 = oracle.sqdist(x[0], cb[0], oracle.BF16)
    d1 = oracle.sqdist(x[0], cb[1], oracle.BF16)
    assert 0.0 < d1 < d0
    assert oracle.encode(x, cb, 4, 2, oracle.BF16)[0] == 1


# --------------------------------------------------------------------------
# sub_dim = 1: boundary-sum scalar quantization
# --------------------------------------------------------------------------

def test_sub_dim_one_equals_boundary_sum():
    """With sub_dim 1 and a sorted codebook, the nearest index is the number
    of centroid midpoints the value strictly exceeds (VeloxQuant-MLX blog,
    residual-VQ benchmark post, section "The Throughput Problem (and How We
    Solved It)", change 3; and the getting-started guide, "Step 9").  On the
    k/64 grid the oracle's fp32 arithmetic is exact, so the match is exact,
    including values sitting exactly on a midpoint (lowest index wins)."""
    r = np.random.default_rng(12)
    hits = 0
    for case in range(300):
        n_c = int(r.integers(1, 40))
        kc = np.sort(r.choice(np.arange(-255, 256), size=n_c, replace=False))
        kx = r.integers(-300, 301, size=200)
        kx = np.clip(kx, -255, 255)
        cb = W.to_f16_bits(kc / 64.0)
        xb = W.to_f16_bits(kx / 64.0)
        mid2 = kc[:-1] + kc[1:]                      # 2 * midpoint, exact
        want = np.sum(2 * kx[:, None] > mid2[None, :], axis=1)
        hits += int(np.sum(np.any(2 * kx[:, None] == mid2[None, :], axis=1)))
        got = oracle.encode(xb.reshape(-1, 1), cb, 1, n_c, oracle.F16)
        assert np.array_equal(got, want.astype(np.uint32)), f"case {case}"
    assert hits > 500, "midpoint ties should be exercised"


# --------------------------------------------------------------------------
# groups, slots, the top-2 report, decode, threading
# --------------------------------------------------------------------------

def test_group_slots_select_the_right_codebook():
    # slot s: row j is 10*(j - s) in every component, so x = 0 picks row s.
    sd, n_c, n_slots = 4, 6, 5
    stride = n_c * sd + 3
    cb = np.zeros(n_slots * stride, np.uint16)
    for s in range(n_slots):
        rows = np.array([[10.0 * (j - s)] * sd for j in range(n_c)])
        cb[s * stride: s * stride + n_c * sd] = _f16(rows).reshape(-1)
    n, glen = 37, 8
    xb = _f16(np.zeros((n, sd)))
    got = oracle.encode(xb, cb, sd, n_c, oracle.F16, codebook_stride=stride,
                        n_codebooks=n_slots, group_len=glen)
    assert np.array_equal(got, (np.arange(n) // glen).astype(np.uint32))
    gmap = np.array([3, 0, 4, 4, 1], np.int32)
    got = oracle.encode(xb, cb, sd, n_c, oracle.F16, codebook_stride=stride,
                        n_codebooks=n_slots, group_len=glen, group_map=gmap)
    assert np.array_equal(got, gmap[np.arange(n) // glen].astype(np.uint32))
    bad = np.array([3, -1, 5, 0, 1], np.int32)
    got = oracle.encode(xb, cb, sd, n_c, oracle.F16, codebook_stride=stride,
                        n_codebooks=n_slots, group_len=glen, group_map=bad)
    g = np.arange(n) // glen
    assert np.all(got[(g == 1) | (g == 2)] == oracle.BAD_SLOT)
    assert np.all(got[g == 0] == 3) and np.all(got[g == 4] == 1)


def test_top2_report_is_consistent():
    r = np.random.default_rng(13)
    sd, n_c, n = 8, 40, 60
    xb = _f16(r.standard_normal((n, sd)))
    cb = _f16(r.standard_normal((n_c, sd))).reshape(n_c, sd)
    cb[7] = cb[30]
    idx, best, second = oracle.encode_top2(xb, cb, sd, n_c, oracle.F16)
    assert np.array_equal(idx, oracle.encode(xb, cb, sd, n_c, oracle.F16))
    for i in range(n):
        d = np.array([oracle.sqdist(xb[i], cb[c], oracle.F16) for c in range(n_c)], np.float32)
        assert best[i] == d.min() and d[idx[i]] == best[i]
        assert second[i] == np.delete(d, idx[i]).min()
    one_idx, one_best, one_second = oracle.encode_top2(xb, cb[:1], sd, 1, oracle.F16)
    assert np.all(one_idx == 0) and np.all(np.isinf(one_second))


def test_decode_gathers_rows_and_zeroes_bad_indices():
    r = np.random.default_rng(14)
    sd, n_c = 8, 16
    cb = _f16(r.standard_normal((n_c, sd))).reshape(n_c, sd)
    idx = np.array([0, 15, 3, 16, 0xFFFFFFFF, 7], np.uint32)
    out = oracle.decode(idx, cb, sd, n_c, oracle.F16)
    for k, i in enumerate(idx):
        want = cb[i] if i < n_c else np.zeros(sd, np.uint16)
        assert np.array_equal(out[k], want)


def test_decoded_row_is_never_farther_than_any_centroid():
    wl = W.random_case(21, 700, 8, 64, W.F16)
    idx = oracle.encode(wl.x, wl.codebook, 8, 64, wl.dtype)
    rec = oracle.decode(idx, wl.codebook, 8, 64, wl.dtype)
    cb = wl.codebook.reshape(64, 8)
    for i in range(0, 700, 7):
        dmin = oracle.sqdist(wl.x[i], rec[i], wl.dtype)
        assert all(dmin <= oracle.sqdist(wl.x[i], cb[c], wl.dtype) for c in range(64))


def test_threaded_slices_equal_single_thread():
    wl = W.random_case(22, 20000, 4, 32, W.F16, n_codebooks=3, group_len=7001)
    a = oracle.encode(wl.x, wl.codebook, 4, 32, wl.dtype, **wl.kwargs())
    b = oracle.encode(wl.x, wl.codebook, 4, 32, wl.dtype, threads=5, **wl.kwargs())
    assert np.array_equal(a, b)
    rows = np.array([0, 7000, 7001, 19999])
    c = oracle.encode_rows(wl.x, wl.codebook, rows, 4, 32, wl.dtype, **wl.kwargs())
    assert np.array_equal(c, a[rows])


def test_rejects_bad_arguments():
    xb = _f16(np.zeros((4, 4)))
    with pytest.raises(ValueError):
        oracle.encode(xb, xb, 4, 0, oracle.F16)
    with pytest.raises(ValueError):
        oracle.encode(xb, xb, 4, 1, 7)
