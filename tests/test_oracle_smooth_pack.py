"""Pins for the oracle's smoothing, fp32 search and packed-code functions.

What is pinned, and against what (none of it re-uses the oracle's own code):
  * the packed stream against numpy's ``packbits(bitorder="little")`` for
    every width 1..32, and against the examples worked by hand from the pages'
    text in ``tests/golden/pack_examples.txt`` (each cited there);
  * smoothing against numpy's float32 multiply in the natural
    ``[tokens, head_dim]`` layout (broadcasting, not the oracle's index
    arithmetic);
  * power-of-two factors, where smoothing is exact and the whole encode must
    equal the already-pinned ``encode`` on keys pre-scaled in fp16;
  * the search over smoothed keys against exact rational brute force (Python
    integers), exempting only gaps inside the fp32 error bound;
  * slot selection of the factor vector against per-slot calls.
"""
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_examples.txt")


def _golden():
    cases = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        kv = dict(part.split("=") for part in line.split())
        cases.append((int(kv["bits"]), [int(v) for v in kv["codes"].split(",")],
                      [int(v) for v in kv["bytes"].split(",")]))
    return cases


def test_pack_golden_examples_from_the_pages():
    cases = _golden()
    assert len(cases) >= 4
    for bits, codes, want in cases:
        got = oracle.pack(np.array(codes, dtype=np.uint32), bits)
        assert got.tolist() == want, (bits, codes)
        assert oracle.unpack(got, len(codes), bits).tolist() == codes


@pytest.mark.parametrize("bits", list(range(1, 33)))
def test_pack_matches_numpy_little_endian_bits(bits):
    r = np.random.default_rng([77, bits])
    for n in (0, 1, 7, 8, 9, 63, 64, 65, 1000):
        codes = r.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
        stream_bits = ((codes[:, None].astype(np.uint64) >> np.arange(bits, dtype=np.uint64))
                       & 1).astype(np.uint8).reshape(-1)
        want = np.packbits(stream_bits, bitorder="little")
        got = oracle.pack(codes, bits)
        assert got.size == (n * bits + 7) // 8
        np.testing.assert_array_equal(got, want)
        mask = np.uint64((1 << bits) - 1)
        np.testing.assert_array_equal(oracle.unpack(got, n, bits),
                                      (codes.astype(np.uint64) & mask).astype(np.uint32))


def _cache(seed, tokens, heads, head_dim, sub_dim, dtype=W.F16, lo=None):
    """Keys [heads, tokens, head_dim] and their sub-vector view."""
    r = np.random.default_rng([500, seed])
    k = r.standard_normal((heads, tokens, head_dim)) * np.exp(0.5 * r.standard_normal(head_dim))
    if lo is not None:
        k = np.where(np.abs(k) < lo, np.sign(k + 1e-300) * lo, k)
    bits = W.to_f16_bits(k) if dtype == W.F16 else W.to_bf16_bits(k)
    return bits.reshape(heads, tokens, head_dim), bits.reshape(-1, sub_dim)


def test_smooth_matches_numpy_float32_multiply_in_cache_layout():
    for dtype in (W.F16, W.BF16):
        for sd, hd in ((4, 256), (8, 128), (4, 12)):
            kbits, xs = _cache(1 + sd + dtype, 9, 3, hd, sd, dtype)
            scale = np.exp(np.random.default_rng([501, sd]).standard_normal(hd)).astype(np.float32)
            want = W.bits_to_f32(kbits, dtype) * scale[None, None, :]   # float32 * float32
            got = oracle.smooth(xs, sd, dtype, channel_scale=scale, head_dim=hd)
            np.testing.assert_array_equal(got.view(np.uint32),
                                          want.astype(np.float32).reshape(-1, sd).view(np.uint32))
            # no factors: the exact widening
            np.testing.assert_array_equal(oracle.smooth(xs, sd, dtype, head_dim=hd),
                                          W.bits_to_f32(xs, dtype))


def test_unit_factors_reduce_to_the_plain_encode():
    wl = W.random_case(3, 700, 8, 100)
    plain = oracle.encode(wl.x, wl.codebook, 8, 100, W.F16)
    ones = np.ones(16, dtype=np.float32)
    for sc in (None, ones):
        got = oracle.encode_packed(wl.x, wl.codebook, 8, 100, W.F16, channel_scale=sc,
                                   head_dim=16, code_bits=32)
        np.testing.assert_array_equal(got.view(np.uint32), plain)
        got8 = oracle.encode_packed(wl.x, wl.codebook, 8, 100, W.F16, channel_scale=sc,
                                    head_dim=16, code_bits=8)
        np.testing.assert_array_equal(got8, plain.astype(np.uint8))


def test_power_of_two_factors_equal_encode_of_prescaled_keys():
    """Multiplying by 2^k is exact, so smoothing then searching must equal
    searching fp16 keys pre-scaled exactly (built with numpy in the cache
    layout)."""
    sd, hd, heads, tokens = 4, 32, 2, 40
    kbits, xs = _cache(7, tokens, heads, hd, sd, lo=2.0 ** -4)
    k = W.bits_to_f32(kbits, W.F16).astype(np.float64)
    expo = np.random.default_rng(8).integers(-2, 3, size=hd)
    scale = np.ldexp(1.0, expo)
    pre = k * scale[None, None, :]
    pre_bits = W.to_f16_bits(pre)
    assert np.array_equal(pre_bits.view(np.float16).astype(np.float64), pre)  # exact
    cb = W.to_f16_bits(2.0 * np.random.default_rng(9).standard_normal((64, sd))).reshape(-1)
    want = oracle.encode(pre_bits.reshape(-1, sd), cb, sd, 64, W.F16)
    got = oracle.encode_packed(xs, cb, sd, 64, W.F16, channel_scale=scale.astype(np.float32),
                               head_dim=hd, code_bits=32).view(np.uint32)
    np.testing.assert_array_equal(got, want)
    assert len(np.unique(want)) > 20


_SHIFT = 200  # every fp32 value (subnormals included) times 2^200 is an integer


def _as_int(v: np.ndarray):
    """Exact integer value of float32 numbers times 2^_SHIFT (a float32 has
    at most 24 significant bits, so the shift never drops a set bit)."""
    out = []
    for f in np.asarray(v, dtype=np.float32).reshape(-1):
        m, e = np.frexp(np.float64(f))           # exact for float32 inputs
        mi = int(np.ldexp(m, 53))                 # 53-bit integer mantissa
        sh = int(e) - 53 + _SHIFT
        out.append(mi << sh if sh >= 0 else mi >> -sh)
    return out


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_smoothed_search_against_exact_rational_brute_force(dtype):
    exempt = 0
    total = 0
    for seed in range(40):
        r = np.random.default_rng([502, seed, dtype])
        sd = (4, 8)[seed % 2]
        hd = sd * int(r.integers(1, 5))
        n_c = int(r.integers(1, 48))
        kbits, xs = _cache(600 + seed, int(r.integers(1, 9)), 1, hd, sd, dtype)
        cb_real = r.standard_normal((n_c, sd)) * (0.5 + r.random())
        if seed % 5 == 0 and n_c > 3:
            cb_real[n_c - 1] = cb_real[1]          # an exact duplicate row
        cb = (W.to_f16_bits(cb_real) if dtype == W.F16 else W.to_bf16_bits(cb_real)).reshape(-1)
        scale = np.exp(0.7 * r.standard_normal(hd)).astype(np.float32)
        got = oracle.encode_packed(xs, cb, sd, n_c, dtype, channel_scale=scale, head_dim=hd,
                                   code_bits=32).view(np.uint32)
        xt = (W.bits_to_f32(kbits, dtype) * scale).astype(np.float32).reshape(-1, sd)
        ci = [_as_int(W.bits_to_f32(cb.reshape(n_c, sd)[c], dtype)) for c in range(n_c)]
        for row in range(xt.shape[0]):
            xi = _as_int(xt[row])
            d = [sum((a - b) ** 2 for a, b in zip(xi, ci[c])) for c in range(n_c)]
            best = min(d)
            exact = d.index(best)
            total += 1
            if got[row] == exact:
                continue
            # fp32 evaluation error: at most (2 sd + 1) u of the distance
            bound = (2 * sd + 1) * 2 ** -24 * max(d[got[row]], best) * 1.01
            assert d[got[row]] - best <= bound, (seed, row, got[row], exact)
            exempt += 1
    assert total > 300
    assert exempt <= total // 50


def test_factor_vector_follows_the_codebook_slot():
    sd, hd, n_slots, glen = 8, 32, 3, 24
    r = np.random.default_rng(503)
    n = glen * 5
    x = W.to_f16_bits(r.standard_normal((n, sd)))
    cb = W.to_f16_bits(r.standard_normal((n_slots, 50, sd))).reshape(-1)
    scales = np.exp(r.standard_normal((n_slots, hd))).astype(np.float32)
    gmap = np.array([2, 0, 1, 2, 1], dtype=np.int32)
    stride = hd + 5
    sc_buf = np.zeros(n_slots * stride, dtype=np.float32)
    for s in range(n_slots):
        sc_buf[s * stride: s * stride + hd] = scales[s]
    got = oracle.encode_packed(x, cb, sd, 50, W.F16, channel_scale=sc_buf, head_dim=hd,
                               scale_stride=stride, code_bits=8, n_codebooks=n_slots,
                               group_len=glen, group_map=gmap)
    for g in range(5):
        s = int(gmap[g])
        part = oracle.encode_packed(x[g * glen:(g + 1) * glen], cb[s * 50 * sd:(s + 1) * 50 * sd],
                                    sd, 50, W.F16, channel_scale=scales[s], head_dim=hd,
                                    code_bits=8)
        np.testing.assert_array_equal(got[g * glen:(g + 1) * glen], part)
    # one shared vector (stride 0) differs from per-slot vectors
    shared = oracle.encode_packed(x, cb, sd, 50, W.F16, channel_scale=scales[0], head_dim=hd,
                                  scale_stride=0, code_bits=8, n_codebooks=n_slots,
                                  group_len=glen, group_map=gmap)
    assert not np.array_equal(shared, got)


def test_bad_slot_gets_all_ones_code_and_threads_agree():
    wl = W.random_case(11, 300, 4, 20, n_codebooks=2, group_len=64, use_map=True)
    gmap = wl.group_map.copy()
    gmap[1] = 7
    gmap[3] = -1
    sc = np.exp(np.random.default_rng(504).standard_normal(8)).astype(np.float32)
    kw = dict(codebook_stride=wl.codebook_stride, n_codebooks=2, group_len=64, group_map=gmap,
              channel_scale=sc, head_dim=8, code_bits=5)
    a = oracle.encode_packed(wl.x, wl.codebook, 4, 20, W.F16, **kw)
    codes = oracle.unpack(a, 300, 5)
    assert (codes[64:128] == 31).all() and (codes[192:256] == 31).all()
    assert (codes[:64] < 20).all()
    b = oracle.encode_packed(wl.x, wl.codebook, 4, 20, W.F16, threads=4, **kw)
    np.testing.assert_array_equal(a, b)


def test_encode_f32_top2_second_is_the_runner_up():
    r = np.random.default_rng(505)
    cb = W.to_f16_bits(r.standard_normal((30, 4))).reshape(-1)
    xs = r.standard_normal((50, 4)).astype(np.float32)
    idx, best, second = oracle.encode_f32(xs, cb, 4, 30, W.F16, want_top2=True)
    c = W.bits_to_f32(cb, W.F16).reshape(30, 4).astype(np.float64)
    d = ((xs.astype(np.float64)[:, None, :] - c[None]) ** 2).sum(-1)
    srt = np.sort(d, axis=1)
    np.testing.assert_allclose(best, srt[:, 0], rtol=1e-6)
    np.testing.assert_allclose(second, srt[:, 1], rtol=1e-6)
    np.testing.assert_array_equal(idx, oracle.encode_f32(xs, cb, 4, 30, W.F16))


def test_packed_arguments_rejected():
    wl = W.random_case(12, 10, 4, 257)
    with pytest.raises(ValueError):
        oracle.encode_packed(wl.x, wl.codebook, 4, 257, W.F16, code_bits=8)
    with pytest.raises(ValueError):
        oracle.encode_packed(wl.x, wl.codebook, 4, 257, W.F16, code_bits=0)
    with pytest.raises(ValueError):
        oracle.smooth(wl.x, 4, W.F16, head_dim=6)
    assert oracle.encode_packed(wl.x, wl.codebook, 4, 257, W.F16, code_bits=9).size == 12
