"""GPU parity of the fused encode (per-channel smoothing + packed codes).

``vq_encode_packed`` through its C ABI against the oracle's ``encode_packed``
(smooth, search, pack), byte for byte.  Small seeded cases cover every code
width class (1, 3, 4, 6, 8, 9 .. 13, 32 bits), both element types, both
sub-vector lengths, every kernel form (matrix-core with and without the fp32
codebook copy, one and two columns per wave, the direct kernel beyond 4096
centroids), ragged tails, several slots with per-slot factors, group maps with
bad slots, and extreme factors (overflow, subnormal, zero, negative, NaN).
The smoothed Falcon3-7B-shape cache and the smoothed full cache (33,554,432
sub-vectors, 256 slots) run at full size and every row is checked.  Acceptance: the same rule as the plain encode (exact equality
except near-ties within 1e-6 relative); the kernels are exact, so every byte
is required to match.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import product_vq_kv_amd as vq  # noqa: E402  (raises if the library is missing)

from tests.test_parity_gpu import to_dev  # noqa: E402

DEV = torch.device("cuda:0")
GUARD = 64


def scale_buffer(scale: np.ndarray, pad: int = 0):
    """[slots, head_dim] factors as a device tensor with row stride head_dim + pad."""
    slots, hd = scale.shape
    buf = np.full((slots, hd + pad), np.nan, dtype=np.float32)
    buf[:, :hd] = scale
    return torch.from_numpy(buf).to(DEV)[:, :hd]


def gpu_packed(wl, code_bits, scale_pad=0):
    """GPU code stream (numpy uint8), with a guard region checked after the call."""
    x, cb3, gmap = to_dev(wl)
    cb = cb3[0] if wl.n_codebooks == 1 else cb3
    sc = None
    if wl.channel_scale is not None:
        sc = scale_buffer(wl.channel_scale, scale_pad)
        if sc.shape[0] == 1:
            sc = sc[0]
    nbytes = vq.packed_bytes(wl.n, code_bits)
    buf = torch.full((nbytes + GUARD,), 0xAB, dtype=torch.uint8, device=DEV)
    vq.encode_packed(x, cb, channel_scale=sc, head_dim=wl.head_dim, code_bits=code_bits,
                     group_len=wl.group_len, group_map=gmap, out=buf)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[nbytes:] == 0xAB), "bytes past the code stream were written"
    return host[:nbytes]


def oracle_packed(wl, code_bits):
    return oracle.encode_packed(wl.x, wl.codebook, wl.sub_dim, wl.n_centroids, wl.dtype,
                                code_bits=code_bits, threads=parity.oracle_threads(),
                                **wl.kwargs(), **wl.packed_kwargs())


def assert_packed_parity(wl, got, code_bits):
    want = oracle_packed(wl, code_bits)
    if np.array_equal(got, want):
        print(f"[parity] {wl.name} bits={code_bits}: {wl.n} codes identical", flush=True)
        return
    g = oracle.unpack(got, wl.n, code_bits)
    w = oracle.unpack(want, wl.n, code_bits)
    bad = np.nonzero(g != w)[0]
    # diagnose with the oracle's top-2 over the smoothed keys
    xs = oracle.smooth(wl.x, wl.sub_dim, wl.dtype, **wl.packed_kwargs(),
                       n_codebooks=wl.n_codebooks, group_len=wl.group_len,
                       group_map=wl.group_map)
    _, best, second = oracle.encode_f32(xs, wl.codebook, wl.sub_dim, wl.n_centroids, wl.dtype,
                                        codebook_stride=wl.codebook_stride,
                                        n_codebooks=wl.n_codebooks, group_len=wl.group_len,
                                        group_map=wl.group_map, want_top2=True)
    near = [(int(r), int(g[r]), int(w[r]), float(best[r]), float(second[r])) for r in bad[:8]]
    pytest.fail(f"{wl.name} bits={code_bits}: {bad.size} codes differ; first (row, gpu, oracle, "
                f"best, second): {near}")


def with_factors(wl, seed, head_mult=2, per_slot=True):
    """Attach seeded per-channel factors exp(0.7 z) to a random case."""
    r = np.random.default_rng([900, seed])
    hd = wl.sub_dim * head_mult
    slots = wl.n_codebooks if per_slot else 1
    wl.channel_scale = np.exp(0.7 * r.standard_normal((slots, hd))).astype(np.float32)
    wl.head_dim = hd
    return wl


PACKED = [
    # (seed, n, sd, n_c, dtype, code_bits, factors, head_mult, random_case extras)
    (1, 1, 8, 256, W.F16, 8, True, 16, {}),
    (2, 255, 4, 256, W.F16, 8, True, 64, {}),
    (3, 1023, 8, 16, W.BF16, 4, True, 16, {}),
    (4, 5000, 4, 7, W.F16, 3, True, 3, {}),
    (5, 4099, 8, 2, W.F16, 1, True, 16, {}),
    (6, 3333, 4, 1, W.F16, 1, True, 2, {}),
    (7, 2500, 8, 1000, W.F16, 10, True, 16, {}),
    (8, 2500, 4, 1025, W.BF16, 11, True, 32, {}),
    (9, 3000, 8, 4096, W.BF16, 12, True, 16, dict(dup_frac=0.05)),
    (10, 2100, 8, 5000, W.F16, 13, True, 16, {}),
    (11, 7000, 4, 300, W.F16, 9, True, 64, dict(n_codebooks=7, group_len=1024, stride_pad=5)),
    (12, 9000, 8, 256, W.F16, 8, True, 16, dict(n_codebooks=4, group_len=2048, use_map=True)),
    (13, 20000, 4, 256, W.F16, 8, False, 1, {}),
    (14, 1500, 8, 256, W.BF16, 32, True, 4, {}),
    (15, 6000, 4, 64, W.F16, 6, True, 4, dict(n_codebooks=3, group_len=16, use_map=True)),
    (16, 8192, 4, 256, W.F16, 8, True, 64, dict(dup_frac=0.2, scale=10.0)),
    (17, 3000, 8, 33, W.BF16, 7, True, 1, dict(scale=1e-3)),
    # no factors, byte-wide codes: the plain kernel writes them directly
    (18, 6000, 8, 300, W.F16, 16, False, 1, dict(n_codebooks=3, group_len=1024, use_map=True)),
    (19, 7777, 4, 200, W.BF16, 8, False, 1, dict(n_codebooks=2, group_len=4000)),
    # |c|^2 / 2 beyond the fp16 range: the slot takes the unfolded form (with
    # duplicate rows in it)
    (20, 8192, 4, 256, W.F16, 8, True, 64, dict(scale=300.0)),
    (21, 8192, 4, 256, W.F16, 8, True, 16, dict(dup_frac=0.2, scale=300.0)),
    # 128 sub-slots per key (head_dim 512 / 1024): a unit's first row and a
    # group's first row sit at nonzero sub-slots (power-of-two form); group
    # lengths that are not multiples of the key length
    (22, 4700, 4, 256, W.F16, 8, True, 128, dict(n_codebooks=5, group_len=1000)),
    (23, 5000, 8, 256, W.F16, 8, True, 128, dict(n_codebooks=3, group_len=1800)),
    (24, 3000, 4, 300, W.BF16, 9, True, 256, dict(n_codebooks=2, group_len=2016)),
    # key lengths that are not a power of two (general sub-slot form): sub_dim
    # 8, bf16, more than 1024 centroids, several groups
    (25, 3000, 8, 2000, W.BF16, 11, True, 10, dict(n_codebooks=2, group_len=1600)),
    (26, 2600, 4, 1500, W.BF16, 11, True, 24, {}),
    (27, 3000, 8, 256, W.F16, 8, True, 12, dict(n_codebooks=3, group_len=1004)),
    (28, 4000, 4, 256, W.F16, 8, True, 20, dict(n_codebooks=4, group_len=1004, use_map=True)),
    (29, 2100, 8, 5000, W.BF16, 13, True, 6, {}),
]


@pytest.mark.parametrize("case", PACKED,
                         ids=[f"p{c[0]}_n{c[1]}_sd{c[2]}_nc{c[3]}_b{c[5]}" for c in PACKED])
def test_packed_small_cases_match_oracle(case):
    seed, n, sd, n_c, dt, bits, factors, hm, extra = case
    wl = W.random_case(100 + seed, n, sd, n_c, dt, **extra)
    if factors:
        with_factors(wl, seed, hm)
    print(f"[case] {wl.name} bits={bits} factors={factors} {extra}", flush=True)
    assert_packed_parity(wl, gpu_packed(wl, bits, scale_pad=3 if seed % 2 else 0), bits)


# Large enough that one workgroup (one per CU) owns several units of several
# groups (units taken from a counter in LDS, the slot and its factors
# restaged per segment).
MULTI = [
    # (seed, n, sd, n_c, dtype, code_bits, factors, head_mult, random_case extras)
    (60, 200_000, 4, 256, W.F16, 8, True, 64, dict(n_codebooks=9, group_len=4096, use_map=True)),
    (61, 150_000, 8, 64, W.BF16, 6, True, 16, dict(n_codebooks=5, group_len=1008, use_map=True)),
    (62, 120_000, 4, 32, W.F16, 5, True, 16, dict(n_codebooks=40, group_len=3200)),
]


@pytest.mark.parametrize("case", MULTI,
                         ids=[f"m{c[0]}_n{c[1]}_sd{c[2]}_nc{c[3]}_b{c[5]}" for c in MULTI])
def test_packed_multi_segment_workgroups_match_oracle(case):
    seed, n, sd, n_c, dt, bits, factors, hm, extra = case
    wl = W.random_case(100 + seed, n, sd, n_c, dt, **extra)
    if wl.group_map is not None:
        wl.group_map[::5] = -1
    if factors:
        with_factors(wl, seed, hm)
    print(f"[case] {wl.name} bits={bits} factors={factors} {extra}", flush=True)
    assert_packed_parity(wl, gpu_packed(wl, bits), bits)


def test_shared_factor_vector_across_slots():
    wl = W.random_case(140, 6000, 8, 128, W.F16, n_codebooks=3, group_len=1024, use_map=True)
    with_factors(wl, 40, 4, per_slot=False)
    assert_packed_parity(wl, gpu_packed(wl, 7), 7)


def test_without_factors_equals_plain_encode():
    wl = W.random_case(141, 10000, 4, 256, W.F16)
    x, cb3, _ = to_dev(wl)
    plain = vq.encode(x, cb3[0]).cpu().numpy().view(np.uint32)
    p32 = vq.encode_packed(x, cb3[0], code_bits=32).cpu().numpy().view(np.uint32)
    p8 = vq.encode_packed(x, cb3[0], code_bits=8).cpu().numpy()
    p16 = vq.encode_packed(x, cb3[0], code_bits=16).cpu().numpy().view(np.uint16)
    assert np.array_equal(plain, p32)
    assert np.array_equal(plain.astype(np.uint8), p8)
    assert np.array_equal(plain.astype(np.uint16), p16)


def test_bad_slots_give_all_one_codes():
    wl = W.random_case(142, 5000, 8, 32, W.F16, n_codebooks=3, group_len=704, use_map=True)
    wl.group_map = np.array([0, 2, -1, 1, 3, 2, 7, 0], np.int32)
    with_factors(wl, 42, 2)
    got = gpu_packed(wl, 5)
    codes = oracle.unpack(got, wl.n, 5)
    g = np.arange(wl.n) // wl.group_len
    assert np.all(codes[np.isin(g, [2, 4, 6])] == 31)
    assert_packed_parity(wl, got, 5)


@pytest.mark.parametrize("bits,factors", [(8, False), (16, False), (8, True)])
def test_bad_slots_all_one_codes_byte_widths(bits, factors):
    wl = W.random_case(148, 5000, 4, 100, W.F16, n_codebooks=3, group_len=704, use_map=True)
    wl.group_map = np.array([0, 2, -1, 1, 3, 2, 7, 0], np.int32)
    if factors:
        with_factors(wl, 48, 4)
    got = gpu_packed(wl, bits)
    codes = oracle.unpack(got, wl.n, bits)
    g = np.arange(wl.n) // wl.group_len
    assert np.all(codes[np.isin(g, [2, 4, 6])] == (1 << bits) - 1)
    assert_packed_parity(wl, got, bits)


def test_extreme_factors():
    sd, hd = 4, 16
    wl = W.random_case(143, 4000, sd, 64, W.F16)
    f = np.array([1e30, 1e-30, 0.0, -1.0, 3e4, 1e-8, 2.0 ** -20, np.nan,
                  1.0, 7.5, -0.001, 65504.0, 1e-3, 1e5, 1.0, np.inf], dtype=np.float32)
    wl.channel_scale = f[None, :]
    wl.head_dim = hd
    assert_packed_parity(wl, gpu_packed(wl, 6), 6)
    wlb = W.random_case(144, 4000, 8, 64, W.BF16)
    wlb.channel_scale = np.concatenate([f, f[::-1]])[None, :]
    wlb.head_dim = 32
    assert_packed_parity(wlb, gpu_packed(wlb, 6), 6)


@pytest.mark.parametrize("sd,dt", [(4, W.F16), (8, W.BF16)])
def test_near_tied_centroids_with_factors(sd, dt):
    # pairs of centroids one or two ulps apart in different 16-row groups and
    # smoothed keys between them: the bound must send every such column to
    # the exact stage
    r = np.random.default_rng(145 + sd)
    n_c, n, hd = 512, 20000, 4 * sd
    bits = W.to_f16_bits if dt == W.F16 else W.to_bf16_bits
    a = bits(r.standard_normal((n_c // 2, sd))).reshape(-1, sd)
    b = a.copy()
    b[:, 0] = b[:, 0] + r.integers(1, 3, size=b.shape[0]).astype(np.uint16)
    cb = np.empty((n_c, sd), np.uint16)
    perm = r.permutation(n_c)
    cb[perm[: n_c // 2]] = a
    cb[perm[n_c // 2:]] = b
    f = np.exp(0.3 * r.standard_normal(hd)).astype(np.float32)
    target = W.bits_to_f32(a, dt).astype(np.float64)[r.integers(0, n_c // 2, size=n)]
    ch = (np.arange(n) % (hd // sd))[:, None] * sd + np.arange(sd)[None, :]
    x = target / f[ch] + 1e-3 * r.standard_normal((n, sd))
    wl = W.Workload("near-tied pairs, smoothed", bits(x).reshape(-1, sd), cb.reshape(-1), sd, n_c,
                    dt, n_c * sd, 1, n, channel_scale=f[None, :], head_dim=hd)
    assert_packed_parity(wl, gpu_packed(wl, 9), 9)


def test_group_layout_that_splits_a_word_is_rejected():
    wl = W.random_case(146, 100, 4, 16, W.F16, n_codebooks=4, group_len=30)
    x, cb3, _ = to_dev(wl)
    with pytest.raises(vq.VQError, match="UNSUPPORTED"):
        vq.encode_packed(x, cb3, code_bits=4, group_len=30)
    with pytest.raises(vq.VQError, match="INVALID_ARG"):
        vq.encode_packed(x, cb3, code_bits=3, group_len=32)


def test_full_size_falcon_smoothed_every_row():
    wl = W.falcon_smoothed()
    print(f"[case] {wl.name}", flush=True)
    assert_packed_parity(wl, gpu_packed(wl, 8), 8)


def test_full_cache_smoothed_every_row():
    """The smoothed full cache (33,554,432 sub-vectors, 256 slots with their
    own factors): every code byte against the oracle."""
    wl = W.full_cache_smoothed()
    print(f"[case] {wl.name} n={wl.n}", flush=True)
    assert wl.n == 33554432
    assert_packed_parity(wl, gpu_packed(wl, 8), 8)


def test_smoothed_keys_beyond_the_fp16_error_operand():
    """Factors of about 2^14 lift smoothed keys past 2^26 in norm: the error
    term's key operand b' no longer fits fp16, so the bounds of those keys
    become -inf and every group of theirs is evaluated exactly (fp32 distances
    near 1e16 also tie often).  The codes must still equal the oracle's."""
    wl = W.random_case(42, 6000, 4, 256, W.F16, scale=1000.0)
    wl = with_factors(wl, 42, head_mult=16, per_slot=False)
    wl.channel_scale = (wl.channel_scale * np.float32(2.0 ** 14)).astype(np.float32)
    print(f"[case] {wl.name} factors x 2^14", flush=True)
    got = gpu_packed(wl, 8)
    assert_packed_parity(wl, got, 8)


@pytest.mark.parametrize("head_dim", [80, 128])
def test_one_group_past_2_32_rows_sampled(head_dim):
    """One group of 2^32 + 2^20 + 100 smoothed sub-vectors of sub_dim 4 (32 GiB
    of keys): unit offsets inside the group pass 2^32 rows, where the
    sub-slot of a unit's first row must still be (group start + offset) mod
    n_sub, for a key length that is not a power of two (80 / 4 = 20 sub-slots)
    and one that is (128 / 4 = 32).  Keys are drawn on the device; seeded whole
    keys around 2^32, at random and at the ragged tail are checked against
    the oracle."""
    sd = 4
    n_sub = head_dim // sd
    n = 2 ** 32 + 2 ** 20 + 100
    cbw = W.random_case(45, 1, sd, 256, W.F16)
    f = np.exp(0.5 * np.random.default_rng([901, head_dim]).standard_normal(head_dim))
    f = f.astype(np.float32)
    x = torch.empty(n, sd, dtype=torch.float16, device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(45)
    step = 2 ** 28
    for i in range(0, n, step):
        j = min(n, i + step)
        x[i:j] = torch.randn(j - i, sd, generator=gen, device=DEV).to(torch.float16)
    cb = torch.from_numpy(cbw.codebook.view(np.int16)).view(torch.float16).to(DEV).view(256, sd)
    codes = vq.encode_packed(x, cb, channel_scale=torch.from_numpy(f).to(DEV), head_dim=head_dim,
                             code_bits=8)
    torch.cuda.synchronize()
    rng = np.random.default_rng(45)
    key = 64 * n_sub          # whole keys of 64 tokens
    starts = [0, (2 ** 32 // n_sub) * n_sub - key, (2 ** 32 // n_sub) * n_sub,
              ((n - key) // n_sub) * n_sub]
    starts += [int(r) * n_sub for r in rng.integers(0, (n - key) // n_sub, 24)]
    checked = 0
    for r0 in starts:
        r1 = min(n, r0 + key)
        xs = x[r0:r1].cpu().view(torch.int16).numpy().view(np.uint16)
        got = codes[r0:r1].cpu().numpy()
        want = oracle.encode_packed(xs, cbw.codebook, sd, 256, W.F16, channel_scale=f,
                                    head_dim=head_dim, code_bits=8)
        assert np.array_equal(got, want), f"rows {r0}..{r1} (head_dim {head_dim})"
        checked += r1 - r0
    del x, codes
    torch.cuda.empty_cache()
    print(f"[parity] one group of {n} rows, head_dim {head_dim}: {checked} sampled rows equal",
          flush=True)
