"""GPU parity of K-means calibration (vq_kmeans) against the CPU oracle.

Every update is the exact member mean rounded once to the element type (fp16
or bf16) on both sides, so the codebooks and assignments must be
bit-identical after every iteration.  bf16 cases cover both sub-dims, LDS-
and global-sized codebooks, the direct kernel, slots and maps, members whose
exponents span the whole bf16 range (sums across every limb, with carries),
subnormal and non-finite components, and 2^18 sub-vectors of the
large-codebook workload (4,096 centroids with duplicate rows).
Cases cover sub_dim 4 and 8, LDS and global accumulation (n_centroids above
512), the matrix-core and direct assignment kernels (up to 5000 centroids),
several slots with group maps and bad slots, workgroups spanning several
groups, member sums at the limit of their exact accumulation, exactly
representable clusters,
the Falcon3-7B keys at full size, and whole slots sampled from the 256-slot
full cache trained in one call.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle import kmeans as K

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import product_vq_kv_amd as vq  # noqa: E402

from tests.test_parity_gpu import to_dev  # noqa: E402

DEV = torch.device("cuda:0")


def gpu_kmeans(wl, iterations):
    x, cb3, gmap = to_dev(wl)
    cb = cb3[0] if wl.n_codebooks == 1 else cb3
    idx = vq.kmeans(x, cb, iterations, group_len=wl.group_len, group_map=gmap)
    torch.cuda.synchronize()
    full = cb3.reshape(wl.n_codebooks, -1).view(torch.int16).cpu().numpy().view(np.uint16)
    return full, idx.cpu().numpy().view(np.uint32)


def slots_of(cb_flat, wl):
    """[n_codebooks, n_c * sd] view of a flat codebook buffer."""
    return np.stack([cb_flat[s * wl.codebook_stride: s * wl.codebook_stride
                             + wl.n_centroids * wl.sub_dim] for s in range(wl.n_codebooks)])


def assert_kmeans_parity(wl, iterations):
    got_cb, got_idx = gpu_kmeans(wl, iterations)
    want_cb, want_idx, counts = K.kmeans(wl.x, wl.codebook, wl.sub_dim, wl.n_centroids,
                                         iterations, dtype=wl.dtype, threads=16, **wl.kwargs())
    want = slots_of(want_cb, wl)
    moved = int(np.sum(want != slots_of(wl.codebook, wl)))
    print(f"[parity] {wl.name} x{iterations}: {moved} codebook elements moved, "
          f"{int(np.sum(counts == 0))} empty clusters at the end", flush=True)
    np.testing.assert_array_equal(got_idx, want_idx)
    np.testing.assert_array_equal(got_cb, want)


CASES = [
    # (seed, n, sd, n_c, iterations, extras)
    (1, 3000, 8, 7, 3, {}),
    (2, 5000, 4, 64, 4, {}),
    (3, 20000, 8, 256, 5, dict(scale=3.0)),
    (4, 9000, 4, 600, 2, {}),                 # global accumulation
    (5, 6000, 8, 2000, 2, dict(dup_frac=0.1)),
    (6, 3000, 8, 5000, 1, {}),                # direct assignment kernel
    (7, 9000, 8, 32, 3, dict(n_codebooks=4, group_len=2048, use_map=True)),
    (8, 7000, 4, 100, 3, dict(n_codebooks=7, group_len=1000, stride_pad=5)),
    (9, 30000, 4, 16, 6, dict(scale=1e-3)),
    # workgroups whose units span several groups (member sums flushed per group)
    (10, 200000, 4, 64, 2, dict(n_codebooks=10, group_len=1000, use_map=True)),
    (11, 150000, 8, 128, 2, dict(n_codebooks=5, group_len=700, use_map=True)),
    # the largest codebook whose sums the encode adds itself, and one more
    (12, 40000, 4, 512, 2, dict(dup_frac=0.02)),
    (13, 40000, 8, 513, 2, {}),
]


@pytest.mark.parametrize("case", CASES, ids=[f"k{c[0]}_n{c[1]}_sd{c[2]}_nc{c[3]}" for c in CASES])
def test_kmeans_matches_oracle(case):
    seed, n, sd, n_c, iters, extra = case
    wl = W.random_case(300 + seed, n, sd, n_c, W.F16, **extra)
    print(f"[case] {wl.name} {extra}", flush=True)
    assert_kmeans_parity(wl, iters)


def test_kmeans_bad_slots_are_left_alone():
    wl = W.random_case(320, 6000, 8, 24, W.F16, n_codebooks=3, group_len=700, use_map=True)
    wl.group_map = np.array([0, 2, -1, 1, 3, 2, 7, 0, 1], np.int32)
    got_cb, got_idx = gpu_kmeans(wl, 2)
    g = np.arange(wl.n) // 700
    assert np.all(got_idx[np.isin(g, [2, 4, 6])] == vq.BAD_SLOT)
    assert_kmeans_parity(wl, 2)


def test_kmeans_exact_clusters():
    pts = np.array([[0, 0, 0, 0], [2, 0, 0, 2], [0, 2, 2, 0], [2, 2, 2, 2],
                    [10, 10, 10, 10], [12, 12, 12, 12],
                    [-8, 4, -8, 4], [-6, 6, -6, 6], [-7, 5, -7, 5]], np.float64)
    init = np.array([[0.5, 0.5, 0.5, 0.5], [10.5, 10, 10, 10], [-7, 4, -7, 4], [100] * 4])
    wl = W.Workload("exact clusters", W.to_f16_bits(pts).reshape(-1, 4),
                    W.to_f16_bits(init).reshape(-1), 4, 4, W.F16, 16, 1, 9)
    got_cb, _ = gpu_kmeans(wl, 3)
    f = got_cb.view(np.float16).astype(np.float64).reshape(4, 4)
    assert f[0].tolist() == [1, 1, 1, 1] and f[1].tolist() == [11] * 4
    assert f[2].tolist() == [-7, 5, -7, 5] and f[3].tolist() == [100] * 4
    assert_kmeans_parity(wl, 3)


def test_kmeans_member_sums_at_the_exactness_limit():
    """Members of +-65504 and 2^-24: per workgroup the encode adds up to 8192
    rows in fp64, whose sums then reach 2^29 at a resolution of 2^-24 (53
    bits), so any lost bit changes a mean."""
    rng = np.random.default_rng(341)
    n = 3 * 2 ** 20
    sign = np.where(rng.random(n) < 0.5, 1.0, -1.0)
    x = np.empty((n, 4))
    x[:, 1:] = sign[:, None] * rng.choice([65504.0, 65472.0, 64000.0], size=(n, 3))
    tiny = rng.random(n) < 0.3
    x[:, 0] = np.where(tiny, sign * 2.0 ** -24, sign * 65504.0)
    x[rng.random(n) < 0.01, 0] = 2.0 ** -14 + 2.0 ** -24   # subnormal and normal mix
    init = np.array([[1000.0] * 4, [-1000.0] * 4, [0.0, 0.0, 0.0, 5.0]])
    wl = W.Workload("exactness limit", W.to_f16_bits(x).reshape(-1, 4),
                    W.to_f16_bits(init).reshape(-1), 4, 3, W.F16, 12, 1, n)
    print(f"[case] {wl.name}: {n} rows", flush=True)
    assert_kmeans_parity(wl, 2)


def test_kmeans_falcon_keys_full_size():
    wl = W.config(3)
    assert_kmeans_parity(wl, 3)


def test_kmeans_full_cache_sampled_slots():
    wl = W.full_cache()
    got_cb, got_idx = gpu_kmeans(wl, 2)
    rng = np.random.default_rng(330)
    for s in [0, 255] + list(rng.choice(np.arange(1, 255), size=4, replace=False)):
        rows = slice(s * wl.group_len, (s + 1) * wl.group_len)
        sub = wl.codebook[s * wl.codebook_stride:(s + 1) * wl.codebook_stride]
        want_cb, want_idx, _ = K.kmeans(wl.x[rows], sub, wl.sub_dim, wl.n_centroids, 2,
                                        threads=16)
        np.testing.assert_array_equal(got_idx[rows], want_idx)
        np.testing.assert_array_equal(got_cb[s], want_cb)
        print(f"[parity] full cache slot {s}: identical", flush=True)


BF16_CASES = [
    # (seed, n, sd, n_c, iterations, extras)
    (21, 3000, 8, 7, 3, {}),
    (22, 5000, 4, 64, 3, dict(scale=1e20)),
    (23, 20000, 8, 256, 3, dict(scale=1e-20)),
    (24, 9000, 4, 600, 2, {}),
    (25, 3000, 8, 5000, 1, {}),                # direct assignment kernel
    (26, 9000, 8, 32, 2, dict(n_codebooks=4, group_len=2048, use_map=True)),
    (27, 40000, 4, 513, 2, dict(dup_frac=0.05)),
]


@pytest.mark.parametrize("case", BF16_CASES,
                         ids=[f"b{c[0]}_n{c[1]}_sd{c[2]}_nc{c[3]}" for c in BF16_CASES])
def test_kmeans_bf16_matches_oracle(case):
    seed, n, sd, n_c, iters, extra = case
    wl = W.random_case(400 + seed, n, sd, n_c, W.BF16, **extra)
    print(f"[case] {wl.name} {extra}", flush=True)
    assert_kmeans_parity(wl, iters)


def test_kmeans_bf16_members_across_the_exponent_range():
    """Clusters whose members span 2^-133 .. 2^127 with both signs: the sums
    fill every limb and carry between them; one cluster's members cancel to
    a subnormal mean, another's sum passes 2^127 before the division."""
    rng = np.random.default_rng(431)
    n = 60000
    mag = np.ldexp(rng.uniform(1.0, 2.0, (n, 8)), rng.integers(-133, 128, (n, 8)))
    x = np.where(rng.random((n, 8)) < 0.5, -mag, mag)
    x[: n // 3, :] = np.ldexp(rng.uniform(1.0, 2.0, (n // 3, 8)), 126)   # fp32 distances overflow
    x[n // 3: n // 3 + 50, 0] = np.ldexp(1.0, -133) * rng.integers(1, 4, 50)
    bits = W.to_bf16_bits(x).reshape(-1, 8)
    bits[rng.random((n, 8)) < 0.001] = 0x7F80                   # +inf components add 0
    init = W.to_bf16_bits(np.ldexp(rng.standard_normal((16, 8)), rng.integers(-100, 100, (16, 8))))
    wl = W.Workload("bf16 exponent range", bits, init.reshape(-1), 8, 16, W.BF16, 128, 1, n)
    print(f"[case] {wl.name}: {n} rows", flush=True)
    assert_kmeans_parity(wl, 3)


def test_kmeans_bf16_large_codebook_subset():
    """2^18 sub-vectors of the large-codebook workload: 4,096 bf16 centroids
    of sub_dim 8 with about 5% exact duplicate rows (duplicates never gain
    members: ties go to the lowest index)."""
    full = W.config(5)
    rows = 1 << 18
    wl = W.Workload(full.name + ", first 2^18 rows", full.x[:rows].copy(), full.codebook,
                    full.sub_dim, full.n_centroids, full.dtype, full.codebook_stride, 1, rows)
    print(f"[case] {wl.name}", flush=True)
    assert_kmeans_parity(wl, 2)
