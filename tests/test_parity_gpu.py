"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Small seeded cases span several tiles (1024 sub-vectors per workgroup) and
LDS chunks (1024 centroids), with ragged tails, groups that do not align with
tiles, padded slot strides, group maps with invalid slots, duplicate rows,
non-finite values and the largest codebook the ABI allows.  The five full-size
workloads run in the launch configuration the benchmark times and the
oracle (threaded over the host cores) checks every row of each, the full
cache's 33,554,432 included.  Acceptance rule: see tests/parity.py.
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

DEV = torch.device("cuda:0")


def to_dev(wl):
    tdt = torch.float16 if wl.dtype == W.F16 else torch.bfloat16
    x = torch.from_numpy(wl.x.view(np.int16)).view(tdt).to(DEV)
    cb = torch.from_numpy(wl.codebook.view(np.int16)).view(tdt).to(DEV)
    stride = wl.codebook_stride
    need = wl.n_codebooks * stride
    if cb.numel() < need:   # the last slot may be stored without its padding
        cb = torch.cat([cb, torch.zeros(need - cb.numel(), dtype=tdt, device=DEV)])
    cb3 = cb[:need].view(wl.n_codebooks, stride)[:, : wl.n_centroids * wl.sub_dim]
    cb3 = cb3.view(wl.n_codebooks, wl.n_centroids, wl.sub_dim)
    gmap = None if wl.group_map is None else torch.from_numpy(wl.group_map).to(DEV)
    return x, cb3, gmap


def gpu_encode(wl):
    x, cb3, gmap = to_dev(wl)
    cb = cb3[0] if wl.n_codebooks == 1 else cb3
    out = vq.encode(x, cb, group_len=wl.group_len, group_map=gmap)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint32)


def assert_parity(wl, got, rows=None):
    rep = parity.compare(wl, got, rows)
    print(f"[parity] {wl.name}: {rep.summary()}", flush=True)
    assert rep.ok, rep.summary()
    return rep


SMALL = [
    # (seed, n, sd, n_c, dtype, extra)
    (1, 1, 8, 256, W.F16, {}),
    (2, 255, 4, 256, W.F16, {}),
    (3, 1024, 8, 256, W.F16, {}),
    (4, 1025, 4, 256, W.BF16, {}),
    (5, 5000, 8, 7, W.F16, {}),
    (6, 3333, 4, 1, W.F16, {}),
    (7, 4099, 8, 9, W.BF16, {}),
    (8, 2500, 8, 1023, W.F16, {}),
    (9, 2500, 4, 1024, W.BF16, {}),
    (10, 2500, 8, 1025, W.F16, {}),
    (11, 3000, 8, 4096, W.BF16, dict(dup_frac=0.05)),
    (12, 7000, 4, 300, W.F16, dict(n_codebooks=7, group_len=1000, stride_pad=5)),
    (13, 7000, 8, 64, W.BF16, dict(n_codebooks=3, group_len=3, use_map=True)),
    (14, 9000, 8, 256, W.F16, dict(n_codebooks=4, group_len=2048, use_map=True, stride_pad=8)),
    (15, 20000, 4, 256, W.F16, dict(dup_frac=0.2, scale=10.0)),
    (16, 1500, 8, 256, W.F16, dict(scale=1e-3)),
    (17, 1500, 4, 2, W.F16, {}),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"s{c[0]}_n{c[1]}_sd{c[2]}_nc{c[3]}" for c in SMALL])
def test_small_cases_match_oracle(case):
    seed, n, sd, n_c, dt, extra = case
    wl = W.random_case(seed, n, sd, n_c, dt, **extra)
    print(f"[case] {wl.name} {extra}", flush=True)
    got = gpu_encode(wl)
    rep = assert_parity(wl, got)
    assert rep.equal == rep.rows, "the encode is exact: every index must equal the oracle's"


# Inputs large enough that one workgroup (one per CU) owns several units of
# several groups: the units of a segment are taken from a counter in LDS by
# whichever wave is free, and the codebook slot is restaged per segment.
# Group lengths that are not a multiple of the unit (32 T rows) leave partly
# filled units at every group end; a map sends several groups to one slot,
# some to bad slots.  Above 256 centroids the work goes out in half units
# (2-column pieces for the youngest wave of each SIMD, whole units for the
# others, from one piece counter that starts past the 28 pieces handed out
# at the start): cases 54 and 55 give each workgroup 38 and 44 pieces, so
# pieces also come from the counter, and a whole unit can start on a
# segment's last piece and must stop at the segment's end.
MULTI = [
    # (seed, n, sd, n_c, dtype, extra)
    (50, 200_000, 4, 256, W.F16, dict(n_codebooks=70, group_len=3000)),
    (51, 150_000, 8, 256, W.BF16, dict(n_codebooks=9, group_len=700, use_map=True)),
    (52, 120_000, 4, 100, W.F16, dict(n_codebooks=5, group_len=129, use_map=True, stride_pad=3)),
    (53, 100_000, 8, 2000, W.F16, dict(n_codebooks=3, group_len=9000, use_map=True)),
    (54, 600_000, 4, 300, W.F16, dict(n_codebooks=6, group_len=3000, use_map=True)),
    (55, 700_000, 8, 1100, W.BF16, dict(n_codebooks=4, group_len=4000, use_map=True, dup_frac=0.02)),
]


@pytest.mark.parametrize("case", MULTI, ids=[f"m{c[0]}_n{c[1]}_sd{c[2]}_nc{c[3]}" for c in MULTI])
def test_multi_segment_workgroups_match_oracle(case):
    seed, n, sd, n_c, dt, extra = case
    wl = W.random_case(seed, n, sd, n_c, dt, **extra)
    if wl.group_map is not None:
        wl.group_map[::7] = -1          # bad slots: sentinel codes
        wl.group_map[3::11] = wl.n_codebooks
    print(f"[case] {wl.name} {extra}", flush=True)
    got = gpu_encode(wl)
    rep = assert_parity(wl, got)
    assert rep.equal == rep.rows, "the encode is exact: every index must equal the oracle's"


def test_max_centroids():
    wl = W.random_case(30, 2100, 8, 65536, W.BF16, dup_frac=0.01)
    print(f"[case] {wl.name}", flush=True)
    assert_parity(wl, gpu_encode(wl))


def test_bad_slots_give_sentinel():
    wl = W.random_case(31, 5000, 8, 32, W.F16, n_codebooks=3, group_len=700, use_map=True)
    wl.group_map = np.array([0, 2, -1, 1, 3, 2, 7, 0], np.int32)
    got = gpu_encode(wl)
    g = np.arange(wl.n) // wl.group_len
    bad = np.isin(g, [2, 4, 6])
    assert np.all(got[bad] == vq.BAD_SLOT)
    assert_parity(wl, got)


def test_exact_ties_on_a_coarse_grid():
    r = np.random.default_rng(32)
    for sd, dt in ((4, W.F16), (8, W.BF16)):
        kx = 64 * r.integers(-2, 3, size=(6000, sd))
        kc = 64 * r.integers(-2, 3, size=(200, sd))
        bits = W.to_f16_bits if dt == W.F16 else W.to_bf16_bits
        wl = W.Workload("grid ties", bits(kx / 64.0).reshape(-1, sd), bits(kc / 64.0).reshape(-1),
                        sd, 200, dt, 200 * sd, 1, 6000)
        rep = assert_parity(wl, gpu_encode(wl))
        assert rep.equal == rep.rows


def test_non_finite_values():
    sd, n_c = 8, 40
    r = np.random.default_rng(33)
    x = r.standard_normal((3000, sd))
    x[::7, 3] = np.nan
    x[::11, 0] = np.inf
    x[::13, 5] = -np.inf
    c = r.standard_normal((n_c, sd))
    c[0, 2] = np.nan
    c[5, 1] = np.inf
    c[9, :] = np.inf
    for dt, bits in ((W.F16, W.to_f16_bits), (W.BF16, W.to_bf16_bits)):
        wl = W.Workload("non-finite", bits(x).reshape(-1, sd), bits(c).reshape(-1), sd, n_c, dt,
                        n_c * sd, 1, 3000)
        rep = assert_parity(wl, gpu_encode(wl))
        assert rep.equal == rep.rows


@pytest.mark.parametrize("n_c", [41, 40])
def test_non_finite_values_odd_codebook(n_c):
    # non-finite x takes the full exact scan, split over a lane pair: an odd
    # number of centroids gives the two lanes different halves
    sd = 4
    r = np.random.default_rng(37)
    x = r.standard_normal((5000, sd))
    x[::5, 1] = np.nan
    x[::9, 2] = np.inf
    c = r.standard_normal((n_c, sd))
    wl = W.Workload("non-finite x, odd n_c", W.to_f16_bits(x).reshape(-1, sd),
                    W.to_f16_bits(c).reshape(-1), sd, n_c, W.F16, n_c * sd, 1, 5000)
    rep = assert_parity(wl, gpu_encode(wl))
    assert rep.equal == rep.rows


@pytest.mark.parametrize("sd,dt,n_c", [(4, W.F16, 512), (8, W.BF16, 512), (4, W.F16, 256),
                                        (8, W.BF16, 256), (4, W.BF16, 200), (8, W.F16, 200)])
def test_near_tied_centroids_across_groups(sd, dt, n_c):
    # centroids in pairs one or two ulps apart, placed in different groups
    # (16 rows; 8 rows, with the group index kept in the bound, at 256
    # centroids or fewer, 200 with a padded last block), and sub-vectors
    # sitting between them: most columns are ambiguous after the
    # matrix-core stage and must be resolved exactly
    r = np.random.default_rng(38 + sd + n_c)
    base = r.standard_normal((n_c // 2, sd))
    bits = W.to_f16_bits if dt == W.F16 else W.to_bf16_bits
    a = bits(base).reshape(-1, sd)
    b = a.copy()
    b[:, 0] = b[:, 0] + r.integers(1, 3, size=b.shape[0]).astype(np.uint16)   # +1..2 ulp
    cb = np.empty((n_c, sd), np.uint16)
    perm = r.permutation(n_c)
    cb[perm[: n_c // 2]] = a
    cb[perm[n_c // 2:]] = b
    xf = W.bits_to_f32(a, dt).astype(np.float64)
    pick = r.integers(0, n_c // 2, size=20000)
    x = xf[pick] + 1e-3 * r.standard_normal((20000, sd))
    wl = W.Workload("near-tied pairs", bits(x).reshape(-1, sd), cb.reshape(-1), sd, n_c, dt,
                    n_c * sd, 1, 20000)
    rep = assert_parity(wl, gpu_encode(wl))
    assert rep.equal == rep.rows


@pytest.mark.parametrize("sd,dt,scale", [(4, W.F16, 1.0), (8, W.BF16, 1.0), (4, W.F16, 300.0),
                                         (8, W.F16, 1.0)])
def test_whole_groups_of_duplicate_rows(sd, dt, scale):
    """A codebook whose rows 8.. repeat rows 0..7: every group but the first
    holds only rows that can never win (marked at staging), so their bounds
    are infinite before the group index is written into them; the 8-row
    groups of small codebooks must keep such bounds finite and out of the
    way.  scale 300 makes an fp16 slot take the unfolded form."""
    r = np.random.default_rng(45 + sd)
    n_c = 256
    bits = W.to_f16_bits if dt == W.F16 else W.to_bf16_bits
    head = bits(scale * r.standard_normal((8, sd))).reshape(-1, sd)
    cb = np.tile(head, (n_c // 8, 1))
    xf = W.bits_to_f32(head, dt).astype(np.float64)
    x = xf[r.integers(0, 8, size=12000)] + 0.3 * scale * r.standard_normal((12000, sd))
    wl = W.Workload("whole duplicate groups", bits(x).reshape(-1, sd), cb.reshape(-1), sd, n_c,
                    dt, n_c * sd, 1, 12000)
    print(f"[case] {wl.name} sd {sd} scale {scale}", flush=True)
    got = gpu_encode(wl)
    rep = assert_parity(wl, got)
    assert rep.equal == rep.rows
    assert int(got.max()) < 8, "a repeated row can never be the first minimum"


@pytest.mark.parametrize("sd,scale,dups", [(4, 300.0, 0.0), (4, 150.0, 0.0), (8, 300.0, 0.0),
                                           (4, 300.0, 0.2)])
def test_codebook_norms_beyond_fp16_c(sd, scale, dups):
    """fp16 centroids with |c|^2 / 2 above the fp16 range (|c| > 362): such a
    slot cannot carry C in the product's spare slots and takes the unfolded
    form; every centroid must still be bounded (none may drop out), and
    duplicate rows in such a slot are excluded through C alone."""
    wl = W.random_case(41, 20000, sd, 256, W.F16, scale=scale, dup_frac=dups)
    print(f"[case] {wl.name} scale {scale} duplicates {dups}", flush=True)
    got = gpu_encode(wl)
    rep = assert_parity(wl, got)
    assert rep.equal == rep.rows, "the encode is exact: every index must equal the oracle's"


def test_huge_codebook_norms_odd_bf16():
    sd, n_c = 8, 33
    r = np.random.default_rng(39)
    x = 1e25 * r.standard_normal((3000, sd))
    c = 1e25 * r.standard_normal((n_c, sd))
    wl = W.Workload("huge norms", W.to_bf16_bits(x).reshape(-1, sd), W.to_bf16_bits(c).reshape(-1),
                    sd, n_c, W.BF16, n_c * sd, 1, 3000)
    rep = assert_parity(wl, gpu_encode(wl))
    assert rep.equal == rep.rows


def test_overflowing_and_subnormal_distances_bf16():
    sd, n_c = 4, 16
    r = np.random.default_rng(34)
    x = np.concatenate([1e37 * r.standard_normal((500, sd)), 1e-20 * r.standard_normal((500, sd))])
    c = np.concatenate([1e37 * r.standard_normal((8, sd)), 1e-20 * r.standard_normal((8, sd))])
    wl = W.Workload("extremes", W.to_bf16_bits(x).reshape(-1, sd), W.to_bf16_bits(c).reshape(-1),
                    sd, n_c, W.BF16, n_c * sd, 1, 1000)
    rep = assert_parity(wl, gpu_encode(wl))
    assert rep.equal == rep.rows


def test_decode_matches_oracle_gather():
    wl = W.random_case(35, 9000, 8, 100, W.BF16, n_codebooks=3, group_len=3500, stride_pad=4)
    x, cb3, gmap = to_dev(wl)
    idx = vq.encode(x, cb3, group_len=wl.group_len)
    idx_np = idx.cpu().numpy().view(np.uint32).copy()
    idx_np[::97] = 100            # out of range -> zero row
    idx_np[5] = 0xFFFFFFFF
    idx_t = torch.from_numpy(idx_np.view(np.int32)).to(DEV).view(torch.uint32)
    rec = vq.decode(idx_t, cb3, group_len=wl.group_len)
    torch.cuda.synchronize()
    want = oracle.decode(idx_np, wl.codebook, 8, 100, wl.dtype, **wl.kwargs())
    assert np.array_equal(rec.cpu().view(torch.int16).numpy().view(np.uint16), want)


def test_empty_input_launches_nothing():
    x = torch.empty(0, 8, dtype=torch.float16, device=DEV)
    cb = torch.zeros(256, 8, dtype=torch.float16, device=DEV)
    out = vq.encode(x, cb)
    assert out.numel() == 0


def test_misaligned_x_raises():
    x = torch.zeros(1025 * 8, dtype=torch.float16, device=DEV)[4:4 + 1024 * 8]
    cb = torch.zeros(256, 8, dtype=torch.float16, device=DEV)
    with pytest.raises(vq.VQError, match="MISALIGNED"):
        vq.encode(x, cb)


def test_side_streams_and_host_threads():
    """Encodes on two side streams, and from two host threads at once (each
    with its own stream), match the oracle: every launch runs on the stream
    it is given, and the launch path keeps no state that calls share."""
    import threading
    cases = [W.random_case(37, 70000, 4, 256, W.F16), W.random_case(38, 50000, 8, 100, W.BF16),
             W.random_case(39, 30000, 8, 256, W.F16, n_codebooks=3, group_len=10000)]
    devs = [to_dev(wl) for wl in cases]
    want = [oracle.encode(wl.x, wl.codebook, wl.sub_dim, wl.n_centroids, wl.dtype, threads=8,
                          **wl.kwargs()) for wl in cases]
    streams = [torch.cuda.Stream(device=DEV) for _ in cases]   # default priority
    torch.cuda.synchronize()

    def run(k, outs):
        wl, (x, cb3, gmap) = cases[k], devs[k]
        cb = cb3[0] if wl.n_codebooks == 1 else cb3
        with torch.cuda.stream(streams[k]):
            outs[k] = vq.encode(x, cb, group_len=wl.group_len, group_map=gmap,
                                stream=streams[k])

    outs = [None] * len(cases)
    for k in range(len(cases)):          # back to back, no synchronization between
        run(k, outs)
    torch.cuda.synchronize()
    for k in range(len(cases)):
        assert np.array_equal(outs[k].cpu().numpy().view(np.uint32), want[k]), k
    outs = [None] * len(cases)
    threads = [threading.Thread(target=run, args=(k, outs)) for k in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for k in range(len(cases)):
        assert np.array_equal(outs[k].cpu().numpy().view(np.uint32), want[k]), k


def test_no_device_memory_is_allocated():
    wl = W.random_case(36, 50000, 4, 256, W.F16)
    x, cb3, _ = to_dev(wl)
    out = torch.empty(wl.n, dtype=torch.uint32, device=DEV)
    vq.encode(x, cb3[0], out=out)          # first launch loads the code object
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        vq.encode(x, cb3[0], out=out)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0


# ---------------------------------------------------------------------------
# full-size workloads
# ---------------------------------------------------------------------------

def test_more_than_2_31_sub_vectors_sampled():
    """2^31 + 4099 sub-vectors (17 GB of keys): row offsets, unit indices and
    byte addresses pass 2^31.  Keys are drawn on the device from a seeded
    generator; sampled rows (random, around 2^31 and the ragged tail) are
    copied back and checked against the oracle on the same values."""
    n = 2 ** 31 + 4099
    sd = 4
    cbw = W.random_case(44, 1, sd, 256, W.F16)
    x = torch.empty(n, sd, dtype=torch.float16, device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(44)
    step = 2 ** 28
    for i in range(0, n, step):
        j = min(n, i + step)
        x[i:j] = torch.randn(j - i, sd, generator=gen, device=DEV).to(torch.float16)
    cb = torch.from_numpy(cbw.codebook.view(np.int16)).view(torch.float16).to(DEV).view(256, sd)
    out = vq.encode(x, cb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(44)
    rows = np.unique(np.concatenate([
        rng.integers(0, n, 1 << 16), np.arange(2 ** 31 - 300, 2 ** 31 + 300),
        np.arange(n - 5000, n), np.arange(0, 300)]))
    idx = torch.from_numpy(rows).to(DEV)
    xs = x[idx].cpu().view(torch.int16).numpy().view(np.uint16)
    got = out.view(torch.int32)[idx].cpu().numpy().view(np.uint32)
    del x, out
    torch.cuda.empty_cache()
    want = oracle.encode(xs, cbw.codebook, sd, 256, W.F16, threads=8)
    print(f"[parity] {n} sub-vectors, {rows.size} sampled rows: "
          f"{int(np.sum(got == want))} equal", flush=True)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_full_size_config_every_row(cfg):
    wl = W.config(cfg)
    print(f"[config {cfg}] {wl.name} n={wl.n}", flush=True)
    got = gpu_encode(wl)
    ref = parity.oracle_indices(wl)
    rep = parity.compare(wl, got, ref_idx=ref)
    print(f"[parity] {wl.name}: {rep.summary()}", flush=True)
    assert rep.ok, rep.summary()
    # the pages' own criterion: reconstruction MSE of both index sets
    xf = W.bits_to_f32(wl.x, wl.dtype).astype(np.float64)
    cbf = W.bits_to_f32(wl.codebook, wl.dtype).astype(np.float64).reshape(-1, wl.sub_dim)
    mse_gpu = np.mean((xf - cbf[got]) ** 2)
    mse_ref = np.mean((xf - cbf[ref]) ** 2)
    print(f"[config {cfg}] mse gpu={mse_gpu:.6e} oracle={mse_ref:.6e} "
          f"equal rows {rep.equal}/{rep.rows}", flush=True)
    assert abs(mse_gpu - mse_ref) <= 1e-6 * mse_ref


def test_full_cache_every_row():
    """The full batched cache (33,554,432 sub-vectors, 256 codebook slots):
    every row against the oracle, threaded over the host cores."""
    wl = W.config(4)
    print(f"[config 4] {wl.name} n={wl.n}", flush=True)
    got = gpu_encode(wl)
    ref = parity.oracle_indices(wl)
    rep = parity.compare(wl, got, ref_idx=ref)
    print(f"[parity] {wl.name}: {rep.summary()}", flush=True)
    assert rep.ok, rep.summary()
    assert rep.rows == wl.n == 33554432
