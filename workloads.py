"""Seeded synthetic inputs for the product-VQ encode step.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the oracle side and the GPU side of every test, the
smoke check and the benchmark take their inputs from here.

Values are drawn in float64 with ``numpy.random.default_rng([config, role])``
(PCG64) and rounded once to the element type: float64 -> float16 with numpy's
round-to-nearest-even, or float64 -> float32 -> bfloat16 with
round-to-nearest-even on the upper 16 bits.  Roles: x = 0, codebook = 1,
per-channel scales = 2, outlier channels = 3, duplicate rows = 4, mixture = 5.

The shapes stand in for the key caches the VeloxQuant-MLX post "I Wrote a
Metal Kernel to Stop My Mac From OOMing" measures (section "The Numbers":
head_dim 128 and 256 caches; the Falcon3-7B trigger shape of section "What
quantize_vq Was Doing Wrong") and for a calibrated codebook, which the pages
do not ship.  Caches are laid out [layers][kv_heads][tokens][head_dim] and cut
into sub-vectors along head_dim, so consecutive sub-vectors share a token.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

F16 = 0
BF16 = 1

ROLE_X, ROLE_CB, ROLE_SCALE, ROLE_OUTLIER, ROLE_DUP, ROLE_GMM = range(6)


@dataclasses.dataclass
class Workload:
    name: str
    x: np.ndarray                # uint16 [n, sub_dim] element bits
    codebook: np.ndarray         # uint16 [n_codebooks * codebook_stride] element bits
    sub_dim: int
    n_centroids: int
    dtype: int                   # F16 or BF16
    codebook_stride: int         # elements between codebook slots
    n_codebooks: int
    group_len: int               # sub-vectors per group (group g uses slot g)
    group_map: Optional[np.ndarray] = None
    meta: dict = dataclasses.field(default_factory=dict)
    # per-channel smoothing factors (fp32 [slots or 1, head_dim]) for the
    # fused encode; None for the plain search
    channel_scale: Optional[np.ndarray] = None
    head_dim: Optional[int] = None

    @property
    def n(self) -> int:
        return self.x.shape[0]

    def kwargs(self) -> dict:
        """Keyword arguments shared by the oracle and the GPU binding."""
        return dict(codebook_stride=self.codebook_stride, n_codebooks=self.n_codebooks,
                    group_len=self.group_len, group_map=self.group_map)

    def packed_kwargs(self) -> dict:
        """Smoothing arguments of the fused encode (oracle side)."""
        sc = self.channel_scale
        return dict(channel_scale=None if sc is None else sc.reshape(-1),
                    head_dim=self.head_dim if self.head_dim else self.sub_dim,
                    scale_stride=0 if sc is None or sc.shape[0] == 1 else sc.shape[1])

    def sha256(self) -> dict:
        return {"x": hashlib.sha256(self.x.tobytes()).hexdigest()[:16],
                "codebook": hashlib.sha256(self.codebook.tobytes()).hexdigest()[:16]}


def _rng(cfg: int, role: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng([cfg, role, *extra])


def to_f16_bits(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bits_to_f32(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Widen element bits to float32 with numpy (for statistics and reports)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _round(a, dtype):
    return to_f16_bits(a) if dtype == F16 else to_bf16_bits(a)


# ---------------------------------------------------------------------------
# The five configurations
# ---------------------------------------------------------------------------

def _scaled_cache_scales(rng_s, rng_o, heads: int, head_dim: int) -> np.ndarray:
    """Per-(head, channel) std: LogNormal(0, 0.5), 4 outlier channels x10."""
    sigma = np.exp(0.5 * rng_s.standard_normal((heads, head_dim)))
    for h in range(heads):
        ch = rng_o.choice(head_dim, size=4, replace=False)
        sigma[h, ch] *= 10.0
    return sigma


def _scaled_cache_codebook(rng, sigma: np.ndarray, sub_dim: int, n_centroids: int) -> np.ndarray:
    """Codebook rows drawn fresh from the cache's own per-channel distribution,
    each at a uniformly random (head, sub-slot) position."""
    heads, head_dim = sigma.shape
    n_sub = head_dim // sub_dim
    h = rng.integers(0, heads, size=n_centroids)
    s = rng.integers(0, n_sub, size=n_centroids)
    cols = s[:, None] * sub_dim + np.arange(sub_dim)[None, :]
    return sigma[h[:, None], cols] * rng.standard_normal((n_centroids, sub_dim))


def tiny(cfg: int = 1) -> Workload:
    """128 tokens x 1 KV head x head_dim 128, sub_dim 8 -> N = 2048; codebook
    [256, 8] = N(0,1) rows plus N(0, 0.01) noise (read as variance 0.01)."""
    sd, n_c = 8, 256
    x = _rng(cfg, ROLE_X).standard_normal((1, 1, 128, 128))
    r = _rng(cfg, ROLE_CB)
    cb = r.standard_normal((n_c, sd)) + 0.1 * r.standard_normal((n_c, sd))
    return Workload("tiny: 128 tok x 1 head x hd128, sd8, n_c256, fp16",
                    to_f16_bits(x).reshape(-1, sd), to_f16_bits(cb).reshape(-1),
                    sd, n_c, F16, n_c * sd, 1, 2048,
                    meta=dict(tokens=128, kv_heads=1, head_dim=128))


def _scaled_cache(cfg: int, name: str, tokens: int, heads: int, head_dim: int,
                  sub_dim: int) -> Workload:
    n_c = 256
    sigma = _scaled_cache_scales(_rng(cfg, ROLE_SCALE), _rng(cfg, ROLE_OUTLIER), heads, head_dim)
    z = _rng(cfg, ROLE_X).standard_normal((heads, tokens, head_dim))
    x = z * sigma[:, None, :]
    cb = _scaled_cache_codebook(_rng(cfg, ROLE_CB), sigma, sub_dim, n_c)
    n = heads * tokens * head_dim // sub_dim
    return Workload(name, to_f16_bits(x).reshape(-1, sub_dim), to_f16_bits(cb).reshape(-1),
                    sub_dim, n_c, F16, n_c * sub_dim, 1, n,
                    meta=dict(tokens=tokens, kv_heads=heads, head_dim=head_dim))


def llama(cfg: int = 2) -> Workload:
    """Llama-3.1-8B-shape keys: 4096 tok x 8 KV heads x hd 128, sub_dim 8."""
    return _scaled_cache(cfg, "llama3.1-8b keys: 4096 tok x 8 heads x hd128, sd8, n_c256, fp16",
                         4096, 8, 128, 8)


def falcon(cfg: int = 3) -> Workload:
    """Falcon3-7B-shape keys: 4096 tok x 4 KV heads x hd 256, sub_dim 4."""
    return _scaled_cache(cfg, "falcon3-7b keys: 4096 tok x 4 heads x hd256, sd4, n_c256, fp16",
                         4096, 4, 256, 4)


def full_cache(cfg: int = 4, layers: int = 32, heads: int = 8, tokens: int = 8192) -> Workload:
    """Whole key cache in one call: 32 layers x 8 KV heads x 8192 tokens x hd 128,
    sub_dim 8; one codebook [256, 8] per (layer, head), slot = layer*heads + head.
    Per-head channel scales and outlier channels are redrawn for every layer."""
    sd, n_c, hd = 8, 256, 128
    n_sub = hd // sd
    group_len = tokens * n_sub
    x = np.empty((layers * heads * tokens * n_sub, sd), dtype=np.uint16)
    cb = np.empty((layers * heads, n_c, sd), dtype=np.uint16)
    rx = _rng(cfg, ROLE_X)
    for l in range(layers):
        sigma = _scaled_cache_scales(_rng(cfg, ROLE_SCALE, l), _rng(cfg, ROLE_OUTLIER, l), heads, hd)
        z = rx.standard_normal((heads, tokens, hd))
        lo = l * heads * group_len
        x[lo: lo + heads * group_len] = to_f16_bits(z * sigma[:, None, :]).reshape(-1, sd)
        for h in range(heads):
            rc = _rng(cfg, ROLE_CB, l, h)
            cb[l * heads + h] = to_f16_bits(_scaled_cache_codebook(rc, sigma[h:h + 1], sd, n_c))
    return Workload(f"full cache: {layers} layers x {heads} heads x {tokens} tok x hd128, sd8, "
                    f"n_c256 per (layer, head), fp16",
                    x, cb.reshape(-1), sd, n_c, F16, n_c * sd, layers * heads, group_len,
                    meta=dict(layers=layers, kv_heads=heads, tokens=tokens, head_dim=hd))


def large_codebook(cfg: int = 5, n: int = 1 << 20) -> Workload:
    """N = 2^20 sub-vectors (sub_dim 8, bf16) from a 64-component Gaussian
    mixture (means ~ N(0, I), std 0.1); codebook [4096, 8] bf16 from the same
    mixture with round(0.05 * 4096) = 205 rows overwritten by exact copies of
    other rows, so exact ties must resolve to the lowest index."""
    sd, n_c, k = 8, 4096, 64
    means = _rng(cfg, ROLE_GMM).standard_normal((k, sd))
    rx = _rng(cfg, ROLE_X)
    comp = rx.integers(0, k, size=n)
    x = means[comp] + 0.1 * rx.standard_normal((n, sd))
    rc = _rng(cfg, ROLE_CB)
    comp_c = rc.integers(0, k, size=n_c)
    cb = to_bf16_bits(means[comp_c] + 0.1 * rc.standard_normal((n_c, sd)))
    rd = _rng(cfg, ROLE_DUP)
    n_dup = int(round(0.05 * n_c))
    dst = rd.choice(n_c, size=n_dup, replace=False)
    keep = np.setdiff1d(np.arange(n_c), dst)
    src = keep[rd.integers(0, keep.size, size=n_dup)]
    cb[dst] = cb[src]
    return Workload("large codebook: 2^20 x sd8 bf16 GMM(64, 0.1), n_c4096 with 205 duplicate rows",
                    to_bf16_bits(x).reshape(-1, sd), cb.reshape(-1), sd, n_c, BF16, n_c * sd, 1, n,
                    meta=dict(components=k, duplicates=n_dup, dup_dst=dst, dup_src=src))


CONFIGS = {1: tiny, 2: llama, 3: falcon, 4: full_cache, 5: large_codebook}


# ---------------------------------------------------------------------------
# Smoothed caches for the fused encode (factors + packed codes)
# ---------------------------------------------------------------------------
#
# The pages give no calibrated smooth factors.  Stand-in recipe: the factor of
# a channel is 1 / sqrt(s) with s the largest per-head std of that channel
# (the square-root balance of activation smoothing), rounded to fp32; the
# codebook is drawn from the smoothed keys' own distribution (std sigma * f),
# as a calibration on smoothed keys would produce.

def _factors(sigma: np.ndarray) -> np.ndarray:
    return (1.0 / np.sqrt(sigma.max(axis=0))).astype(np.float32)


def falcon_smoothed(cfg: int = 3) -> Workload:
    """The Falcon3-7B-shape keys of config 3 with per-channel smoothing
    factors [256] (one codebook slot shared by the 4 KV heads)."""
    tokens, heads, hd, sd, n_c = 4096, 4, 256, 4, 256
    sigma = _scaled_cache_scales(_rng(cfg, ROLE_SCALE), _rng(cfg, ROLE_OUTLIER), heads, hd)
    z = _rng(cfg, ROLE_X).standard_normal((heads, tokens, hd))
    x = z * sigma[:, None, :]
    f = _factors(sigma)
    cb = _scaled_cache_codebook(_rng(cfg, ROLE_CB, 1), sigma * f[None, :], sd, n_c)
    n = heads * tokens * hd // sd
    return Workload("falcon3-7b keys, smoothed: 4096 tok x 4 heads x hd256, sd4, n_c256, fp16",
                    to_f16_bits(x).reshape(-1, sd), to_f16_bits(cb).reshape(-1), sd, n_c, F16,
                    n_c * sd, 1, n, meta=dict(tokens=tokens, kv_heads=heads, head_dim=hd),
                    channel_scale=f[None, :], head_dim=hd)


def full_cache_smoothed(cfg: int = 4, layers: int = 32, heads: int = 8,
                        tokens: int = 8192) -> Workload:
    """Config 4's whole key cache with one smoothing vector and one codebook per
    (layer, head): factor = 1 / sqrt(that head's channel std)."""
    base = full_cache(cfg, layers, heads, tokens)
    sd, n_c, hd = 8, 256, 128
    scale = np.empty((layers * heads, hd), dtype=np.float32)
    cb = np.empty((layers * heads, n_c, sd), dtype=np.uint16)
    for l in range(layers):
        sigma = _scaled_cache_scales(_rng(cfg, ROLE_SCALE, l), _rng(cfg, ROLE_OUTLIER, l), heads, hd)
        for h in range(heads):
            f = (1.0 / np.sqrt(sigma[h])).astype(np.float32)
            scale[l * heads + h] = f
            rc = _rng(cfg, ROLE_CB, l, h, 1)
            cb[l * heads + h] = to_f16_bits(_scaled_cache_codebook(rc, (sigma[h] * f)[None, :],
                                                                   sd, n_c))
    base.name = base.name.replace("full cache:", "full cache, smoothed:")
    base.codebook = cb.reshape(-1)
    base.channel_scale = scale
    base.head_dim = hd
    return base


def config(i: int) -> Workload:
    return CONFIGS[i]()


# ---------------------------------------------------------------------------
# Small random cases for parity sweeps
# ---------------------------------------------------------------------------

def random_case(seed: int, n: int, sub_dim: int, n_centroids: int, dtype: int = F16, *,
                n_codebooks: int = 1, group_len: Optional[int] = None, use_map: bool = False,
                scale: float = 1.0, dup_frac: float = 0.0, stride_pad: int = 0) -> Workload:
    """Gaussian sub-vectors and codebooks of any shape, optionally with exact
    duplicate codebook rows, several codebook slots, padded slot stride and a
    shuffled group -> slot map."""
    r = np.random.default_rng([1000, seed])
    x = _round(scale * r.standard_normal((n, sub_dim)), dtype).reshape(n, sub_dim)
    stride = n_centroids * sub_dim + stride_pad
    cb = np.zeros(n_codebooks * stride, dtype=np.uint16)
    for s in range(n_codebooks):
        rows = _round(scale * r.standard_normal((n_centroids, sub_dim)), dtype)
        if dup_frac > 0 and n_centroids > 1:
            k = max(1, int(dup_frac * n_centroids))
            dst = r.choice(n_centroids, size=k, replace=False)
            src = r.integers(0, n_centroids, size=k)
            rows[dst] = rows[src]
        cb[s * stride: s * stride + n_centroids * sub_dim] = rows.reshape(-1)
    if group_len is None:
        group_len = max(n, 1)
    n_groups = max(1, -(-n // group_len))
    gmap = None
    if use_map:
        gmap = r.integers(0, n_codebooks, size=n_groups).astype(np.int32)
    elif n_groups > n_codebooks:
        raise ValueError("identity group mapping needs one codebook slot per group")
    return Workload(f"random(seed={seed}, n={n}, sd={sub_dim}, n_c={n_centroids})", x, cb,
                    sub_dim, n_centroids, dtype, stride, n_codebooks, group_len, gmap)


# ---------------------------------------------------------------------------
# Decode attention over VQ-coded caches
# ---------------------------------------------------------------------------
#
# The pages ship no calibrated codebooks or caches, so the coded cache is
# synthetic: key and value codes are drawn directly (uniform over the
# codebook, or from a skewed law), key codebooks from the smoothed per-channel
# law of the key generator above, value codebooks N(0, 1), queries N(0, 1)
# scaled per channel by 1/f so that q~ = q / f stays O(1).  Roles: queries 6,
# key codes 7, value codes 8, lengths 9 (after the encode roles 0-5).

ROLE_Q, ROLE_KCODE, ROLE_VCODE, ROLE_LEN = 6, 7, 8, 9


@dataclasses.dataclass
class AttnWorkload:
    name: str
    q: np.ndarray            # element bits [B, Hq, D]
    k_codes: np.ndarray      # uint8 [B, Hkv, S, D / k_sub_dim]
    v_codes: np.ndarray      # uint8 [B, Hkv, S, D / v_sub_dim]
    k_codebook: np.ndarray   # element bits [Hkv, n_c, k_sub_dim]
    v_codebook: np.ndarray   # element bits [Hkv, n_c, v_sub_dim]
    k_scale: Optional[np.ndarray]   # float32 [Hkv, D] or None
    kv_len: np.ndarray       # int32 [B]
    dtype: int
    window: int = 0
    softmax_scale: Optional[float] = None

    @property
    def shape(self):
        B, Hq, D = self.q.shape
        return B, Hq, self.k_codes.shape[1], D, self.k_codes.shape[2]

    def kwargs(self) -> dict:
        return dict(k_scale=self.k_scale, kv_len=self.kv_len, window=self.window,
                    softmax_scale=self.softmax_scale)


def attention_case(seed: int, B: int, Hq: int, Hkv: int, D: int, S: int, k_sub_dim: int,
                   v_sub_dim: int, n_c: int = 256, dtype: int = F16, *, smooth: bool = True,
                   lens: str = "full", window: int = 0, skew: float = 0.0,
                   cfg: int = 2000) -> AttnWorkload:
    """A seeded coded cache.  lens: "full" (every sequence S long), "mixed"
    (uniform in [1, S]) or "ragged" (mixed plus some empty and some length-1
    sequences).  skew > 0 draws codes from a Zipf-like law (index c with
    weight (c + 1)^-skew) instead of uniformly."""
    rq = np.random.default_rng([cfg, ROLE_Q, seed])
    sigma = _scaled_cache_scales(_rng(cfg, ROLE_SCALE, seed), _rng(cfg, ROLE_OUTLIER, seed), Hkv, D)
    if smooth:
        f = (1.0 / np.sqrt(sigma)).astype(np.float32)
    else:
        f = np.ones((Hkv, D), dtype=np.float32)
    kcb = np.empty((Hkv, n_c, k_sub_dim))
    rc = _rng(cfg, ROLE_CB, seed)
    for h in range(Hkv):
        kcb[h] = _scaled_cache_codebook(rc, (sigma[h] * f[h])[None, :], k_sub_dim, n_c)
    vcb = rc.standard_normal((Hkv, n_c, v_sub_dim))
    g = Hq // Hkv
    qv = rq.standard_normal((B, Hq, D)) / np.repeat(f, g, axis=0)[None, :, :]

    def codes(role, sub_dim):
        r = np.random.default_rng([cfg, role, seed])
        shape = (B, Hkv, S, D // sub_dim)
        if skew > 0:
            w = (np.arange(n_c) + 1.0) ** -skew
            return r.choice(n_c, size=shape, p=w / w.sum()).astype(np.uint8)
        return r.integers(0, n_c, size=shape, dtype=np.int64).astype(np.uint8)

    rl = np.random.default_rng([cfg, ROLE_LEN, seed])
    if lens == "full":
        kv_len = np.full(B, S, dtype=np.int32)
    else:
        kv_len = rl.integers(1, S + 1, size=B).astype(np.int32)
        if lens == "ragged" and B >= 3:
            kv_len[0] = 0
            kv_len[1] = 1
            kv_len[2] = S
    rnd = to_f16_bits if dtype == F16 else to_bf16_bits
    return AttnWorkload(f"attention(seed={seed}, B={B}, Hq={Hq}, Hkv={Hkv}, D={D}, S={S}, "
                        f"sd={k_sub_dim}/{v_sub_dim}, n_c={n_c}, lens={lens}, window={window})",
                        rnd(qv).reshape(B, Hq, D), codes(ROLE_KCODE, k_sub_dim),
                        codes(ROLE_VCODE, v_sub_dim),
                        rnd(kcb).reshape(Hkv, n_c, k_sub_dim), rnd(vcb).reshape(Hkv, n_c, v_sub_dim),
                        f if smooth else None, kv_len, dtype, window)


def falcon_decode_attention(B: int = 32, S: int = 4096) -> AttnWorkload:
    """Falcon3-7B decode step over a VQ-coded cache: 12 query heads sharing 4
    KV heads (groups of 3), head_dim 256, keys and values in 8-bit codes of
    sub_dim 4 (the post's VecInfer config), smoothed keys, B sequences whose
    lengths are uniform in [S/2, S]."""
    wl = attention_case(1, B, 12, 4, 256, S, 4, 4, 256, F16, smooth=True, lens="full",
                        cfg=2001)
    rl = np.random.default_rng([2001, ROLE_LEN, 1])
    wl.kv_len = rl.integers(S // 2, S + 1, size=B).astype(np.int32)
    wl.name = (f"falcon3-7b decode attention: {B} seqs x 12 q heads / 4 kv heads, hd256, "
               f"kv len U[{S // 2}, {S}], 8-bit codes sd4/sd4, smoothed keys, fp16")
    return wl
