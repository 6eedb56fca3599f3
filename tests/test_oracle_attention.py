"""Pins of the decode-attention oracle (oracle/attention.py), CPU only.

Against what:
  * torch's float64 ``scaled_dot_product_attention`` (an independent
    implementation) on the dequantized, unsmoothed cache, heads expanded for
    grouped-query attention;
  * closed forms: one attended token returns its value row exactly; equal
    keys (or a zero query) give the mean of the value rows; an empty
    sequence gives zeros;
  * the lookup-table identity the kernels use: scores summed from
    LUT[s, c] = (q / f)_s . C_k[c] equal the dense scores;
  * brute force of the grouped-query head mapping and of the window;
  * planted mistakes in copies of the oracle must fail these pins.
"""
import os
import types

import numpy as np
import pytest

import workloads as W
from oracle import attention as A

torch = pytest.importorskip("torch")


def run(wl, mod=A):
    return mod.decode_attention(wl.q, wl.k_codes, wl.v_codes, wl.k_codebook, wl.v_codebook,
                                wl.dtype, **wl.kwargs())


def torch_reference(wl):
    """float64 SDPA per (b, kv head) on the dequantized cache."""
    B, Hq, Hkv, D, S = wl.shape
    g = Hq // Hkv
    scale = wl.softmax_scale if wl.softmax_scale is not None else 1.0 / np.sqrt(D)
    out = np.zeros((B, Hq, D))
    kcb = A.widen(wl.k_codebook, wl.dtype)
    vcb = A.widen(wl.v_codebook, wl.dtype)
    q = A.widen(wl.q, wl.dtype)
    for b in range(B):
        L = int(wl.kv_len[b])
        t0 = max(0, L - wl.window) if wl.window else 0
        if L <= t0:
            continue
        for h in range(Hkv):
            K = kcb[h][wl.k_codes[b, h, t0:L].astype(np.int64)].reshape(L - t0, D)
            if wl.k_scale is not None:
                K = K / wl.k_scale[h].astype(np.float64)
            V = vcb[h][wl.v_codes[b, h, t0:L].astype(np.int64)].reshape(L - t0, D)
            qs = torch.from_numpy(q[b, h * g:(h + 1) * g])[None, :, None, :]   # [1, g, 1, D]
            Kt = torch.from_numpy(K)[None, None].expand(1, g, L - t0, D)
            Vt = torch.from_numpy(V)[None, None].expand(1, g, L - t0, D)
            o = torch.nn.functional.scaled_dot_product_attention(qs, Kt, Vt, scale=scale)
            out[b, h * g:(h + 1) * g] = o[0, :, 0].numpy()
    return out


CASES = [
    dict(seed=1, B=3, Hq=6, Hkv=2, D=32, S=50, k_sub_dim=4, v_sub_dim=8, n_c=64, lens="ragged"),
    dict(seed=2, B=2, Hq=4, Hkv=4, D=64, S=129, k_sub_dim=8, v_sub_dim=4, n_c=256, lens="mixed",
         dtype=W.BF16, smooth=False),
    dict(seed=3, B=2, Hq=12, Hkv=4, D=16, S=40, k_sub_dim=4, v_sub_dim=4, n_c=16, window=7),
    dict(seed=4, B=4, Hq=8, Hkv=1, D=24, S=33, k_sub_dim=8, v_sub_dim=8, n_c=200, lens="ragged",
         skew=1.2, window=100),
]


@pytest.mark.parametrize("case", CASES, ids=[f"a{c['seed']}" for c in CASES])
def test_matches_torch_float64_sdpa(case):
    window = case.pop("window", 0)
    wl = W.attention_case(**case, window=window)
    case["window"] = window
    got = run(wl)
    want = torch_reference(wl)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-13)


def test_single_attended_token_returns_its_value_row():
    wl = W.attention_case(5, 2, 4, 2, 32, 20, 4, 8, 32)
    wl.window = 1
    got = run(wl)
    vcb = A.widen(wl.v_codebook, wl.dtype)
    for b in range(2):
        for hq in range(4):
            h = hq // 2
            row = vcb[h][wl.v_codes[b, h, wl.kv_len[b] - 1].astype(np.int64)].reshape(-1)
            assert np.array_equal(got[b, hq], row)
    wl.window = 0
    wl.kv_len = np.array([1, 1], np.int32)
    got = run(wl)
    assert np.array_equal(got[1, 3], vcb[1][wl.v_codes[1, 1, 0].astype(np.int64)].reshape(-1))


def test_equal_keys_or_zero_query_give_the_mean_value():
    wl = W.attention_case(6, 2, 2, 1, 16, 30, 4, 4, 16)
    wl.k_codes[:] = wl.k_codes[:, :, :1, :]          # every token has the same key
    got = run(wl)
    vcb = A.widen(wl.v_codebook, wl.dtype)
    for b in range(2):
        V = vcb[0][wl.v_codes[b, 0, :wl.kv_len[b]].astype(np.int64)].reshape(-1, 16)
        np.testing.assert_allclose(got[b, 0], V.mean(axis=0), rtol=1e-13, atol=1e-15)
    wl2 = W.attention_case(7, 1, 1, 1, 16, 30, 4, 4, 16)
    wl2.q[:] = 0
    V = vcb = A.widen(wl2.v_codebook, wl2.dtype)[0][wl2.v_codes[0, 0].astype(np.int64)].reshape(-1, 16)
    np.testing.assert_allclose(run(wl2)[0, 0], V.mean(axis=0), rtol=1e-13, atol=1e-15)


def test_empty_sequence_gives_zero():
    wl = W.attention_case(8, 3, 2, 1, 16, 10, 4, 4, 16, lens="ragged")
    assert wl.kv_len[0] == 0
    got = run(wl)
    assert np.all(got[0] == 0) and np.any(got[1] != 0)


def test_codes_past_the_codebook_decode_to_zero_rows():
    wl = W.attention_case(13, 1, 1, 1, 8, 3, 4, 4, 4)
    wl.k_codes[0, 0] = np.array([[0, 1], [200, 2], [3, 255]], np.uint8)
    wl.v_codes[0, 0] = np.array([[9, 0], [1, 2], [3, 4]], np.uint8)
    K = A.dequantize(wl.k_codes[0, 0], wl.k_codebook[0], wl.dtype)
    V = A.dequantize(wl.v_codes[0, 0], wl.v_codebook[0], wl.dtype)
    assert np.all(K[1, :4] == 0) and np.all(K[2, 4:] == 0) and np.any(K[0] != 0)
    assert np.all(V[0, :4] == 0) and np.all(V[2, 4:] == 0)
    assert np.all(np.isfinite(run(wl)))


def test_lookup_table_scores_equal_dense_scores():
    """The identity the kernels rely on: with q~ = q / f,
    sum_s LUT[s, code_s] = q . (k~ / f) for LUT[s, c] = q~_s . C_k[c]."""
    wl = W.attention_case(9, 1, 1, 1, 64, 40, 8, 8, 128)
    D, sd = 64, 8
    q = A.widen(wl.q, wl.dtype)[0, 0]
    cb = A.widen(wl.k_codebook, wl.dtype)[0]
    f = wl.k_scale[0].astype(np.float64)
    qt = q / f
    lut = np.stack([cb @ qt[s * sd:(s + 1) * sd] for s in range(D // sd)])     # [n_sub, n_c]
    codes = wl.k_codes[0, 0].astype(np.int64)
    lut_scores = np.array([sum(lut[s, codes[t, s]] for s in range(D // sd)) for t in range(40)])
    dense = (A.dequantize(codes, wl.k_codebook[0], wl.dtype) / f) @ q
    np.testing.assert_allclose(lut_scores, dense, rtol=1e-12, atol=1e-12)


def test_grouped_query_heads_use_their_kv_head():
    wl = W.attention_case(10, 2, 6, 2, 16, 25, 4, 4, 32, lens="mixed")
    full = run(wl)
    for hq in range(6):
        h = hq // 3
        one = W.AttnWorkload("one head", wl.q[:, hq:hq + 1], wl.k_codes[:, h:h + 1],
                             wl.v_codes[:, h:h + 1], wl.k_codebook[h:h + 1],
                             wl.v_codebook[h:h + 1], wl.k_scale[h:h + 1], wl.kv_len, wl.dtype)
        np.testing.assert_array_equal(run(one)[:, 0], full[:, hq])


def test_window_equals_the_sliced_cache():
    wl = W.attention_case(11, 3, 2, 2, 16, 40, 4, 4, 32, lens="mixed")
    wl.window = 9
    full = run(wl)
    for b in range(3):
        L = int(wl.kv_len[b])
        t0 = max(0, L - 9)
        part = W.AttnWorkload("slice", wl.q[b:b + 1], wl.k_codes[b:b + 1, :, t0:L],
                              wl.v_codes[b:b + 1, :, t0:L], wl.k_codebook, wl.v_codebook,
                              wl.k_scale, np.array([L - t0], np.int32), wl.dtype)
        np.testing.assert_array_equal(run(part)[0], full[b])


PINS = [
    lambda m: [_pin_matches_torch_sdpa(m, dict(c)) for c in CASES],
    lambda m: _pin_grouped_query_heads(m),
]


def _pin_matches_torch_sdpa(mod, case):
    window = case.pop("window", 0)
    wl = W.attention_case(**case, window=window)
    np.testing.assert_allclose(run(wl, mod), torch_reference(wl), rtol=1e-11, atol=1e-13)


def _pin_grouped_query_heads(mod):
    wl = W.attention_case(12, 2, 6, 2, 16, 25, 4, 4, 32, lens="mixed")
    np.testing.assert_allclose(run(wl, mod), torch_reference(wl), rtol=1e-11, atol=1e-13)


MUTANTS = {
    "gqa_modulo": ("h * g + j", "j * Hkv + h"),
    "scale_multiplied": ("K = K / np.asarray(k_scale[h], dtype=np.float64)[None, :]",
                         "K = K * np.asarray(k_scale[h], dtype=np.float64)[None, :]"),
    "window_off_by_one": ("start = max(0, L - window) if window > 0 else 0",
                          "start = max(0, L - window + 1) if window > 0 else 0"),
    "no_softmax_scale": ("s = (K @ qf[b, hq]) * softmax_scale\n                p = np.exp(s - s.max())\n                p = p / p.sum()\n                out",
                         "s = (K @ qf[b, hq])\n                p = np.exp(s - s.max())\n                p = p / p.sum()\n                out"),
    "unnormalized": ("p = p / p.sum()\n                out[b, hq] = p @ V",
                     "out[b, hq] = p @ V"),
    "values_from_key_codes": ("V = dequantize(v_codes[b, h, t0:t1], v_codebook[h], dtype)\n            for j in range(g):\n                hq = h * g + j\n                s = (K @ qf[b, hq]) * softmax_scale\n                p = np.exp(s - s.max())\n                p = p / p.sum()\n                out",
                              "V = dequantize(k_codes[b, h, t0:t1], v_codebook[h], dtype)\n            for j in range(g):\n                hq = h * g + j\n                s = (K @ qf[b, hq]) * softmax_scale\n                p = np.exp(s - s.max())\n                p = p / p.sum()\n                out"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_attention_mistake(name):
    src = open(A.__file__).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mod = types.ModuleType("mutant_attention")
    exec(compile(src.replace(old, new, 1), os.path.basename(A.__file__), "exec"), mod.__dict__)
    caught = False
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError):   # a wrong value or a wrong shape
            caught = True
            break
    assert caught, f"no pin caught {name!r}"
