"""GPU parity of decode attention over VQ codes against the float64 oracle.

``vq_attention_decode`` (through its C ABI) must match oracle/attention.py
within the error bound of tests/attention_bound.py, derived from fp32
arithmetic in any summation order:

  |out - ref|  <=  (2 Delta + (3 T + 32) u) * M_d,
  Delta = 1.5 (sd_k + n_sub_k + 4) u A,

with A, T and M_d from the (pinned) ``tolerance_terms``.  The measured error
is reported too and is typically ~1e-7 of M.  Cases cover both code sub-dims
for keys and values, fp16 and bf16, smoothed and plain keys, grouped-query
groups 1..8, head_dim 16..256, multi-chunk and ragged lengths (empty and
one-token sequences), windows, codes past the codebook, a dirty workspace,
sizes that run the streaming form (balanced token ranges, running softmax,
up to 2048 sequences), the Falcon3-7B decode workload at full size (32 and
128 sequences: the chunked and the streaming form), and that workload with the
tokens next to every 256-token chunk boundary carrying the attention (so a
dropped, repeated or misweighted boundary token is far outside the bound).
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from tests import attention_bound as AB

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import product_vq_kv_amd as vq  # noqa: E402

DEV = torch.device("cuda:0")


def to_dev(wl):
    tdt = torch.float16 if wl.dtype == W.F16 else torch.bfloat16

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).to(DEV)

    return dict(q=bits(wl.q), k_codes=torch.from_numpy(wl.k_codes).to(DEV),
                v_codes=torch.from_numpy(wl.v_codes).to(DEV), k_codebook=bits(wl.k_codebook),
                v_codebook=bits(wl.v_codebook),
                k_scale=None if wl.k_scale is None else torch.from_numpy(wl.k_scale).to(DEV),
                kv_len=torch.from_numpy(wl.kv_len.astype(np.int32)).to(DEV))


def gpu_attention(wl, dirty_workspace=True):
    t = to_dev(wl)
    B, Hq, Hkv, D, S = wl.shape
    ws = None
    if dirty_workspace:
        n = vq.attention_workspace_bytes(B, Hq, D, S) // 4
        ws = torch.full((max(n, 1),), float("nan"), dtype=torch.float32, device=DEV)
    out = vq.attention_decode(t["q"], t["k_codes"], t["v_codes"], t["k_codebook"],
                              t["v_codebook"], k_scale=t["k_scale"], kv_len=t["kv_len"],
                              window=wl.window, softmax_scale=wl.softmax_scale, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def assert_attention_parity(wl):
    B, Hq, Hkv, D, S = wl.shape
    ref = A.decode_attention(wl.q, wl.k_codes, wl.v_codes, wl.k_codebook, wl.v_codebook,
                             wl.dtype, **wl.kwargs())
    Aq, T, M = A.tolerance_terms(wl.q, wl.k_codes, wl.v_codes, wl.k_codebook, wl.v_codebook,
                                 wl.dtype, **wl.kwargs())
    got = gpu_attention(wl)
    sdk = D // wl.k_codes.shape[3]
    n_sub_k = wl.k_codes.shape[3]
    rel = AB.relative_bound(Aq, T, sdk, n_sub_k)
    bound = AB.bound(Aq, T, M, sdk, n_sub_k)
    err = np.abs(got - ref)
    worst = float(np.max(err / np.maximum(M, 1e-300))) if M.size else 0.0
    print(f"[parity] {wl.name}: max |err| / M = {worst:.3e}, "
          f"bound/M up to {float(rel.max()) if rel.size else 0:.3e}", flush=True)
    assert np.all(np.isfinite(got))
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{len(bad)} outputs outside the bound; first {bad[:3].tolist()}: "
                           f"got {got[tuple(bad[0])]} want {ref[tuple(bad[0])]}")
    # empty sequences give exact zeros
    assert np.all(got[wl.kv_len == 0] == 0)


CASES = [
    # (seed, B, Hq, Hkv, D, S, sdk, sdv, n_c, dtype, extras)
    (1, 3, 6, 2, 32, 50, 4, 8, 64, W.F16, dict(lens="ragged")),
    (2, 2, 4, 4, 64, 129, 8, 4, 256, W.BF16, dict(lens="mixed", smooth=False)),
    (3, 2, 12, 4, 16, 40, 4, 4, 16, W.F16, dict(window=7)),
    (4, 4, 8, 1, 32, 33, 8, 8, 200, W.F16, dict(lens="ragged", skew=1.2, window=100)),
    (5, 3, 12, 4, 256, 1500, 4, 4, 256, W.F16, dict(lens="ragged")),
    (6, 2, 32, 8, 128, 2049, 8, 8, 256, W.BF16, dict(lens="mixed")),
    (7, 5, 8, 8, 128, 700, 8, 4, 256, W.F16, dict(lens="mixed", window=333)),
    (8, 2, 16, 2, 64, 1100, 4, 8, 100, W.F16, dict(lens="ragged", skew=0.8)),
    (9, 1, 1, 1, 256, 4096, 4, 4, 256, W.BF16, dict()),
    (10, 6, 4, 1, 96, 520, 8, 8, 33, W.F16, dict(lens="ragged", window=513)),
    # more sequences than a workgroup has threads, 8 query heads per kv head,
    # sub_dim 8 bf16 keys and values
    (11, 300, 8, 2, 64, 300, 4, 4, 64, W.F16, dict(lens="ragged")),
    (12, 4, 16, 2, 128, 1000, 4, 4, 256, W.F16, dict(lens="mixed", window=300)),
    (13, 7, 4, 4, 256, 777, 8, 8, 256, W.BF16, dict(lens="ragged")),
    (14, 3, 8, 2, 256, 3000, 4, 8, 128, W.F16, dict(lens="mixed", smooth=False)),
]


# Sizes at which the streaming form runs (at least 32 slices of 64 tokens per
# workgroup, counted on max_kv_len): more sequences than a workgroup has
# threads (the length scan takes several rounds) with empty and one-token
# sequences, bf16 with sub_dim 8 keys, 8 query heads per kv head with a window.
STREAM_CASES = [
    (31, 2048, 2, 1, 64, 1024, 4, 4, 256, W.F16, dict(lens="ragged")),
    (32, 640, 8, 2, 128, 2048, 8, 4, 256, W.BF16, dict(lens="ragged")),
    (33, 260, 16, 2, 256, 2048, 4, 4, 256, W.F16, dict(lens="mixed", window=1500)),
]


@pytest.mark.parametrize("case", CASES + STREAM_CASES,
                         ids=[f"t{c[0]}_B{c[1]}_D{c[4]}_S{c[5]}" for c in CASES + STREAM_CASES])
def test_attention_matches_oracle(case):
    seed, B, Hq, Hkv, D, S, sdk, sdv, n_c, dt, extra = case
    window = extra.pop("window", 0)
    wl = W.attention_case(seed, B, Hq, Hkv, D, S, sdk, sdv, n_c, dt, window=window, **extra)
    extra["window"] = window
    print(f"[case] {wl.name}", flush=True)
    assert_attention_parity(wl)


def test_codes_past_the_codebook_read_zero_rows():
    wl = W.attention_case(20, 2, 4, 2, 64, 300, 4, 8, 50, W.F16, lens="mixed")
    r = np.random.default_rng(20)
    wl.k_codes[r.random(wl.k_codes.shape) < 0.05] = 255
    wl.v_codes[r.random(wl.v_codes.shape) < 0.05] = 200
    assert_attention_parity(wl)


@pytest.mark.parametrize("sd", [8, 4])
def test_softmax_scale_and_identical_results_across_workspaces(sd):
    wl = W.attention_case(21, 2, 6, 3, 64, 900, sd, sd, 256, W.F16, lens="mixed")
    wl.softmax_scale = 0.3
    assert_attention_parity(wl)
    a = gpu_attention(wl, dirty_workspace=True)
    b = gpu_attention(wl, dirty_workspace=False)
    assert np.array_equal(a, b)


def test_codes_past_the_codebook_read_zero_rows_matrix_core_shape():
    wl = W.attention_case(23, 3, 8, 2, 128, 700, 4, 4, 77, W.F16, lens="ragged")
    r = np.random.default_rng(23)
    wl.k_codes[r.random(wl.k_codes.shape) < 0.05] = 255
    wl.v_codes[r.random(wl.v_codes.shape) < 0.05] = 130
    assert_attention_parity(wl)


def test_all_sequences_empty():
    wl = W.attention_case(22, 3, 4, 2, 32, 64, 4, 4, 64, W.F16)
    wl.kv_len[:] = 0
    assert np.all(gpu_attention(wl) == 0)


@pytest.mark.parametrize("B", [32, 128])
def test_falcon_decode_workload_full_size(B):
    wl = W.falcon_decode_attention(B=B)
    print(f"[case] {wl.name}", flush=True)
    assert_attention_parity(wl)


def test_falcon_decode_boundary_tokens_carry_the_attention():
    wl = W.falcon_decode_attention(B=8)
    AB.make_boundary_tokens_heavy(wl)
    wl.name += ", boundary tokens heavy"
    print(f"[case] {wl.name}", flush=True)
    assert_attention_parity(wl)


def test_query_and_codebooks_only_2_byte_aligned():
    """Query and codebooks at addresses 2 bytes past a 16-byte boundary (the
    contract's minimum alignment) give results identical to aligned ones."""
    wl = W.attention_case(24, 4, 12, 4, 256, 700, 4, 4, 256, W.F16, lens="ragged")
    print(f"[case] {wl.name}", flush=True)
    t = to_dev(wl)

    def shifted(x):  # same values at an address 2 bytes past a 16-byte boundary
        buf = torch.empty(x.numel() + 8, dtype=x.dtype, device=DEV)
        v = buf[1:1 + x.numel()].view(x.shape)
        v.copy_(x)
        assert v.data_ptr() % 16 == 2 and v.is_contiguous()
        return v

    def run(q, kcb, vcb):
        out = vq.attention_decode(q, t["k_codes"], t["v_codes"], kcb, vcb, k_scale=t["k_scale"],
                                  kv_len=t["kv_len"], window=wl.window,
                                  softmax_scale=wl.softmax_scale)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64)

    assert t["q"].data_ptr() % 16 == 0 and t["k_codebook"].data_ptr() % 16 == 0
    aligned = run(t["q"], t["k_codebook"], t["v_codebook"])
    for q, kcb, vcb in ((shifted(t["q"]), t["k_codebook"], t["v_codebook"]),
                        (t["q"], shifted(t["k_codebook"]), shifted(t["v_codebook"]))):
        assert np.array_equal(run(q, kcb, vcb), aligned)
    assert_attention_parity(wl)
