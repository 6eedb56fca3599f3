"""The allocation-free decode-attention entry point on the GPU.

``vq_attention_decode_static`` (through its C ABI) must give the same output
as ``vq_attention_decode`` with a caller workspace (the same kernels; the
static per-GPU scratch replaces the workspace), and both must be within the
derived error bound of the float64 oracle.  Two calls in a row, the second
on a smaller input, so the second reads a scratch buffer the first left
dirty; the device's free memory must not change across a static call.
Captured in a HIP graph (through torch's graph API), the call must give
the eager result on every replay, with new queries copied in and other
eager work between the replays.  Both decode forms are covered: the chunked
one, and the streaming one at 128 Falcon3-7B sequences (its partials and
segment table in the same scratch).
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


def _dev(wl):
    tdt = torch.float16 if wl.dtype == W.F16 else torch.bfloat16

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).to(DEV)

    return dict(q=bits(wl.q), k_codes=torch.from_numpy(wl.k_codes).to(DEV),
                v_codes=torch.from_numpy(wl.v_codes).to(DEV), k_codebook=bits(wl.k_codebook),
                v_codebook=bits(wl.v_codebook),
                k_scale=None if wl.k_scale is None else torch.from_numpy(wl.k_scale).to(DEV),
                kv_len=torch.from_numpy(wl.kv_len.astype(np.int32)).to(DEV))


def _check_against_oracle(wl, got):
    B, Hq, Hkv, D, S = wl.shape
    ref = A.decode_attention(wl.q, wl.k_codes, wl.v_codes, wl.k_codebook, wl.v_codebook,
                             wl.dtype, **wl.kwargs())
    Aq, T, M = A.tolerance_terms(wl.q, wl.k_codes, wl.v_codes, wl.k_codebook, wl.v_codebook,
                                 wl.dtype, **wl.kwargs())
    n_sub_k = wl.k_codes.shape[3]
    bound = AB.bound(Aq, T, M, D // n_sub_k, n_sub_k)
    assert np.all(np.abs(got - ref) <= bound)


def _workload(case):
    if case == "falcon128":  # runs the streaming form
        return W.falcon_decode_attention(B=128)
    seed, B, Hq, Hkv, D, S, sdk, sdv, n_c, dt, lens = case
    return W.attention_case(seed, B, Hq, Hkv, D, S, sdk, sdv, n_c, dt, lens=lens)


@pytest.mark.parametrize("first,second", [
    # (seed, B, Hq, Hkv, D, S, sdk, sdv, n_c, dtype, lens)
    ((51, 8, 12, 4, 256, 3000, 4, 4, 256, W.F16, "mixed"),
     (52, 3, 12, 4, 256, 700, 4, 4, 256, W.F16, "ragged")),
    ((53, 4, 8, 2, 96, 1500, 8, 8, 200, W.BF16, "mixed"),
     (54, 2, 4, 1, 32, 300, 4, 8, 64, W.F16, "ragged")),
    ("falcon128", (52, 3, 12, 4, 256, 700, 4, 4, 256, W.F16, "ragged")),
], ids=["chunked", "chunked-lut", "streaming"])
def test_static_scratch_matches_the_workspace_entry_point(first, second):
    for case in (first, second):
        wl = _workload(case)
        B, Hq, Hkv, D, S = wl.shape
        print(f"[case] {wl.name}", flush=True)
        t = _dev(wl)
        ref = vq.attention_decode(t["q"], t["k_codes"], t["v_codes"], t["k_codebook"],
                                  t["v_codebook"], k_scale=t["k_scale"], kv_len=t["kv_len"])
        out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info(DEV)[0]
        vq.attention_decode_static(t["q"], t["k_codes"], t["v_codes"], t["k_codebook"],
                                   t["v_codebook"], k_scale=t["k_scale"], kv_len=t["kv_len"],
                                   out=out)
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info(DEV)[0]
        assert free1 == free0, f"free device memory changed by {free0 - free1} bytes"
        a = out.cpu().numpy()
        b = ref.cpu().numpy()
        assert np.array_equal(a, b), "static-scratch output differs from the workspace call"
        _check_against_oracle(wl, a.astype(np.float64))


def test_static_scratch_rejects_inputs_beyond_its_size():
    wl = W.attention_case(55, 2, 4, 2, 64, 100, 4, 4, 64, W.F16)
    t = _dev(wl)
    out = torch.empty((2, 4, 64), dtype=torch.float32, device=DEV)
    # 1024 sequences x 8 heads x 16 chunks x 258 floats: 135 MB of partials
    with pytest.raises(vq.VQError, match="TOO_LARGE"):
        vq.attention_decode_static_raw(t["q"].data_ptr(), t["k_codes"].data_ptr(),
                                       t["v_codes"].data_ptr(), t["k_codebook"].data_ptr(),
                                       t["v_codebook"].data_ptr(), None, None, 1024, 8, 1, 256,
                                       4096, 4, 4, 64, W.F16, 0, 0.0625, out.data_ptr(), None)


@pytest.mark.parametrize("case", [(56, 6, 12, 4, 256, 1800, 4, 4, 256, W.F16, "mixed"),
                                  "falcon128"], ids=["chunked", "streaming"])
def test_static_entry_point_captured_in_a_graph(case):
    wl = _workload(case)
    t = _dev(wl)
    B, Hq, Hkv, D, S = wl.shape
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    args = (t["q"], t["k_codes"], t["v_codes"], t["k_codebook"], t["v_codebook"])
    kw = dict(k_scale=t["k_scale"], kv_len=t["kv_len"])
    vq.attention_decode_static(*args, **kw, out=out)      # resolves the scratch address
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        vq.attention_decode_static(*args, **kw, out=out)
    rng = np.random.default_rng(56)
    for rep in range(3):
        qn = torch.from_numpy(rng.standard_normal((B, Hq, D)).astype(np.float16)).to(DEV)
        t["q"].copy_(qn)                                   # eager work between replays
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        ref = vq.attention_decode(*args, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from the eager call"
    print("[graph] 3 replays equal to the eager call", flush=True)
