"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/vq.h declares, and
reject bad arguments on the host before any HIP call (so these calls never
touch a device; the pointers below are never dereferenced).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vq.h")

vq = pytest.importorskip("product_vq_kv_amd")

OK, INVALID, UNSUPPORTED, MISALIGNED, TOO_LARGE = 0, -1, -2, -3, -5
FAKE = 0x10000  # aligned, never dereferenced by a rejected call


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(vq_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == ["vq_abi_version", "vq_attention_decode",
                                    "vq_attention_decode_static",
                                    "vq_attention_workspace_bytes", "vq_decode", "vq_encode",
                                    "vq_encode_packed", "vq_kmeans", "vq_kmeans_workspace_bytes",
                                    "vq_last_hip_error", "vq_status_str"]


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(vq.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    assert vq.lib.vq_abi_version() == 6
    for code in (0, -1, -2, -3, -4, -5, 99):
        assert isinstance(vq.lib.vq_status_str(code), bytes)
    assert vq.lib.vq_status_str(-3) == b"misaligned pointer"
    assert vq.lib.vq_last_hip_error() == 0


def enc(**over):
    a = dict(x=FAKE, cb=FAKE, n=1024, sd=8, n_c=256, dt=0, stride=0, k=1, glen=1024, gmap=None,
             out=FAKE, stream=None)
    a.update(over)
    return vq.lib.vq_encode(a["x"], a["cb"], a["n"], a["sd"], a["n_c"], a["dt"], a["stride"],
                            a["k"], a["glen"], a["gmap"], a["out"], a["stream"])


def enc_packed(**over):
    a = dict(x=FAKE, cb=FAKE, n=1024, sd=8, n_c=256, dt=0, stride=0, k=1, glen=1024, gmap=None,
             scale=FAKE, hd=128, sstride=0, bits=8, out=FAKE, stream=None)
    a.update(over)
    return vq.lib.vq_encode_packed(a["x"], a["cb"], a["n"], a["sd"], a["n_c"], a["dt"],
                                   a["stride"], a["k"], a["glen"], a["gmap"], a["scale"], a["hd"],
                                   a["sstride"], a["bits"], a["out"], a["stream"])


def dec(**over):
    a = dict(idx=FAKE, cb=FAKE, n=1024, sd=8, n_c=256, dt=0, stride=0, k=1, glen=1024, gmap=None,
             out=FAKE, stream=None)
    a.update(over)
    return vq.lib.vq_decode(a["idx"], a["cb"], a["n"], a["sd"], a["n_c"], a["dt"], a["stride"],
                            a["k"], a["glen"], a["gmap"], a["out"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(sd=2), UNSUPPORTED), (dict(sd=16), UNSUPPORTED), (dict(sd=0), UNSUPPORTED),
    (dict(dt=2), UNSUPPORTED), (dict(dt=-1), UNSUPPORTED),
    (dict(n_c=65537), UNSUPPORTED), (dict(n_c=0), INVALID), (dict(n_c=-5), INVALID),
    (dict(n=-1), INVALID), (dict(k=0), INVALID), (dict(glen=0), INVALID),
    (dict(x=None), INVALID), (dict(cb=None), INVALID), (dict(out=None), INVALID),
    (dict(x=FAKE + 8), MISALIGNED), (dict(sd=4, x=FAKE + 4), MISALIGNED),
    (dict(cb=FAKE + 1), MISALIGNED), (dict(out=FAKE + 2), MISALIGNED),
    (dict(gmap=FAKE + 2, glen=100), MISALIGNED),
    # two groups but one codebook slot and no map
    (dict(glen=512), INVALID),
    # several slots need a stride of at least n_centroids * sub_dim
    (dict(k=2, glen=512, stride=256 * 8 - 1), INVALID),
    # n * sub_dim * 2 bytes would overflow
    (dict(n=2 ** 62), INVALID),
    # grid would exceed 2^31 - 1 workgroups: 2^31 one-row groups
    (dict(n=2 ** 31, glen=1, k=2 ** 31), INVALID),
])
def test_encode_rejects_on_host(over, code):
    assert enc(**over) == code


@pytest.mark.parametrize("over", [dict(n=0), dict(n=0, x=None, cb=None, out=None),
                                  dict(n=0, sd=4, dt=1, n_c=65536)])
def test_encode_empty_is_ok_without_launch(over):
    assert enc(**over) == OK


@pytest.mark.parametrize("over,code", [
    (dict(sd=3), UNSUPPORTED), (dict(dt=5), UNSUPPORTED), (dict(n_c=0), INVALID),
    (dict(idx=None), INVALID), (dict(out=None), INVALID), (dict(idx=FAKE + 2), MISALIGNED),
    (dict(out=FAKE + 1), MISALIGNED), (dict(glen=10), INVALID),
])
def test_decode_rejects_on_host(over, code):
    assert dec(**over) == code


def test_decode_empty_is_ok():
    assert dec(n=0) == OK


def test_python_wrapper_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(16, 8, dtype=torch.float16)
    cb = torch.zeros(4, 8, dtype=torch.float16)
    with pytest.raises(ValueError, match="device"):
        vq.encode(x, cb)
    with pytest.raises(ValueError, match="device"):
        vq.decode(torch.zeros(16, dtype=torch.uint32), cb)


def test_vqerror_message_names_the_status():
    e = vq.VQError(-3, "vq_encode")
    assert "VQ_ERR_MISALIGNED" in str(e) and "misaligned" in str(e)


@pytest.mark.parametrize("over,code", [
    # the checks shared with vq_encode
    (dict(sd=2), UNSUPPORTED), (dict(n_c=65537, bits=32), UNSUPPORTED), (dict(n=-1), INVALID),
    (dict(x=None), INVALID), (dict(out=None), INVALID), (dict(x=FAKE + 8), MISALIGNED),
    # code width
    (dict(bits=0), INVALID), (dict(bits=33), INVALID), (dict(bits=7), INVALID),
    (dict(n_c=2, bits=1, scale=None, n=0), OK), (dict(n_c=3, bits=1), INVALID),
    # smoothing factors
    (dict(hd=4), INVALID), (dict(hd=12), INVALID), (dict(hd=0), INVALID),
    (dict(hd=4104), INVALID), (dict(sstride=-1), INVALID), (dict(scale=FAKE + 2), MISALIGNED),
    (dict(scale=None, hd=0, n=0), OK),
    # the stream must be 4-byte aligned
    (dict(out=FAKE + 1), MISALIGNED), (dict(out=FAKE + 2), MISALIGNED),
    # groups must start on a 32-bit word of the stream
    (dict(k=2, stride=2048, glen=514, bits=8), UNSUPPORTED),
    (dict(k=2, stride=2048, glen=521, bits=4, n_c=16), UNSUPPORTED),
    (dict(k=4, stride=2048, glen=301, bits=8), UNSUPPORTED),
])
def test_encode_packed_rejects_on_host(over, code):
    assert enc_packed(**over) == code


def test_encode_packed_empty_is_ok_without_launch():
    assert enc_packed(n=0, x=None, cb=None, out=None, scale=None) == OK


@pytest.mark.parametrize("over", [
    dict(k=2, stride=2048, glen=520, bits=8), dict(k=2, stride=2048, glen=520, bits=4, n_c=16),
    dict(k=2, stride=2048, glen=513, bits=32), dict(k=2, stride=2048, glen=1024, n=2048, bits=1, n_c=2),
])
def test_encode_packed_word_aligned_groups_pass_validation(over):
    """Supported group layouts get past every host check; with no device the
    call then fails at the launch (these fake pointers are never launched on
    a machine with a GPU)."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("would launch on the fake pointers")
    assert enc_packed(**over) == -4


def attn(**over):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, kcb=FAKE, vcb=FAKE, ks=None, kl=None, B=2, Hq=12, Hkv=4,
             D=256, S=100, sdk=4, sdv=4, n_c=256, dt=0, window=0, scale=0.0625, out=FAKE,
             ws=FAKE, wsb=1 << 30, stream=None)
    a.update(over)
    return vq.lib.vq_attention_decode(a["q"], a["kc"], a["vc"], a["kcb"], a["vcb"], a["ks"],
                                      a["kl"], a["B"], a["Hq"], a["Hkv"], a["D"], a["S"],
                                      a["sdk"], a["sdv"], a["n_c"], a["dt"], a["window"],
                                      a["scale"], a["out"], a["ws"], a["wsb"], a["stream"])


def test_workspace_sizes_that_overflow_are_rejected():
    """Sizes whose byte counts do not fit 63 bits give 0, and the calls
    reject them instead of accepting a wrapped (small) workspace."""
    big = (1 << 31) - 1
    assert vq.lib.vq_attention_workspace_bytes(65535, 32768, 256, big) == 0
    assert vq.lib.vq_attention_workspace_bytes(2, 12, 256, big) == 2 * 12 * (big // 256 + 1) * 258 * 4
    assert vq.lib.vq_kmeans_workspace_bytes(8, 65536, (1 << 62), 1) == 0
    assert attn(B=65535, Hq=32768, Hkv=32768, D=256, S=big, wsb=1 << 20) == INVALID
    assert attn_static(B=65535, Hq=32768, Hkv=32768, D=256, S=big) == INVALID


def test_attention_workspace_size():
    # one (D + 2)-float partial per (sequence, query head, 256-token chunk)
    assert vq.lib.vq_attention_workspace_bytes(2, 12, 256, 100) == 2 * 12 * 1 * 258 * 4
    assert vq.lib.vq_attention_workspace_bytes(2, 12, 256, 1025) == 2 * 12 * 5 * 258 * 4
    assert vq.lib.vq_attention_workspace_bytes(-1, 12, 256, 100) == 0


@pytest.mark.parametrize("over,code", [
    (dict(sdk=2), UNSUPPORTED), (dict(sdv=16), UNSUPPORTED), (dict(dt=3), UNSUPPORTED),
    (dict(n_c=257), UNSUPPORTED), (dict(n_c=0), UNSUPPORTED), (dict(D=512), UNSUPPORTED),
    (dict(D=40, sdk=4), UNSUPPORTED), (dict(D=36, sdk=4, sdv=8), UNSUPPORTED),
    (dict(Hq=13), INVALID), (dict(Hq=36, Hkv=4), UNSUPPORTED), (dict(Hkv=0), INVALID),
    (dict(B=-1), INVALID), (dict(S=-1), INVALID), (dict(window=-1), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(q=None), INVALID), (dict(out=None), INVALID), (dict(kc=None), INVALID),
    (dict(ws=None), INVALID), (dict(wsb=100), INVALID),
    (dict(q=FAKE + 1), MISALIGNED), (dict(kc=FAKE + 2), MISALIGNED),
    (dict(out=FAKE + 2), MISALIGNED), (dict(ws=FAKE + 2), MISALIGNED),
    (dict(ks=FAKE + 2), MISALIGNED), (dict(kl=FAKE + 1), MISALIGNED),
    (dict(B=70000), INVALID),
    (dict(B=0), OK), (dict(B=0, q=None, out=None, ws=None), OK),
])
def test_attention_rejects_on_host(over, code):
    assert attn(**over) == code


def attn_static(**over):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, kcb=FAKE, vcb=FAKE, ks=None, kl=None, B=2, Hq=12, Hkv=4,
             D=256, S=100, sdk=4, sdv=4, n_c=256, dt=0, window=0, scale=0.0625, out=FAKE,
             stream=None)
    a.update(over)
    return vq.lib.vq_attention_decode_static(a["q"], a["kc"], a["vc"], a["kcb"], a["vcb"],
                                             a["ks"], a["kl"], a["B"], a["Hq"], a["Hkv"], a["D"],
                                             a["S"], a["sdk"], a["sdv"], a["n_c"], a["dt"],
                                             a["window"], a["scale"], a["out"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(sdk=2), UNSUPPORTED), (dict(n_c=257), UNSUPPORTED), (dict(Hq=13), INVALID),
    (dict(B=-1), INVALID), (dict(scale=float("nan")), INVALID), (dict(q=None), INVALID),
    (dict(kc=None), INVALID), (dict(q=FAKE + 1), MISALIGNED), (dict(out=FAKE + 2), MISALIGNED),
    # partials beyond the static buffer: 1024 x 8 x 16 chunks x 258 floats
    (dict(B=1024, Hq=8, Hkv=1, S=4096), TOO_LARGE),
    (dict(B=64, Hq=32, Hkv=8, S=8192), TOO_LARGE),
    (dict(B=0), OK), (dict(B=0, q=None, out=None), OK),
])
def test_attention_static_rejects_on_host(over, code):
    assert attn_static(**over) == code


def test_attention_static_limit_is_the_header_constant():
    assert vq.ATTN_STATIC_SCRATCH_BYTES == 32 << 20
    text = open(HEADER).read()
    assert "#define VQ_ATTN_STATIC_SCRATCH_BYTES (32u << 20)" in text
    # the largest Falcon3-7B decode batch at 4096 tokens that fits
    need = vq.lib.vq_attention_workspace_bytes(160, 12, 256, 4096)
    assert need <= vq.ATTN_STATIC_SCRATCH_BYTES < vq.lib.vq_attention_workspace_bytes(170, 12, 256,
                                                                                     4096)


def km(**over):
    a = dict(x=FAKE, cb=FAKE, n=1024, sd=8, n_c=256, dt=0, stride=0, k=1, glen=1024, gmap=None,
             it=5, out=FAKE, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(over)
    return vq.lib.vq_kmeans(a["x"], a["cb"], a["n"], a["sd"], a["n_c"], a["dt"], a["stride"],
                            a["k"], a["glen"], a["gmap"], a["it"], a["out"], a["ws"], a["wsb"],
                            a["stream"])


def test_kmeans_workspace_size():
    # 8 replicas of the exact member sums (one int64 per component for fp16,
    # 8 limbs for bf16) and uint32 counts per (slot, centroid)
    assert vq.lib.vq_kmeans_workspace_bytes(8, 256, 4, 0) == 8 * 4 * 256 * (8 * 8 + 4)
    assert vq.lib.vq_kmeans_workspace_bytes(8, 256, 4, 1) == 8 * 4 * 256 * (8 * 8 * 8 + 4)
    assert vq.lib.vq_kmeans_workspace_bytes(4, 4096, 1, 1) == 8 * 4096 * (4 * 8 * 8 + 4)
    assert vq.lib.vq_kmeans_workspace_bytes(3, 256, 4, 0) == 0
    assert vq.lib.vq_kmeans_workspace_bytes(8, 256, 4, 2) == 0


@pytest.mark.parametrize("over,code", [
    (dict(dt=2), UNSUPPORTED), (dict(sd=2), UNSUPPORTED), (dict(n_c=0), INVALID),
    (dict(dt=1, wsb=8 * 256 * (8 * 8 + 4)), INVALID),    # an fp16-sized workspace for bf16
    (dict(it=-1), INVALID), (dict(x=None), INVALID), (dict(out=None), INVALID),
    (dict(ws=None), INVALID), (dict(wsb=16), INVALID), (dict(x=FAKE + 8), MISALIGNED),
    (dict(out=FAKE + 2), MISALIGNED), (dict(ws=FAKE + 4), MISALIGNED),
    (dict(glen=512), INVALID),                            # two groups, one slot, no map
    (dict(n=(1 << 23) + 1, glen=(1 << 23) + 1), UNSUPPORTED),
    (dict(n=(1 << 24), glen=1 << 23, gmap=FAKE), UNSUPPORTED),
    (dict(n=0), OK), (dict(it=0), OK), (dict(n=0, x=None, out=None, ws=None), OK),
])
def test_kmeans_rejects_on_host(over, code):
    assert km(**over) == code
