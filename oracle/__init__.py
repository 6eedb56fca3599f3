"""CPU oracle for the product-VQ encode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (``product_vq_kv_amd``)
never imports, links or runs it; it shares no code with the HIP library.

The arithmetic lives in ``vq_oracle.c`` (plain single-threaded C, built with
``-ffp-contract=off`` so the explicit ``fmaf`` is the only fused operation).
This module only compiles it and marshals numpy arrays to it.  What each C
function computes, and which passage of the VeloxQuant-MLX blog post "I Wrote
a Metal Kernel to Stop My Mac From OOMing" it follows, is stated in the C
file's header.

Parity status: every function here is pinned.  ``tests/test_oracle_pins.py``
pins the search (exact integer brute force, hand-built known answers, the
sub_dim = 1 boundary-sum special case, conversion against library routines);
``tests/test_oracle_smooth_pack.py`` pins smoothing, the search over fp32
sub-vectors and the packed code stream (numpy's float32 multiply and
little-endian packbits, the pages' worked packing examples, exact rational
brute force).  ``tests/test_oracle_mutants.py`` checks that planted mistakes
fail those pins.  ``oracle/attention.py`` (decode attention over VQ-coded
caches, float64 numpy from its plain definition) is pinned by
``tests/test_oracle_attention.py``; ``oracle/kmeans.py`` (Lloyd iterations
with exact member means rounded once to fp16) by ``tests/test_oracle_kmeans.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

F16 = 0
BF16 = 1
BAD_SLOT = 0xFFFFFFFF

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libvq_oracle.so")
_lib = None
_lock = threading.Lock()


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int
        lib.vqo_encode.argtypes = [p, p, i64, i32, i32, i32, i64, i64, i64, p, p]
        lib.vqo_encode.restype = i32
        lib.vqo_encode_top2.argtypes = [p, p, i64, i32, i32, i32, i64, i64, i64, p, p, p, p]
        lib.vqo_encode_top2.restype = i32
        lib.vqo_decode.argtypes = [p, p, i64, i32, i32, i32, i64, i64, i64, p, p]
        lib.vqo_decode.restype = i32
        lib.vqo_sqdist.argtypes = [p, p, i32, i32]
        lib.vqo_sqdist.restype = ctypes.c_float
        lib.vqo_to_f32.argtypes = [ctypes.c_uint16, i32]
        lib.vqo_to_f32.restype = ctypes.c_float
        lib.vqo_smooth.argtypes = [p, i64, i32, i32, p, i32, i64, i64, i64, p, p]
        lib.vqo_smooth.restype = i32
        lib.vqo_encode_f32.argtypes = [p, p, i64, i32, i32, i32, i64, i64, i64, p, p, p, p]
        lib.vqo_encode_f32.restype = i32
        lib.vqo_packed_bytes.argtypes = [i64, i32]
        lib.vqo_packed_bytes.restype = i64
        lib.vqo_pack.argtypes = [p, i64, i32, p]
        lib.vqo_pack.restype = i32
        lib.vqo_unpack.argtypes = [p, i64, i32, p]
        lib.vqo_unpack.restype = i32
        lib.vqo_encode_packed.argtypes = [p, p, i64, i32, i32, i32, i64, i64, i64, p, p, i32,
                                          i64, i32, p]
        lib.vqo_encode_packed.restype = i32
        _lib = lib
        return lib


def _u16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype in (np.float16,):
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected 16-bit element bits, got {a.dtype}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def _common(x, codebook, sub_dim, n_centroids, codebook_stride, n_codebooks,
            group_len, group_map):
    x = _u16(x).reshape(-1)
    codebook = _u16(codebook).reshape(-1)
    n = x.size // sub_dim
    if x.size != n * sub_dim:
        raise ValueError("x size is not a multiple of sub_dim")
    if codebook_stride is None:
        codebook_stride = n_centroids * sub_dim
    if group_len is None:
        group_len = max(n, 1)
    if group_map is not None:
        group_map = np.ascontiguousarray(group_map, dtype=np.int32)
    need = (n_codebooks - 1) * codebook_stride + n_centroids * sub_dim
    if codebook.size < need:
        raise ValueError("codebook buffer is smaller than n_codebooks slots")
    return x, codebook, n, codebook_stride, group_len, group_map


def encode(x, codebook, sub_dim, n_centroids, dtype, *, codebook_stride=None,
           n_codebooks=1, group_len=None, group_map=None, threads=1):
    """Nearest-centroid indices (uint32) for every sub-vector of ``x``.

    ``threads > 1`` slices the rows across Python threads that each call the
    same single-threaded C routine (ctypes drops the GIL); the result does not
    depend on the slicing.
    """
    x, cb, n, stride, glen, gmap = _common(x, codebook, sub_dim, n_centroids,
                                           codebook_stride, n_codebooks, group_len, group_map)
    lib = _load()
    out = np.empty(n, dtype=np.uint32)
    if n == 0:
        return out
    if threads <= 1 or n < 4096:
        rc = lib.vqo_encode(_ptr(x), _ptr(cb), n, sub_dim, n_centroids, dtype, stride,
                            n_codebooks, glen, _ptr(gmap), _ptr(out))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return out
    # Each slice gets a per-row slot map (group_len = 1), so a slice may start
    # anywhere inside a group.
    bounds = np.linspace(0, n, threads + 1).astype(np.int64)
    errs = []

    def work(lo, hi):
        g = np.arange(lo, hi, dtype=np.int64) // glen
        slots = (gmap[g] if gmap is not None else g).astype(np.int32)
        xs = x[lo * sub_dim: hi * sub_dim]
        o = out[lo:hi]
        rc = lib.vqo_encode(_ptr(xs), _ptr(cb), hi - lo, sub_dim, n_centroids, dtype, stride,
                            n_codebooks, 1, _ptr(slots), o.ctypes.data)
        if rc != 0:
            errs.append(rc)

    ts = [threading.Thread(target=work, args=(int(bounds[i]), int(bounds[i + 1])))
          for i in range(threads) if bounds[i + 1] > bounds[i]]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    if errs:
        raise ValueError("oracle rejected its arguments")
    return out


def encode_rows(x, codebook, rows, sub_dim, n_centroids, dtype, *, codebook_stride=None,
                n_codebooks=1, group_len=None, group_map=None, want_top2=False):
    """Oracle result for the selected rows only (sampling at full size).

    Each selected row keeps the codebook slot its position in ``x`` gives it.
    """
    x, cb, n, stride, glen, gmap = _common(x, codebook, sub_dim, n_centroids,
                                           codebook_stride, n_codebooks, group_len, group_map)
    rows = np.asarray(rows, dtype=np.int64)
    xs = np.ascontiguousarray(x.reshape(n, sub_dim)[rows]).reshape(-1)
    g = rows // glen
    slots = (gmap[g] if gmap is not None else g).astype(np.int32)
    return _run(xs, cb, rows.size, sub_dim, n_centroids, dtype, stride, n_codebooks, 1,
                slots, want_top2)


def encode_top2(x, codebook, sub_dim, n_centroids, dtype, *, codebook_stride=None,
                n_codebooks=1, group_len=None, group_map=None):
    """(indices, best distance, second-best distance) per sub-vector."""
    x, cb, n, stride, glen, gmap = _common(x, codebook, sub_dim, n_centroids,
                                           codebook_stride, n_codebooks, group_len, group_map)
    return _run(x, cb, n, sub_dim, n_centroids, dtype, stride, n_codebooks, glen, gmap, True)


def _run(x, cb, n, sub_dim, n_centroids, dtype, stride, n_codebooks, glen, gmap, top2):
    lib = _load()
    out = np.empty(n, dtype=np.uint32)
    if not top2:
        if n:
            rc = lib.vqo_encode(_ptr(x), _ptr(cb), n, sub_dim, n_centroids, dtype, stride,
                                n_codebooks, glen, _ptr(gmap), _ptr(out))
            if rc != 0:
                raise ValueError("oracle rejected its arguments")
        return out
    best = np.empty(n, dtype=np.float32)
    second = np.empty(n, dtype=np.float32)
    if n:
        rc = lib.vqo_encode_top2(_ptr(x), _ptr(cb), n, sub_dim, n_centroids, dtype, stride,
                                 n_codebooks, glen, _ptr(gmap), _ptr(out), _ptr(best),
                                 _ptr(second))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
    return out, best, second


def decode(idx, codebook, sub_dim, n_centroids, dtype, *, codebook_stride=None,
           n_codebooks=1, group_len=None, group_map=None):
    """Gather codebook rows for ``idx`` (bits copied; bad index -> zero row)."""
    idx = np.ascontiguousarray(idx, dtype=np.uint32)
    n = idx.size
    cb = _u16(codebook).reshape(-1)
    stride = n_centroids * sub_dim if codebook_stride is None else codebook_stride
    glen = max(n, 1) if group_len is None else group_len
    gmap = None if group_map is None else np.ascontiguousarray(group_map, dtype=np.int32)
    out = np.empty(n * sub_dim, dtype=np.uint16)
    if n:
        rc = _load().vqo_decode(_ptr(idx), _ptr(cb), n, sub_dim, n_centroids, dtype, stride,
                                n_codebooks, glen, _ptr(gmap), _ptr(out))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
    return out.reshape(n, sub_dim)


def sqdist(xrow, crow, dtype) -> float:
    """fp32 squared distance of one sub-vector to one centroid."""
    xrow = _u16(xrow).reshape(-1)
    crow = _u16(crow).reshape(-1)
    if xrow.size != crow.size:
        raise ValueError("row lengths differ")
    return float(_load().vqo_sqdist(_ptr(xrow), _ptr(crow), xrow.size, dtype))


def sqdist_rows(x, codebook, rows, idx, sub_dim, dtype, *, codebook_stride=None,
                group_len=None, group_map=None, n_centroids=None):
    """fp32 oracle distance from row ``rows[k]`` of x to centroid ``idx[k]`` of its slot."""
    x = _u16(x).reshape(-1, sub_dim)
    cb = _u16(codebook).reshape(-1)
    n = x.shape[0]
    stride = (n_centroids * sub_dim) if codebook_stride is None else codebook_stride
    glen = max(n, 1) if group_len is None else group_len
    lib = _load()
    out = np.empty(len(rows), dtype=np.float32)
    for k, (r, c) in enumerate(zip(rows, idx)):
        g = int(r) // glen
        s = int(group_map[g]) if group_map is not None else g
        crow = np.ascontiguousarray(cb[s * stride + int(c) * sub_dim: s * stride + (int(c) + 1) * sub_dim])
        xr = np.ascontiguousarray(x[int(r)])
        out[k] = lib.vqo_sqdist(_ptr(xr), _ptr(crow), sub_dim, dtype)
    return out


def to_f32(bits: int, dtype: int) -> float:
    """The oracle's own fp16/bf16 -> fp32 widening of one value."""
    return float(_load().vqo_to_f32(int(bits) & 0xFFFF, dtype))


# ---------------------------------------------------------------------------
# Smoothing and packed codes (the steps either side of the search)
# ---------------------------------------------------------------------------

def _scale_arr(channel_scale):
    if channel_scale is None:
        return None
    return np.ascontiguousarray(channel_scale, dtype=np.float32).reshape(-1)


def smooth(x, sub_dim, dtype, *, channel_scale=None, head_dim=None, scale_stride=0,
           n_codebooks=1, group_len=None, group_map=None):
    """Smoothed fp32 sub-vectors [n, sub_dim]: each channel times its factor."""
    x = _u16(x).reshape(-1)
    n = x.size // sub_dim
    head_dim = sub_dim if head_dim is None else head_dim
    glen = max(n, 1) if group_len is None else group_len
    gmap = None if group_map is None else np.ascontiguousarray(group_map, dtype=np.int32)
    sc = _scale_arr(channel_scale)
    out = np.empty((n, sub_dim), dtype=np.float32)
    if n:
        rc = _load().vqo_smooth(_ptr(x), n, sub_dim, dtype, _ptr(sc), head_dim, scale_stride,
                                n_codebooks, glen, _ptr(gmap), _ptr(out))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
    return out


def encode_f32(xs, codebook, sub_dim, n_centroids, dtype, *, codebook_stride=None,
               n_codebooks=1, group_len=None, group_map=None, want_top2=False, threads=1):
    """The search over fp32 sub-vectors; (idx, best, second) with want_top2."""
    xs = np.ascontiguousarray(xs, dtype=np.float32).reshape(-1, sub_dim)
    n = xs.shape[0]
    cb = _u16(codebook).reshape(-1)
    stride = n_centroids * sub_dim if codebook_stride is None else codebook_stride
    glen = max(n, 1) if group_len is None else group_len
    gmap = None if group_map is None else np.ascontiguousarray(group_map, dtype=np.int32)
    lib = _load()
    out = np.empty(n, dtype=np.uint32)
    best = np.empty(n, dtype=np.float32) if want_top2 else None
    second = np.empty(n, dtype=np.float32) if want_top2 else None
    bounds = np.linspace(0, n, max(1, threads if n >= 4096 else 1) + 1).astype(np.int64)
    errs = []

    def work(lo, hi):
        g = np.arange(lo, hi, dtype=np.int64) // glen
        slots = (gmap[g] if gmap is not None else g).astype(np.int32)
        rc = lib.vqo_encode_f32(_ptr(xs[lo:hi]), _ptr(cb), hi - lo, sub_dim, n_centroids, dtype,
                                stride, n_codebooks, 1, _ptr(slots), out[lo:hi].ctypes.data,
                                None if best is None else best[lo:hi].ctypes.data,
                                None if second is None else second[lo:hi].ctypes.data)
        if rc != 0:
            errs.append(rc)

    ts = [threading.Thread(target=work, args=(int(bounds[i]), int(bounds[i + 1])))
          for i in range(len(bounds) - 1) if bounds[i + 1] > bounds[i]]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    if errs:
        raise ValueError("oracle rejected its arguments")
    return (out, best, second) if want_top2 else out


def packed_bytes(n: int, code_bits: int) -> int:
    return int(_load().vqo_packed_bytes(n, code_bits))


def pack(codes, code_bits: int) -> np.ndarray:
    """LSB-first bit stream of the low ``code_bits`` bits of every code."""
    codes = np.ascontiguousarray(codes, dtype=np.uint32).reshape(-1)
    out = np.empty(packed_bytes(codes.size, code_bits), dtype=np.uint8)
    if _load().vqo_pack(_ptr(codes), codes.size, code_bits, _ptr(out)) != 0:
        raise ValueError("oracle rejected its arguments")
    return out


def unpack(stream, n: int, code_bits: int) -> np.ndarray:
    stream = np.ascontiguousarray(stream, dtype=np.uint8).reshape(-1)
    if stream.size < packed_bytes(n, code_bits):
        raise ValueError("stream shorter than n codes")
    out = np.empty(n, dtype=np.uint32)
    if _load().vqo_unpack(_ptr(stream), n, code_bits, _ptr(out)) != 0:
        raise ValueError("oracle rejected its arguments")
    return out


def encode_packed(x, codebook, sub_dim, n_centroids, dtype, *, channel_scale=None,
                  head_dim=None, scale_stride=0, code_bits=8, codebook_stride=None,
                  n_codebooks=1, group_len=None, group_map=None, threads=1):
    """Smooth, search and pack: the stored code stream for raw keys ``x``.

    ``threads == 1`` is the single C routine; otherwise the same three steps
    run with the search sliced over threads (identical result).
    """
    x, cb, n, stride, glen, gmap = _common(x, codebook, sub_dim, n_centroids,
                                           codebook_stride, n_codebooks, group_len, group_map)
    head_dim = sub_dim if head_dim is None else head_dim
    sc = _scale_arr(channel_scale)
    if threads <= 1:
        out = np.empty(packed_bytes(n, code_bits), dtype=np.uint8)
        rc = _load().vqo_encode_packed(_ptr(x), _ptr(cb), n, sub_dim, n_centroids, dtype, stride,
                                       n_codebooks, glen, _ptr(gmap), _ptr(sc), head_dim,
                                       scale_stride, code_bits, _ptr(out))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return out
    if code_bits < 32 and n_centroids > (1 << code_bits):
        raise ValueError("oracle rejected its arguments")
    xs = smooth(x, sub_dim, dtype, channel_scale=sc, head_dim=head_dim, scale_stride=scale_stride,
                n_codebooks=n_codebooks, group_len=glen, group_map=gmap)
    idx = encode_f32(xs, cb, sub_dim, n_centroids, dtype, codebook_stride=stride,
                     n_codebooks=n_codebooks, group_len=glen, group_map=gmap, threads=threads)
    return pack(idx, code_bits)
