"""MI355X-native product-VQ KV-cache encode (VecInfer ``quantize_vq``).

Thin Python binding over the C ABI of ``libvq.so`` (declared in
``include/vq.h``): every step of the computation runs in the library's HIP
kernels; this module only checks tensor shapes and passes device pointers,
sizes and the current HIP stream.  There is no CPU fallback: if the library
is missing or cannot be loaded, importing this package raises.

    import torch, product_vq_kv_amd as vq
    idx = vq.encode(keys_subvectors, codebook)          # uint32 [N]
    rec = vq.decode(idx, codebook)                      # gather, for checking
    codes = vq.encode_packed(keys, codebook, channel_scale=f, code_bits=8)  # uint8 stream
    o = vq.attention_decode(q, k_codes, v_codes, k_cb, v_cb, k_scale=f)    # fp32 [B, Hq, D]

``encode`` follows the encode step of VecInfer product vector quantization as
the VeloxQuant-MLX blog post "I Wrote a Metal Kernel to Stop My Mac From
OOMing" describes it (sections "What quantize_vq Was Doing Wrong" and "The
Kernel: 18 Lines of MSL"): the index of the nearest centroid by squared L2
distance, evaluated in fp32, ties to the lowest index.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # loads the HIP runtime that libvq.so binds to (same soname)

__all__ = ["encode", "decode", "encode_packed", "packed_bytes", "attention_decode",
           "attention_workspace_bytes", "kmeans", "kmeans_workspace_bytes", "kmeans_raw", "encode_raw", "decode_raw", "encode_packed_raw",
           "attention_decode_raw", "attention_decode_static", "attention_decode_static_raw",
           "ATTN_STATIC_SCRATCH_BYTES", "VQError", "lib", "LIB_PATH", "F16", "BF16", "BAD_SLOT",
           "MAX_CENTROIDS", "MAX_HEAD_DIM", "STATUS"]

F16 = 0
BF16 = 1
BAD_SLOT = 0xFFFFFFFF
MAX_CENTROIDS = 65536
MAX_HEAD_DIM = 4096
ATTN_STATIC_SCRATCH_BYTES = 32 << 20
STATUS = {0: "VQ_OK", -1: "VQ_ERR_INVALID_ARG", -2: "VQ_ERR_UNSUPPORTED",
          -3: "VQ_ERR_MISALIGNED", -4: "VQ_ERR_DEVICE", -5: "VQ_ERR_TOO_LARGE"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python product_vq_kv_amd/build.py` "
                      "(there is no CPU fallback)")

lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
lib.vq_encode.argtypes = [_p, _p, _i64, _i32, _i32, _i32, _i64, _i64, _i64, _p, _p, _p]
lib.vq_encode.restype = _i32
lib.vq_encode_packed.argtypes = [_p, _p, _i64, _i32, _i32, _i32, _i64, _i64, _i64, _p, _p, _i32,
                                 _i64, _i32, _p, _p]
lib.vq_encode_packed.restype = _i32
lib.vq_attention_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32]
lib.vq_attention_workspace_bytes.restype = ctypes.c_size_t
lib.vq_attention_decode.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32,
                                    _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _p, _p,
                                    ctypes.c_size_t, _p]
lib.vq_attention_decode.restype = _i32
lib.vq_attention_decode_static.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32,
                                           _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_float,
                                           _p, _p]
lib.vq_attention_decode_static.restype = _i32
lib.vq_kmeans_workspace_bytes.argtypes = [_i32, _i32, _i64, _i32]
lib.vq_kmeans_workspace_bytes.restype = ctypes.c_size_t
lib.vq_kmeans.argtypes = [_p, _p, _i64, _i32, _i32, _i32, _i64, _i64, _i64, _p, _i32, _p, _p,
                          ctypes.c_size_t, _p]
lib.vq_kmeans.restype = _i32
lib.vq_decode.argtypes = [_p, _p, _i64, _i32, _i32, _i32, _i64, _i64, _i64, _p, _p, _p]
lib.vq_decode.restype = _i32
lib.vq_status_str.argtypes = [_i32]
lib.vq_status_str.restype = ctypes.c_char_p
lib.vq_last_hip_error.argtypes = []
lib.vq_last_hip_error.restype = _i32
lib.vq_abi_version.argtypes = []
lib.vq_abi_version.restype = _i32


class VQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.vq_status_str(status).decode()
        extra = ""
        if status == -4:
            extra = f" (hipError {lib.vq_last_hip_error()})"
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}{extra}")


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise VQError(rc, where)


def encode_raw(x_ptr: int, codebook_ptr: int, n: int, sub_dim: int, n_centroids: int,
               dtype: int, codebook_stride: int, n_codebooks: int, group_len: int,
               group_map_ptr: Optional[int], out_ptr: int, stream: Optional[int]) -> None:
    """Direct call of ``vq_encode`` with integer pointers (raises on error)."""
    _check(lib.vq_encode(x_ptr, codebook_ptr, n, sub_dim, n_centroids, dtype, codebook_stride,
                         n_codebooks, group_len, group_map_ptr, out_ptr, stream), "vq_encode")


def encode_packed_raw(x_ptr: int, codebook_ptr: int, n: int, sub_dim: int, n_centroids: int,
                      dtype: int, codebook_stride: int, n_codebooks: int, group_len: int,
                      group_map_ptr: Optional[int], scale_ptr: Optional[int], head_dim: int,
                      scale_stride: int, code_bits: int, out_ptr: int,
                      stream: Optional[int]) -> None:
    """Direct call of ``vq_encode_packed`` with integer pointers (raises on error)."""
    _check(lib.vq_encode_packed(x_ptr, codebook_ptr, n, sub_dim, n_centroids, dtype,
                                codebook_stride, n_codebooks, group_len, group_map_ptr, scale_ptr,
                                head_dim, scale_stride, code_bits, out_ptr, stream),
           "vq_encode_packed")


def decode_raw(idx_ptr: int, codebook_ptr: int, n: int, sub_dim: int, n_centroids: int,
               dtype: int, codebook_stride: int, n_codebooks: int, group_len: int,
               group_map_ptr: Optional[int], out_ptr: int, stream: Optional[int]) -> None:
    """Direct call of ``vq_decode`` with integer pointers (raises on error)."""
    _check(lib.vq_decode(idx_ptr, codebook_ptr, n, sub_dim, n_centroids, dtype, codebook_stride,
                         n_codebooks, group_len, group_map_ptr, out_ptr, stream), "vq_decode")


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float16:
        return F16
    if t == torch.bfloat16:
        return BF16
    raise TypeError(f"elements must be float16 or bfloat16, got {t}")


def _codebook_layout(codebook: torch.Tensor):
    """(n_codebooks, n_centroids, sub_dim, stride) of a [.., n_c, sd] tensor."""
    if codebook.dim() == 2:
        n_c, sd = codebook.shape
        if not codebook.is_contiguous():
            raise ValueError("codebook must be contiguous")
        return 1, n_c, sd, n_c * sd
    if codebook.dim() == 3:
        k, n_c, sd = codebook.shape
        if codebook.stride(2) != 1 or codebook.stride(1) != sd:
            raise ValueError("each codebook slot must be a contiguous [n_centroids, sub_dim] block")
        return k, n_c, sd, codebook.stride(0)
    raise ValueError("codebook must be [n_centroids, sub_dim] or [slots, n_centroids, sub_dim]")


def _stream_of(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _group_map_ptr(group_map, n: int, group_len: int) -> Optional[int]:
    if group_map is None:
        return None
    if group_map.dtype != torch.int32 or not group_map.is_cuda or not group_map.is_contiguous():
        raise ValueError("group_map must be a contiguous int32 device tensor")
    if group_map.numel() < -(-n // group_len):
        raise ValueError("group_map needs one entry per group")
    return group_map.data_ptr()


def _keys(x: torch.Tensor, codebook: torch.Tensor):
    """(dtype code, n_codebooks, n_centroids, sub_dim, stride, n) for encode."""
    if not (x.is_cuda and codebook.is_cuda):
        raise ValueError("x and codebook must be device tensors (no CPU path exists)")
    dt = _dtype_code(x.dtype)
    if codebook.dtype != x.dtype:
        raise TypeError("x and codebook must have the same dtype")
    k, n_c, sd, stride = _codebook_layout(codebook)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if x.numel() % sd:
        raise ValueError("x's element count is not a multiple of sub_dim")
    return dt, k, n_c, sd, stride, x.numel() // sd


def packed_bytes(n: int, code_bits: int) -> int:
    """Length of the code stream of n codes of code_bits bits."""
    return (n * code_bits + 7) // 8


def encode_packed(x: torch.Tensor, codebook: torch.Tensor, *,
                  channel_scale: Optional[torch.Tensor] = None, head_dim: Optional[int] = None,
                  code_bits: int = 8, group_len: Optional[int] = None,
                  group_map: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Smoothed, packed encode: a uint8 code stream of ceil(N*code_bits/8) bytes.

    channel_scale  fp32 factors [head_dim] (one vector) or [slots, head_dim]
                   (one per codebook slot); every key channel is multiplied by
                   its factor before the search.  None: no smoothing.
    head_dim       channels per key; defaults to the factors' last dimension,
                   or to x's last dimension.
    code_bits      bits per code (n_centroids <= 2^code_bits); codes are
                   packed back to back, least significant bit first.
    Other arguments as for ``encode``.
    """
    dt, k, n_c, sd, stride, n = _keys(x, codebook)
    if group_len is None:
        group_len = max(n, 1)
    gptr = _group_map_ptr(group_map, n, group_len)
    sptr, sstride = None, 0
    if channel_scale is not None:
        if (channel_scale.dtype != torch.float32 or not channel_scale.is_cuda
                or channel_scale.stride(-1) != 1 or channel_scale.dim() not in (1, 2)):
            raise ValueError("channel_scale must be a float32 device tensor [head_dim] or "
                             "[slots, head_dim] with unit channel stride")
        hd = channel_scale.shape[-1]
        if head_dim is not None and head_dim != hd:
            raise ValueError("head_dim differs from channel_scale's last dimension")
        head_dim = hd
        if channel_scale.dim() == 2:
            if channel_scale.shape[0] < k:
                raise ValueError("channel_scale needs one factor vector per codebook slot")
            sstride = channel_scale.stride(0)
        sptr = channel_scale.data_ptr()
    if head_dim is None:
        head_dim = x.shape[-1] if x.dim() > 1 else sd
    nbytes = packed_bytes(n, code_bits)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    elif out.dtype != torch.uint8 or out.numel() < nbytes or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous uint8 tensor of at least {nbytes} bytes")
    encode_packed_raw(x.data_ptr(), codebook.data_ptr(), n, sd, n_c, dt, stride, k, group_len,
                      gptr, sptr, head_dim, sstride, code_bits, out.data_ptr(),
                      _stream_of(x.device, stream))
    return out


def encode(x: torch.Tensor, codebook: torch.Tensor, *, group_len: Optional[int] = None,
           group_map: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
           stream=None) -> torch.Tensor:
    """Nearest-centroid index of every sub-vector, as a uint32 tensor [N].

    x         fp16/bf16 CUDA tensor whose last dimension is a multiple of
              sub_dim (e.g. keys [..., head_dim] or sub-vectors [N, sub_dim]);
              it is viewed as [N, sub_dim] and must be contiguous.
    codebook  [n_centroids, sub_dim] or [slots, n_centroids, sub_dim], same dtype.
    group_len sub-vectors per group when several codebook slots are used:
              sub-vector n uses slot group_map[n // group_len] (or n // group_len).
    """
    dt, k, n_c, sd, stride, n = _keys(x, codebook)
    if group_len is None:
        group_len = max(n, 1)
    gptr = _group_map_ptr(group_map, n, group_len)
    if out is None:
        out = torch.empty(n, dtype=torch.uint32, device=x.device)
    elif out.dtype != torch.uint32 or out.numel() != n or not out.is_contiguous():
        raise ValueError("out must be a contiguous uint32 tensor with one entry per sub-vector")
    encode_raw(x.data_ptr(), codebook.data_ptr(), n, sd, n_c, dt, stride, k, group_len, gptr,
               out.data_ptr(), _stream_of(x.device, stream))
    return out


def decode(idx: torch.Tensor, codebook: torch.Tensor, *, group_len: Optional[int] = None,
           group_map: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
           stream=None) -> torch.Tensor:
    """Gather codebook rows by index: [N] uint32 -> [N, sub_dim] (checking aid)."""
    if not (idx.is_cuda and codebook.is_cuda):
        raise ValueError("idx and codebook must be device tensors")
    if idx.dtype not in (torch.uint32, torch.int32) or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous uint32 tensor")
    dt = _dtype_code(codebook.dtype)
    k, n_c, sd, stride = _codebook_layout(codebook)
    n = idx.numel()
    if group_len is None:
        group_len = max(n, 1)
    gptr = _group_map_ptr(group_map, n, group_len)
    if out is None:
        out = torch.empty((n, sd), dtype=codebook.dtype, device=idx.device)
    elif out.dtype != codebook.dtype or out.numel() != n * sd or not out.is_contiguous():
        raise ValueError("out must be a contiguous [N, sub_dim] tensor of the codebook dtype")
    decode_raw(idx.data_ptr(), codebook.data_ptr(), n, sd, n_c, dt, stride, k, group_len, gptr,
               out.data_ptr(), _stream_of(idx.device, stream))
    return out


def attention_workspace_bytes(batch: int, n_q_heads: int, head_dim: int, max_kv_len: int) -> int:
    return int(lib.vq_attention_workspace_bytes(batch, n_q_heads, head_dim, max_kv_len))


def attention_decode_raw(q_ptr, k_codes_ptr, v_codes_ptr, k_cb_ptr, v_cb_ptr, k_scale_ptr,
                         kv_len_ptr, batch, n_q_heads, n_kv_heads, head_dim, max_kv_len,
                         k_sub_dim, v_sub_dim, n_centroids, dtype, window, softmax_scale,
                         out_ptr, ws_ptr, ws_bytes, stream) -> None:
    """Direct call of ``vq_attention_decode`` with integer pointers (raises on error)."""
    _check(lib.vq_attention_decode(q_ptr, k_codes_ptr, v_codes_ptr, k_cb_ptr, v_cb_ptr,
                                   k_scale_ptr, kv_len_ptr, batch, n_q_heads, n_kv_heads,
                                   head_dim, max_kv_len, k_sub_dim, v_sub_dim, n_centroids, dtype,
                                   window, softmax_scale, out_ptr, ws_ptr, ws_bytes, stream),
           "vq_attention_decode")


def attention_decode_static_raw(q_ptr, k_codes_ptr, v_codes_ptr, k_cb_ptr, v_cb_ptr,
                                k_scale_ptr, kv_len_ptr, batch, n_q_heads, n_kv_heads, head_dim,
                                max_kv_len, k_sub_dim, v_sub_dim, n_centroids, dtype, window,
                                softmax_scale, out_ptr, stream) -> None:
    """Direct call of ``vq_attention_decode_static`` (raises on error)."""
    _check(lib.vq_attention_decode_static(q_ptr, k_codes_ptr, v_codes_ptr, k_cb_ptr, v_cb_ptr,
                                          k_scale_ptr, kv_len_ptr, batch, n_q_heads, n_kv_heads,
                                          head_dim, max_kv_len, k_sub_dim, v_sub_dim,
                                          n_centroids, dtype, window, softmax_scale, out_ptr,
                                          stream),
           "vq_attention_decode_static")


def attention_decode_static(q: torch.Tensor, k_codes: torch.Tensor, v_codes: torch.Tensor,
                            k_codebook: torch.Tensor, v_codebook: torch.Tensor, *,
                            k_scale: Optional[torch.Tensor] = None,
                            kv_len: Optional[torch.Tensor] = None, window: int = 0,
                            softmax_scale: Optional[float] = None, out: torch.Tensor,
                            stream=None) -> torch.Tensor:
    """``attention_decode`` through the allocation-free entry point: the
    caller passes `out` (fp32 [B, Hq, D]); the chunk partials use the
    library's static per-GPU scratch, so nothing is allocated."""
    return attention_decode(q, k_codes, v_codes, k_codebook, v_codebook, k_scale=k_scale,
                            kv_len=kv_len, window=window, softmax_scale=softmax_scale, out=out,
                            stream=stream, _static=True)


def attention_decode(q: torch.Tensor, k_codes: torch.Tensor, v_codes: torch.Tensor,
                     k_codebook: torch.Tensor, v_codebook: torch.Tensor, *,
                     k_scale: Optional[torch.Tensor] = None,
                     kv_len: Optional[torch.Tensor] = None, window: int = 0,
                     softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None,
                     _static: bool = False) -> torch.Tensor:
    """Decode attention from 8-bit VQ codes: fp32 [B, Hq, D].

    q           fp16/bf16 [B, Hq, D]
    k_codes     uint8 [B, Hkv, S, D / k_sub_dim]; v_codes uint8 [B, Hkv, S, D / v_sub_dim]
    k_codebook  [Hkv, n_c, k_sub_dim] (same dtype as q); v_codebook [Hkv, n_c, v_sub_dim]
    k_scale     fp32 [Hkv, D] smoothing factors the keys were encoded with, or None
    kv_len      int32 [B] attended prefix per sequence (None: all S)
    window      attend to the last `window` tokens only (0: all)
    softmax_scale  default 1 / sqrt(D)
    workspace   optional uint8 device tensor of attention_workspace_bytes(...) bytes
    """
    for t in (q, k_codes, v_codes, k_codebook, v_codebook):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous device tensors")
    dt = _dtype_code(q.dtype)
    if k_codebook.dtype != q.dtype or v_codebook.dtype != q.dtype:
        raise TypeError("codebooks must have q's dtype")
    if k_codes.dtype != torch.uint8 or v_codes.dtype != torch.uint8:
        raise TypeError("codes must be uint8")
    B, Hq, D = q.shape
    _, Hkv, S, nk = k_codes.shape
    hkv2, n_c, sdk = k_codebook.shape
    _, _, sdv = v_codebook.shape
    if (k_codes.shape[:3] != (B, Hkv, S) or v_codes.shape[:3] != (B, Hkv, S)
            or nk * sdk != D or v_codes.shape[3] * sdv != D or hkv2 != Hkv
            or tuple(v_codebook.shape[:2]) != (Hkv, n_c)):
        raise ValueError("inconsistent shapes")
    sptr = None
    if k_scale is not None:
        if (k_scale.dtype != torch.float32 or not k_scale.is_cuda or not k_scale.is_contiguous()
                or tuple(k_scale.shape) != (Hkv, D)):
            raise ValueError("k_scale must be a contiguous fp32 device tensor [Hkv, D]")
        sptr = k_scale.data_ptr()
    lptr = None
    if kv_len is not None:
        if kv_len.dtype != torch.int32 or not kv_len.is_cuda or kv_len.numel() != B:
            raise ValueError("kv_len must be an int32 device tensor [B]")
        lptr = kv_len.data_ptr()
    if softmax_scale is None:
        softmax_scale = 1.0 / float(D) ** 0.5
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (B, Hq, D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor [B, Hq, D]")
    if _static:
        attention_decode_static_raw(q.data_ptr(), k_codes.data_ptr(), v_codes.data_ptr(),
                                    k_codebook.data_ptr(), v_codebook.data_ptr(), sptr, lptr, B,
                                    Hq, Hkv, D, S, sdk, sdv, n_c, dt, window, softmax_scale,
                                    out.data_ptr(), _stream_of(q.device, stream))
        return out
    need = attention_workspace_bytes(B, Hq, D, S)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    attention_decode_raw(q.data_ptr(), k_codes.data_ptr(), v_codes.data_ptr(),
                         k_codebook.data_ptr(), v_codebook.data_ptr(), sptr, lptr, B, Hq, Hkv, D,
                         S, sdk, sdv, n_c, dt, window, softmax_scale, out.data_ptr(),
                         workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                         _stream_of(q.device, stream))
    return out


def kmeans_workspace_bytes(sub_dim: int, n_centroids: int, n_codebooks: int = 1,
                           dtype: int = F16) -> int:
    return int(lib.vq_kmeans_workspace_bytes(sub_dim, n_centroids, n_codebooks, dtype))


def kmeans_raw(x_ptr, codebook_ptr, n, sub_dim, n_centroids, dtype, codebook_stride, n_codebooks,
               group_len, group_map_ptr, iterations, out_ptr, ws_ptr, ws_bytes, stream) -> None:
    """Direct call of ``vq_kmeans`` with integer pointers (raises on error)."""
    _check(lib.vq_kmeans(x_ptr, codebook_ptr, n, sub_dim, n_centroids, dtype, codebook_stride,
                         n_codebooks, group_len, group_map_ptr, iterations, out_ptr, ws_ptr,
                         ws_bytes, stream), "vq_kmeans")


def kmeans(x: torch.Tensor, codebook: torch.Tensor, iterations: int, *,
           group_len: Optional[int] = None, group_map: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           stream=None) -> torch.Tensor:
    """Lloyd K-means on the device: `codebook` (fp16 or bf16, [n_c, sd] or
    [slots, n_c, sd]) is updated in place; returns the last assignment
    (uint32 [N])."""
    dt, k, n_c, sd, stride, n = _keys(x, codebook)
    if group_len is None:
        group_len = max(n, 1)
    gptr = _group_map_ptr(group_map, n, group_len)
    if out is None:
        out = torch.empty(n, dtype=torch.uint32, device=x.device)
    elif out.dtype != torch.uint32 or out.numel() != n or not out.is_contiguous():
        raise ValueError("out must be a contiguous uint32 tensor with one entry per sub-vector")
    need = kmeans_workspace_bytes(sd, n_c, k, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=x.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    kmeans_raw(x.data_ptr(), codebook.data_ptr(), n, sd, n_c, dt, stride, k, group_len, gptr,
               iterations, out.data_ptr(), workspace.data_ptr(),
               workspace.numel() * workspace.element_size(), _stream_of(x.device, stream))
    return out
