// vq_capi.cpp -- the extern "C" entry points declared in include/vq.h.
//
// Validates every argument on the host, before any HIP call, then hands the
// launch to the kernel launchers.  Nothing is allocated and no state is kept
// except the per-thread last HIP error.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vq.h"
#include "vq_launch.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

constexpr int64_t kMaxGrid = 0x7fffffffLL;
static_assert(VQ_MAX_HEAD_DIM == vqk::kMaxHeadDim, "factor staging limit");

vq_status check_common(const void *codebook, int64_t n, int32_t sub_dim, int32_t n_centroids,
                       vq_dtype dtype, int64_t codebook_stride, int64_t n_codebooks,
                       int64_t group_len, const int32_t *group_map, vqk::Layout *l) {
  if (sub_dim != 4 && sub_dim != 8) return VQ_ERR_UNSUPPORTED;
  if (dtype != VQ_F16 && dtype != VQ_BF16) return VQ_ERR_UNSUPPORTED;
  if (n_centroids > VQ_MAX_CENTROIDS) return VQ_ERR_UNSUPPORTED;
  if (n < 0 || n_centroids < 1 || n_codebooks < 1 || group_len < 1) return VQ_ERR_INVALID_ARG;
  if (n > INT64_MAX / 64) return VQ_ERR_INVALID_ARG;  // n * sub_dim * 2 bytes must not overflow
  const int64_t row_elems = static_cast<int64_t>(n_centroids) * sub_dim;
  if (n_codebooks > 1) {
    if (codebook_stride < row_elems) return VQ_ERR_INVALID_ARG;
    if (codebook_stride > (INT64_MAX - row_elems) / (n_codebooks - 1)) return VQ_ERR_INVALID_ARG;
  }
  const int64_t n_groups = n == 0 ? 0 : (n - 1) / group_len + 1;
  if (!group_map && n_groups > n_codebooks) return VQ_ERR_INVALID_ARG;
  if (n > 0 && !codebook) return VQ_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(codebook) % 2 != 0) return VQ_ERR_MISALIGNED;
  if (group_map && reinterpret_cast<uintptr_t>(group_map) % 4 != 0) return VQ_ERR_MISALIGNED;
  l->n = n;
  l->sub_dim = sub_dim;
  l->n_centroids = n_centroids;
  l->bf16 = dtype == VQ_BF16 ? 1 : 0;
  l->codebook_stride = n_codebooks > 1 ? codebook_stride : row_elems;
  l->n_codebooks = n_codebooks;
  l->group_len = group_len;
  l->n_groups = n_groups;
  return VQ_OK;
}

vq_status device_result(hipError_t e) {
  if (e == hipSuccess) return VQ_OK;
  g_last_hip_error = static_cast<int32_t>(e);
  return VQ_ERR_DEVICE;
}

// Encode launch for validated arguments with n > 0: the matrix-core kernel
// while the codebook slot fits its LDS plan, the direct kernel beyond.
vq_status launch(const void *x, const void *codebook, const int32_t *group_map, void *out,
                 const vqk::Layout &l, const vqk::Codes &codes, void *stream) {
  if (vqk::encode_grid(l) > kMaxGrid || vqk::encode_mfma_grid(l) > kMaxGrid)
    return VQ_ERR_INVALID_ARG;
  (void)hipGetLastError();  // drop a stale error so it is not reported as ours
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (vqk::encode_mfma_supported(l))
    return device_result(vqk::launch_encode_mfma(x, codebook, group_map, out, l, codes, s));
  return device_result(vqk::launch_encode(x, codebook, group_map, out, l, codes, s));
}

// Checks of the attention arguments shared by both entry points (all but the
// workspace); fills everything in *l except l->workspace.
vq_status check_attention(const void *q, const uint8_t *k_codes, const uint8_t *v_codes,
                          const void *k_codebook, const void *v_codebook, const float *k_scale,
                          const int32_t *kv_len, int32_t batch, int32_t n_q_heads,
                          int32_t n_kv_heads, int32_t head_dim, int32_t max_kv_len,
                          int32_t k_sub_dim, int32_t v_sub_dim, int32_t n_centroids,
                          vq_dtype dtype, int32_t window, float softmax_scale, float *out,
                          vqk::AttnLayout *l) {
  if ((k_sub_dim != 4 && k_sub_dim != 8) || (v_sub_dim != 4 && v_sub_dim != 8))
    return VQ_ERR_UNSUPPORTED;
  if (dtype != VQ_F16 && dtype != VQ_BF16) return VQ_ERR_UNSUPPORTED;
  if (n_centroids < 1 || n_centroids > 256) return VQ_ERR_UNSUPPORTED;  // 8-bit codes
  if (head_dim < 1 || head_dim > VQ_ATTN_MAX_HEAD_DIM) return VQ_ERR_UNSUPPORTED;
  // key rows are read four codes at a time; value sub-spaces map to lanes
  if (head_dim % (4 * k_sub_dim) != 0 || head_dim % v_sub_dim != 0) return VQ_ERR_UNSUPPORTED;
  if (batch < 0 || n_q_heads < 1 || n_kv_heads < 1 || max_kv_len < 0 || window < 0)
    return VQ_ERR_INVALID_ARG;
  if (n_q_heads % n_kv_heads != 0) return VQ_ERR_INVALID_ARG;
  if (n_q_heads / n_kv_heads > VQ_ATTN_MAX_GROUP) return VQ_ERR_UNSUPPORTED;
  if (!(softmax_scale == softmax_scale) || softmax_scale > 3.0e38f || softmax_scale < -3.0e38f)
    return VQ_ERR_INVALID_ARG;
  if (batch > 65535 || n_kv_heads > 65535) return VQ_ERR_INVALID_ARG;  // grid y / z
  if (static_cast<int64_t>(batch) * n_q_heads > kMaxGrid) return VQ_ERR_INVALID_ARG;
  if (batch == 0) return VQ_OK;
  if (!q || !out || !k_codebook || !v_codebook) return VQ_ERR_INVALID_ARG;
  if (max_kv_len > 0 && (!k_codes || !v_codes)) return VQ_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(q) % 2 || reinterpret_cast<uintptr_t>(k_codebook) % 2 ||
      reinterpret_cast<uintptr_t>(v_codebook) % 2 || reinterpret_cast<uintptr_t>(k_codes) % 4 ||
      reinterpret_cast<uintptr_t>(out) % 4 || reinterpret_cast<uintptr_t>(k_scale) % 4 ||
      reinterpret_cast<uintptr_t>(kv_len) % 4)
    return VQ_ERR_MISALIGNED;
  if (vqk::attention_lds_bytes(k_sub_dim, v_sub_dim, head_dim, n_q_heads / n_kv_heads) >
      160 * 1024)
    return VQ_ERR_UNSUPPORTED;
  l->q = q;
  l->k_codes = k_codes;
  l->v_codes = v_codes;
  l->k_codebook = k_codebook;
  l->v_codebook = v_codebook;
  l->k_scale = k_scale;
  l->kv_len = kv_len;
  l->out = out;
  l->workspace = nullptr;
  l->batch = batch;
  l->n_q_heads = n_q_heads;
  l->n_kv_heads = n_kv_heads;
  l->head_dim = head_dim;
  l->max_kv_len = max_kv_len;
  l->k_sub_dim = k_sub_dim;
  l->v_sub_dim = v_sub_dim;
  l->n_centroids = n_centroids;
  l->bf16 = dtype == VQ_BF16 ? 1 : 0;
  l->window = window;
  l->softmax_scale = softmax_scale;
  return VQ_OK;
}

}  // namespace

extern "C" {

vq_status vq_encode(const void *x, const void *codebook, int64_t n, int32_t sub_dim,
                    int32_t n_centroids, vq_dtype dtype, int64_t codebook_stride,
                    int64_t n_codebooks, int64_t group_len, const int32_t *group_map,
                    uint32_t *out_idx, void *stream) {
  vqk::Layout l;
  vq_status st = check_common(codebook, n, sub_dim, n_centroids, dtype, codebook_stride,
                              n_codebooks, group_len, group_map, &l);
  if (st != VQ_OK) return st;
  if (n > 0 && (!x || !out_idx)) return VQ_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(x) % (2 * sub_dim) != 0) return VQ_ERR_MISALIGNED;
  if (reinterpret_cast<uintptr_t>(out_idx) % 4 != 0) return VQ_ERR_MISALIGNED;
  if (n == 0) return VQ_OK;
  return launch(x, codebook, group_map, out_idx, l, vqk::plain_codes(l), stream);
}

vq_status vq_encode_packed(const void *x, const void *codebook, int64_t n, int32_t sub_dim,
                           int32_t n_centroids, vq_dtype dtype, int64_t codebook_stride,
                           int64_t n_codebooks, int64_t group_len, const int32_t *group_map,
                           const float *channel_scale, int32_t head_dim, int64_t scale_stride,
                           int32_t code_bits, void *out_codes, void *stream) {
  vqk::Layout l;
  vq_status st = check_common(codebook, n, sub_dim, n_centroids, dtype, codebook_stride,
                              n_codebooks, group_len, group_map, &l);
  if (st != VQ_OK) return st;
  if (code_bits < 1 || code_bits > 32) return VQ_ERR_INVALID_ARG;
  if (code_bits < 32 && n_centroids > (1 << code_bits)) return VQ_ERR_INVALID_ARG;
  if (channel_scale) {
    if (head_dim < sub_dim || head_dim % sub_dim != 0 || head_dim > VQ_MAX_HEAD_DIM)
      return VQ_ERR_INVALID_ARG;
    if (scale_stride < 0) return VQ_ERR_INVALID_ARG;
    if (n_codebooks > 1 && scale_stride > (INT64_MAX - head_dim) / (n_codebooks - 1))
      return VQ_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(channel_scale) % 4 != 0) return VQ_ERR_MISALIGNED;
  }
  if (n > 0 && (!x || !out_codes)) return VQ_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(x) % (2 * sub_dim) != 0) return VQ_ERR_MISALIGNED;
  if (reinterpret_cast<uintptr_t>(out_codes) % 4 != 0) return VQ_ERR_MISALIGNED;
  // a group boundary inside a 32-bit word of the stream would be written by
  // two workgroups
  if (l.n_groups > 1 && ((group_len % 32) * code_bits) % 32 != 0) return VQ_ERR_UNSUPPORTED;
  if (n == 0) return VQ_OK;
  const vqk::Codes codes{channel_scale, channel_scale ? scale_stride : 0,
                         channel_scale ? head_dim : sub_dim, code_bits};
  return launch(x, codebook, group_map, out_codes, l, codes, stream);
}

vq_status vq_decode(const uint32_t *idx, const void *codebook, int64_t n, int32_t sub_dim,
                    int32_t n_centroids, vq_dtype dtype, int64_t codebook_stride,
                    int64_t n_codebooks, int64_t group_len, const int32_t *group_map,
                    void *out_x, void *stream) {
  vqk::Layout l;
  vq_status st = check_common(codebook, n, sub_dim, n_centroids, dtype, codebook_stride,
                              n_codebooks, group_len, group_map, &l);
  if (st != VQ_OK) return st;
  if (n > 0 && (!idx || !out_x)) return VQ_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(idx) % 4 != 0) return VQ_ERR_MISALIGNED;
  if (reinterpret_cast<uintptr_t>(out_x) % 2 != 0) return VQ_ERR_MISALIGNED;
  if (n == 0) return VQ_OK;
  if ((n + 255) / 256 > kMaxGrid) return VQ_ERR_INVALID_ARG;
  (void)hipGetLastError();
  return device_result(
      vqk::launch_decode(idx, codebook, group_map, out_x, l, static_cast<hipStream_t>(stream)));
}

size_t vq_kmeans_workspace_bytes(int32_t sub_dim, int32_t n_centroids, int64_t n_codebooks,
                                 vq_dtype dtype) {
  if ((sub_dim != 4 && sub_dim != 8) || n_centroids < 1 || n_centroids > VQ_MAX_CENTROIDS ||
      n_codebooks < 1 || (dtype != VQ_F16 && dtype != VQ_BF16))
    return 0;
  return vqk::kmeans_workspace_bytes(sub_dim, n_centroids, n_codebooks, dtype == VQ_BF16);
}

vq_status vq_kmeans(const void *x, void *codebook, int64_t n, int32_t sub_dim,
                    int32_t n_centroids, vq_dtype dtype, int64_t codebook_stride,
                    int64_t n_codebooks, int64_t group_len, const int32_t *group_map,
                    int32_t iterations, uint32_t *out_idx, void *workspace,
                    size_t workspace_bytes, void *stream) {
  vqk::Layout l;
  vq_status st = check_common(codebook, n, sub_dim, n_centroids, dtype, codebook_stride,
                              n_codebooks, group_len, group_map, &l);
  if (st != VQ_OK) return st;
  if (iterations < 0) return VQ_ERR_INVALID_ARG;
  // exact int64 member sums (fp16) and limbs (bf16): at most 2^23 members per slot
  const int64_t per_slot = group_map ? n : (group_len < n ? group_len : n);
  if (per_slot > (int64_t(1) << 23)) return VQ_ERR_UNSUPPORTED;
  if (n == 0 || iterations == 0) return VQ_OK;
  if (!x || !out_idx || !workspace) return VQ_ERR_INVALID_ARG;
  const size_t need = vqk::kmeans_workspace_bytes(sub_dim, n_centroids, n_codebooks, dtype == VQ_BF16);
  if (need == 0 || workspace_bytes < need) return VQ_ERR_INVALID_ARG;  // 0: size overflows
  if (reinterpret_cast<uintptr_t>(x) % (2 * sub_dim) != 0 ||
      reinterpret_cast<uintptr_t>(out_idx) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(workspace) % 8 != 0)
    return VQ_ERR_MISALIGNED;
  if (vqk::encode_grid(l) > kMaxGrid || vqk::encode_mfma_grid(l) > kMaxGrid ||
      vqk::kmeans_grid(l) > kMaxGrid || n_codebooks * n_centroids * sub_dim / 32 + 1 > kMaxGrid ||
      // the clear kernel: one thread per int64 word of the sums
      static_cast<int64_t>(need / 8 / 256) + 1 > kMaxGrid)
    return VQ_ERR_INVALID_ARG;
  (void)hipGetLastError();
  return device_result(vqk::launch_kmeans(x, codebook, group_map, out_idx, l, iterations,
                                          workspace, static_cast<hipStream_t>(stream)));
}

size_t vq_attention_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t head_dim,
                                    int32_t max_kv_len) {
  if (batch < 0 || n_q_heads < 0 || head_dim < 0 || max_kv_len < 0) return 0;
  uint64_t r = 0;
  if (__builtin_mul_overflow(static_cast<uint64_t>(batch), static_cast<uint64_t>(n_q_heads), &r) ||
      __builtin_mul_overflow(r, static_cast<uint64_t>(vqk::attention_chunks(max_kv_len)), &r) ||
      __builtin_mul_overflow(r, (static_cast<uint64_t>(head_dim) + 2) * sizeof(float), &r) ||
      r > static_cast<uint64_t>(INT64_MAX))
    return 0;  // does not fit: the decode calls reject such sizes
  return static_cast<size_t>(r);
}

vq_status vq_attention_decode(const void *q, const uint8_t *k_codes, const uint8_t *v_codes,
                              const void *k_codebook, const void *v_codebook,
                              const float *k_scale, const int32_t *kv_len, int32_t batch,
                              int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                              int32_t max_kv_len, int32_t k_sub_dim, int32_t v_sub_dim,
                              int32_t n_centroids, vq_dtype dtype, int32_t window,
                              float softmax_scale, float *out, void *workspace,
                              size_t workspace_bytes, void *stream) {
  vqk::AttnLayout l;
  const vq_status st = check_attention(q, k_codes, v_codes, k_codebook, v_codebook, k_scale,
                                       kv_len, batch, n_q_heads, n_kv_heads, head_dim, max_kv_len,
                                       k_sub_dim, v_sub_dim, n_centroids, dtype, window,
                                       softmax_scale, out, &l);
  if (st != VQ_OK || batch == 0) return st;
  if (!workspace) return VQ_ERR_INVALID_ARG;
  const size_t need = vq_attention_workspace_bytes(batch, n_q_heads, head_dim, max_kv_len);
  if (need == 0 || workspace_bytes < need) return VQ_ERR_INVALID_ARG;  // 0: size overflows
  if (reinterpret_cast<uintptr_t>(workspace) % 4) return VQ_ERR_MISALIGNED;
  l.workspace = static_cast<float *>(workspace);
  (void)hipGetLastError();
  return device_result(vqk::launch_attention(l, static_cast<hipStream_t>(stream)));
}

vq_status vq_attention_decode_static(const void *q, const uint8_t *k_codes,
                                     const uint8_t *v_codes, const void *k_codebook,
                                     const void *v_codebook, const float *k_scale,
                                     const int32_t *kv_len, int32_t batch, int32_t n_q_heads,
                                     int32_t n_kv_heads, int32_t head_dim, int32_t max_kv_len,
                                     int32_t k_sub_dim, int32_t v_sub_dim, int32_t n_centroids,
                                     vq_dtype dtype, int32_t window, float softmax_scale,
                                     float *out, void *stream) {
  vqk::AttnLayout l;
  const vq_status st = check_attention(q, k_codes, v_codes, k_codebook, v_codebook, k_scale,
                                       kv_len, batch, n_q_heads, n_kv_heads, head_dim, max_kv_len,
                                       k_sub_dim, v_sub_dim, n_centroids, dtype, window,
                                       softmax_scale, out, &l);
  if (st != VQ_OK || batch == 0) return st;
  const size_t need = vq_attention_workspace_bytes(batch, n_q_heads, head_dim, max_kv_len);
  if (need == 0) return VQ_ERR_INVALID_ARG;  // the size overflows
  if (need > VQ_ATTN_STATIC_SCRATCH_BYTES) return VQ_ERR_TOO_LARGE;
  void *scratch = nullptr;
  (void)hipGetLastError();
  const hipError_t e = vqk::attention_static_scratch(&scratch);
  if (e != hipSuccess) return device_result(e);
  l.workspace = static_cast<float *>(scratch);
  return device_result(vqk::launch_attention(l, static_cast<hipStream_t>(stream)));
}

const char *vq_status_str(int32_t status) {
  switch (status) {
    case VQ_OK: return "ok";
    case VQ_ERR_INVALID_ARG: return "invalid argument";
    case VQ_ERR_UNSUPPORTED:
      return "unsupported sub_dim, dtype, n_centroids or packed group layout";
    case VQ_ERR_MISALIGNED: return "misaligned pointer";
    case VQ_ERR_DEVICE: return "HIP launch failed";
    case VQ_ERR_TOO_LARGE:
      return "the call needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

int32_t vq_last_hip_error(void) { return g_last_hip_error; }

int32_t vq_abi_version(void) { return VQ_ABI_VERSION; }

}  // extern "C"
