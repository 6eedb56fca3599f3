/*
 * vq.h -- C ABI of the MI355X (gfx950) product-VQ encode library, libvq.so.
 *
 * The operation is the encode step of VecInfer product vector quantization
 * as described in the VeloxQuant-MLX blog post "I Wrote a Metal Kernel to
 * Stop My Mac From OOMing":
 *   - section "What Even Is a KV Cache And Why Should You Care" (steps 1-3):
 *     a key is cut into sub-vectors of length sub_dim and each sub-vector is
 *     replaced by the index of its nearest codebook centroid;
 *   - section "What quantize_vq Was Doing Wrong": nearest = argmin over the
 *     centroids of the summed squared component differences;
 *   - section "The Kernel: 18 Lines of MSL": fp32 promotion of every
 *     component, squared distance accumulated in one fp32 value, strict-<
 *     running argmin from (+infinity, index 0), one uint32 per sub-vector.
 * Fixed arithmetic (identical to the CPU oracle the library is tested
 * against): per component d = fp32(x_i) - fp32(c_i) rounded once, then
 * dist = fma(d, d, dist), components in order i = 0 .. sub_dim-1 from +0.
 * Ties go to the lowest index; NaN distances never win; a sub-vector whose
 * distances are all +inf or NaN gets index 0.
 *
 * Batched caches: sub-vector n belongs to group g = n / group_len and is
 * encoded against codebook slot k = group_map ? group_map[g] : g, which
 * starts at element k * codebook_stride of the codebook buffer.  One launch
 * covers every group (e.g. one codebook per (layer, kv head) with
 * group_len = tokens * head_dim / sub_dim).  Batching all heads into one call
 * follows the residual-VQ benchmark post's section "The Throughput Problem
 * (and How We Solved It)", change 1.
 *
 * Memory: every pointer is device memory owned by the caller.  The library
 * allocates nothing, keeps no state between calls and is re-entrant.  Calls
 * are asynchronous on `stream` (a hipStream_t; NULL = the default stream):
 * results are valid once the stream has been synchronised.
 *
 * Errors: every argument check happens on the host before any HIP call; a
 * rejected call launches nothing and writes nothing.  Launch failures return
 * VQ_ERR_DEVICE and the HIP error code is kept (per host thread) for
 * vq_last_hip_error().  Device memory the kernels read is never read out of
 * bounds for arguments that pass the checks, given buffers of the documented
 * sizes.
 */
#ifndef PRODUCT_VQ_KV_AMD_VQ_H
#define PRODUCT_VQ_KV_AMD_VQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    VQ_F16 = 0,  /* IEEE binary16 elements */
    VQ_BF16 = 1  /* bfloat16 elements */
} vq_dtype;

typedef enum {
    VQ_OK = 0,
    VQ_ERR_INVALID_ARG = -1, /* null pointer with n > 0, bad count, stride or group layout */
    VQ_ERR_UNSUPPORTED = -2, /* sub_dim not 4 or 8, unknown dtype, n_centroids > 65536,
                                packed groups not ending on a 32-bit word of the stream */
    VQ_ERR_MISALIGNED = -3,  /* x not aligned to 2*sub_dim bytes, codebook to 2,
                                idx/out/codes/factors to 4 */
    VQ_ERR_DEVICE = -4,      /* the HIP launch failed; see vq_last_hip_error() */
    VQ_ERR_TOO_LARGE = -5    /* the call needs more scratch than the static buffer of
                                vq_attention_decode_static holds */
} vq_status;

/* Index written for every sub-vector of a group whose group_map entry is not
 * a valid slot (outside [0, n_codebooks)). */
#define VQ_BAD_SLOT 0xFFFFFFFFu
#define VQ_MAX_CENTROIDS 65536
#define VQ_MAX_HEAD_DIM 4096
#define VQ_ATTN_MAX_HEAD_DIM 256
#define VQ_ATTN_MAX_GROUP 8
#define VQ_KMEANS_MAX_SLOT_ROWS (1 << 23)
#define VQ_ATTN_STATIC_SCRATCH_BYTES (32u << 20)
#define VQ_ABI_VERSION 6

/*
 * vq_encode -- nearest-centroid index of every sub-vector.
 *
 *   x            device, [n][sub_dim] elements of `dtype`, row-major, aligned
 *                to 2*sub_dim bytes.
 *   codebook     device, n_codebooks slots; slot k holds [n_centroids][sub_dim]
 *                elements of `dtype` at element offset k*codebook_stride.
 *   n            number of sub-vectors (>= 0; 0 returns VQ_OK, no launch).
 *   sub_dim      4 or 8.
 *   n_centroids  1 .. 65536.
 *   codebook_stride  elements between slots; >= n_centroids*sub_dim when
 *                n_codebooks > 1 (ignored when n_codebooks == 1).
 *   n_codebooks  >= 1.
 *   group_len    sub-vectors per group, >= 1 (group_len >= n: one group).
 *   group_map    device int32 [ceil(n/group_len)] group -> slot, or NULL for
 *                slot = group (then ceil(n/group_len) <= n_codebooks is
 *                checked on the host).  Entries outside [0, n_codebooks)
 *                make that group's indices VQ_BAD_SLOT.
 *   out_idx      device, [n] uint32, aligned to 4 bytes.
 *   stream       hipStream_t or NULL.
 */
vq_status vq_encode(const void *x, const void *codebook, int64_t n, int32_t sub_dim,
                    int32_t n_centroids, vq_dtype dtype, int64_t codebook_stride,
                    int64_t n_codebooks, int64_t group_len, const int32_t *group_map,
                    uint32_t *out_idx, void *stream);

/*
 * vq_encode_packed -- vq_encode with the two steps either side of the search
 * in a VecInfer key cache fused in: per-channel smoothing on load and packed
 * b-bit codes on store.
 *
 * Smoothing: VeloxQuant-MLX blog, post introducing the library's nine
 * algorithms, section "VecInfer -- 16x with Metal acceleration" (a scale per
 * channel handles the outlier channels that defeat plain VQ), and "I Wrote a
 * Metal Kernel to Stop My Mac From OOMing", section "How to Use This Today"
 * (the cache takes calibrated smooth factors).  Every channel of a key is
 * multiplied by its fp32 factor (one IEEE multiply, round to nearest even)
 * and the search of vq_encode runs on those fp32 values with the same
 * arithmetic and tie rule.  Smoothing by a divisor s is the factor 1/s (the
 * matching query transform, q_tilde of the post's section "What's Next:
 * Phase 2", is then q * s).  Keys are laid out [..][tokens][head_dim] and cut
 * along head_dim, so component i of sub-vector r is channel
 * (r mod (head_dim/sub_dim)) * sub_dim + i, and sub-vector r uses the factor
 * vector of its codebook slot k: channel_scale + k * scale_stride.
 *
 * Codes: "I Wrote a Metal Kernel ...", section "What Even Is a KV Cache And
 * Why Should You Care" (16 indices of 8 bits per 128-dim key: 16x), and "How
 * I built VeloxQuant-MLX -- KV cache compression for LLMs running on your
 * Mac", section "The Bit-Packing Problem" (indices packed back to back, least
 * significant bit first, crossing byte boundaries).  Code r occupies bits
 * r*code_bits .. r*code_bits + code_bits - 1 of out_codes, bit k being bit
 * k mod 8 of byte k / 8; the unused high bits of the last byte are written as
 * zero.  A group whose slot is invalid gets codes of code_bits one-bits.
 *
 *   channel_scale  device fp32 factors, aligned to 4 bytes, or NULL (no
 *                  smoothing: the codes are vq_encode's indices).
 *   head_dim       channels per key, a multiple of sub_dim, <= VQ_MAX_HEAD_DIM
 *                  (ignored when channel_scale is NULL).
 *   scale_stride   floats between the factor vectors of consecutive slots;
 *                  0 = one vector [head_dim] for every slot.
 *   code_bits      1 .. 32 with n_centroids <= 2^code_bits (8 for the pages'
 *                  256-centroid codebooks).
 *   out_codes      device, ceil(n*code_bits/8) bytes, aligned to 4 bytes; no
 *                  byte beyond that length is written.
 *   other arguments as for vq_encode.
 * With several groups, group_len*code_bits must be a multiple of 32 (groups
 * start on a 32-bit word of the stream), else VQ_ERR_UNSUPPORTED.
 */
vq_status vq_encode_packed(const void *x, const void *codebook, int64_t n, int32_t sub_dim,
                           int32_t n_centroids, vq_dtype dtype, int64_t codebook_stride,
                           int64_t n_codebooks, int64_t group_len, const int32_t *group_map,
                           const float *channel_scale, int32_t head_dim, int64_t scale_stride,
                           int32_t code_bits, void *out_codes, void *stream);

/*
 * vq_kmeans -- K-means calibration of the codebook slots on the device.
 *
 * The codebook of VecInfer product VQ is a set of K-means centroids trained
 * on calibration data ("I Wrote a Metal Kernel to Stop My Mac From OOMing",
 * section "What Even Is a KV Cache And Why Should You Care", step 2).  Runs
 * `iterations` steps of Lloyd's algorithm from the codebook given, every slot
 * trained on the sub-vectors of the groups mapped to it:
 *     assignment: out_idx = vq_encode of every sub-vector (same arithmetic)
 *     update:     every centroid with members becomes the exact mean of its
 *                 members rounded once to the element type (to nearest,
 *                 ties to even); a centroid without members keeps its value.
 * Exact means: every finite fp16 value is an integer multiple of 2^-24 and
 * every finite bf16 value one of 2^-133, so member sums are exact integers
 * (int64 for fp16, 8 int64 limbs of weight 2^(32 j) for bf16) and the mean is rounded once,
 * in integer arithmetic.  A non-finite component adds 0 to its sum (its row
 * still counts as a member).  The codebook is updated in place; out_idx holds
 * the assignment of the last iteration (made against the codebook before its
 * last update).  Results are deterministic and identical to the CPU oracle's.
 *
 *   x, n, sub_dim, n_centroids, dtype, codebook_stride, n_codebooks,
 *   group_len, group_map   as for vq_encode.
 *   codebook    device, read and written.
 *   iterations  >= 0 (0: nothing is done).
 *   out_idx     device uint32 [n], 4-aligned.
 *   workspace   device scratch of at least vq_kmeans_workspace_bytes(...)
 *               bytes, 8-aligned, owned by the caller; contents on entry do
 *               not matter.  Calls sharing a workspace must be ordered.
 * A slot may receive at most VQ_KMEANS_MAX_SLOT_ROWS sub-vectors (n with a
 * group_map, else min(group_len, n)), else VQ_ERR_UNSUPPORTED: the exact
 * member sums and their limbs are 64-bit integers.
 * vq_kmeans_workspace_bytes returns 0 for arguments vq_kmeans rejects.
 */
size_t vq_kmeans_workspace_bytes(int32_t sub_dim, int32_t n_centroids, int64_t n_codebooks,
                                 vq_dtype dtype);

vq_status vq_kmeans(const void *x, void *codebook, int64_t n, int32_t sub_dim,
                    int32_t n_centroids, vq_dtype dtype, int64_t codebook_stride,
                    int64_t n_codebooks, int64_t group_len, const int32_t *group_map,
                    int32_t iterations, uint32_t *out_idx, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * vq_attention_decode -- attention of one new query per sequence over a key /
 * value cache held as 8-bit product-VQ codes, computed from the codes.
 *
 * What it computes ("I Wrote a Metal Kernel to Stop My Mac From OOMing",
 * section "What's Next: Phase 2": scores from the codebook indices and a
 * per-query lookup table built from the transformed query, the softmax-
 * weighted value sum in the same pass, never materializing fp16 keys; blog
 * index, section "The Kernel's Hot Path": LUT[sub, c] = q_sub . C_k[c]):
 * for sequence b and query head hq, kv head h = hq / (n_q_heads/n_kv_heads),
 * attended tokens t in [max(0, L - window), L) with L = kv_len[b] (window 0 =
 * all L tokens):
 *     k_t = C_k[h][k_codes[b][h][t][s]] concatenated over s, divided by the
 *           smoothing factors k_scale[h] (keys stored smoothed, as written by
 *           vq_encode_packed); v_t likewise from C_v without factors
 *     out[b][hq] = sum_t softmax_t(softmax_scale * q[b][hq] . k_t) v_t
 * (0 for a sequence with no attended token).  A code >= n_centroids decodes
 * to a zero row.  Arithmetic: q / f in fp32, base-2 softmax in fp32.  For
 * head_dim 64, 128 or 256 with at least 16 codes per key and value row and
 * 16-byte aligned code arrays, scores and the value sum run on the matrix
 * cores with the fp32 query and weights split exactly into element-type parts
 * (products exact, fp32 accumulation); other shapes build a per-query fp32
 * lookup table.  The error bound the tests hold both to is stated with them.
 *
 *   q           device, [batch][n_q_heads][head_dim] of `dtype`, 2-aligned.
 *   k_codes     device, [batch][n_kv_heads][max_kv_len][head_dim/k_sub_dim]
 *               bytes (the 8-bit stream of vq_encode_packed over a
 *               [batch][n_kv_heads][max_kv_len][head_dim] key cache), 4-aligned.
 *   v_codes     device, [batch][n_kv_heads][max_kv_len][head_dim/v_sub_dim] bytes.
 *   k_codebook  device, [n_kv_heads][n_centroids][k_sub_dim] of `dtype`.
 *   v_codebook  device, [n_kv_heads][n_centroids][v_sub_dim] of `dtype`.
 *   k_scale     device fp32 [n_kv_heads][head_dim] smoothing factors, or NULL.
 *   kv_len      device int32 [batch] (clamped to [0, max_kv_len]) or NULL (all
 *               max_kv_len).
 *   k_sub_dim, v_sub_dim  4 or 8; head_dim <= VQ_ATTN_MAX_HEAD_DIM, a multiple
 *               of 4*k_sub_dim and of v_sub_dim.
 *   n_centroids 1 .. 256.  n_q_heads a multiple of n_kv_heads, at most
 *               VQ_ATTN_MAX_GROUP query heads per kv head.
 *   out         device fp32 [batch][n_q_heads][head_dim], 4-aligned.
 *   workspace   device scratch of at least vq_attention_workspace_bytes(...)
 *               bytes, 4-aligned, owned by the caller; its contents on entry do
 *               not matter and on return are unspecified.  Calls that share a
 *               workspace must be ordered on one stream.
 */
size_t vq_attention_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t head_dim,
                                    int32_t max_kv_len);

vq_status vq_attention_decode(const void *q, const uint8_t *k_codes, const uint8_t *v_codes,
                              const void *k_codebook, const void *v_codebook,
                              const float *k_scale, const int32_t *kv_len, int32_t batch,
                              int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                              int32_t max_kv_len, int32_t k_sub_dim, int32_t v_sub_dim,
                              int32_t n_centroids, vq_dtype dtype, int32_t window,
                              float softmax_scale, float *out, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * vq_attention_decode_static -- vq_attention_decode for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc.  Same arguments, arithmetic and
 * result as vq_attention_decode, without `workspace` / `workspace_bytes`:
 * the chunk partials go to a static device buffer of
 * VQ_ATTN_STATIC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  Its address is resolved once per device, on the
 * first call with that device current.  The call allocates nothing.
 *
 * Returns VQ_ERR_TOO_LARGE (and launches nothing) when
 * vq_attention_workspace_bytes(batch, n_q_heads, head_dim, max_kv_len)
 * exceeds VQ_ATTN_STATIC_SCRATCH_BYTES (e.g. 32 sequences x 12 query heads x
 * 4096 tokens x head_dim 256 needs 6.3 MB).  Every call on one GPU shares that
 * GPU's buffer: calls must be ordered (one stream, or synchronised); calls that
 * overlap on one GPU race and their results are undefined.  Nothing in the
 * buffer needs to start at zero (every partial is written before it is read).
 */
vq_status vq_attention_decode_static(const void *q, const uint8_t *k_codes,
                                     const uint8_t *v_codes, const void *k_codebook,
                                     const void *v_codebook, const float *k_scale,
                                     const int32_t *kv_len, int32_t batch, int32_t n_q_heads,
                                     int32_t n_kv_heads, int32_t head_dim, int32_t max_kv_len,
                                     int32_t k_sub_dim, int32_t v_sub_dim, int32_t n_centroids,
                                     vq_dtype dtype, int32_t window, float softmax_scale,
                                     float *out, void *stream);

/*
 * vq_decode -- gather used to check encode: row n of out_x is centroid idx[n]
 * of the slot of n's group, copied bit for bit (the reconstruction the post
 * measures MSE on, section "Correctness: Bit-Exact on fp32, MSE-Identical on
 * fp16"; the gather of section "Mistake 1: I Wrote the Dequant Kernel First").
 * An index >= n_centroids or a bad slot gives a row of zero bits.
 *
 *   idx    device, [n] uint32, aligned to 4 bytes.
 *   out_x  device, [n][sub_dim] elements of `dtype`, aligned to 2 bytes.
 *   other arguments as for vq_encode.
 */
vq_status vq_decode(const uint32_t *idx, const void *codebook, int64_t n, int32_t sub_dim,
                    int32_t n_centroids, vq_dtype dtype, int64_t codebook_stride,
                    int64_t n_codebooks, int64_t group_len, const int32_t *group_map,
                    void *out_x, void *stream);

/* Static description of a status code (never NULL). */
const char *vq_status_str(int32_t status);

/* hipError_t of the last VQ_ERR_DEVICE returned on this host thread (0 if none). */
int32_t vq_last_hip_error(void);

/* VQ_ABI_VERSION of the loaded library. */
int32_t vq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PRODUCT_VQ_KV_AMD_VQ_H */
