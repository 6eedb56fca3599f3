// Internal interface between the C-ABI front end (vq_capi.cpp) and the
// kernel launchers.  Arguments have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vqk {

struct Layout {
  int64_t n;               // sub-vectors
  int32_t sub_dim;         // 4 or 8
  int32_t n_centroids;     // 1 .. 65536
  int32_t bf16;            // 0 = fp16, 1 = bf16
  int64_t codebook_stride; // elements between codebook slots
  int64_t n_codebooks;     // slots in the codebook buffer
  int64_t group_len;       // sub-vectors per group
  int64_t n_groups;        // ceil(n / group_len)
};

// Smoothing and output format of an encode.
struct Codes {
  const float *scale;    // per-slot channel factors (device), or nullptr
  int64_t scale_stride;  // floats between slots' factor vectors
  int32_t head_dim;      // channels per key vector (multiple of sub_dim)
  int32_t code_bits;     // 1 .. 32; 32 = one uint32 index per sub-vector
};

// Plain encode: no factors, uint32 indices.
inline Codes plain_codes(const Layout &l) { return Codes{nullptr, 0, l.sub_dim, 32}; }

// Largest head_dim the kernels stage factors for.
constexpr int kMaxHeadDim = 4096;

// Number of workgroups the encode launch uses for `l` (the host checks that
// it fits the grid before launching).
int64_t encode_grid(const Layout &l);

hipError_t launch_encode(const void *x, const void *codebook, const int32_t *group_map,
                         void *out, const Layout &l, const Codes &codes, hipStream_t stream);

// The matrix-core encode keeps the whole codebook slot in LDS: up to 4096 centroids.
bool encode_mfma_supported(const Layout &l);
int64_t encode_mfma_grid(const Layout &l);

hipError_t launch_encode_mfma(const void *x, const void *codebook, const int32_t *group_map,
                              void *out, const Layout &l, const Codes &codes,
                              hipStream_t stream);

// K-means member sums in the caller's workspace: kKmReplicas copies of
// sums [n_codebooks][n_c][sub_dim] (int64 units of 2^-24, two's complement)
// and counts [n_codebooks][n_c]; a workgroup adds into copy (index mod
// kKmReplicas).
constexpr int kKmReplicas = 8;
// int64 limbs (weights 2^(32 j)) of an exact bf16 member sum (multiples of
// 2^-133 below 2^285)
constexpr int kKmBf16Limbs = 8;
struct KmSums {
  unsigned long long *sums;
  unsigned int *counts;
};

// The matrix-core encode that also adds every sub-vector to its centroid's
// member sums (fp16, unsmoothed, uint32 indices): up to this many centroids.
constexpr int kKmFusedMaxCentroids = 512;
bool encode_mfma_kmeans_supported(const Layout &l);
hipError_t launch_encode_mfma_kmeans(const void *x, const void *codebook,
                                     const int32_t *group_map, uint32_t *out, const Layout &l,
                                     const KmSums &acc, hipStream_t stream);

hipError_t launch_decode(const uint32_t *idx, const void *codebook, const int32_t *group_map,
                         void *out_x, const Layout &l, hipStream_t stream);

// Decode attention over VQ-coded caches (validated by the caller).
struct AttnLayout {
  const void *q;             // [B][Hq][D] fp16/bf16
  const uint8_t *k_codes;    // [B][Hkv][S][D / k_sub_dim]
  const uint8_t *v_codes;    // [B][Hkv][S][D / v_sub_dim]
  const void *k_codebook;    // [Hkv][n_c][k_sub_dim]
  const void *v_codebook;    // [Hkv][n_c][v_sub_dim]
  const float *k_scale;      // [Hkv][D] or nullptr
  const int32_t *kv_len;     // [B] or nullptr
  float *out;                // [B][Hq][D]
  float *workspace;          // attention_chunks(S) partials per (b, hq)
  int32_t batch, n_q_heads, n_kv_heads, head_dim, max_kv_len;
  int32_t k_sub_dim, v_sub_dim, n_centroids, bf16, window;
  float softmax_scale;
};

// K-means calibration (fp16 or bf16): `iterations` Lloyd steps, codebook
// updated in place, final assignment in out_idx; workspace = exact member
// sums (one int64 per component for fp16, kKmBf16Limbs for bf16) + counts.
size_t kmeans_workspace_bytes(int sub_dim, int n_centroids, int64_t n_codebooks, bool bf16);
int64_t kmeans_grid(const Layout &l);
hipError_t launch_kmeans(const void *x, void *codebook, const int32_t *group_map, uint32_t *out_idx,
                         const Layout &l, int iterations, void *workspace, hipStream_t stream);

int attention_chunks(int max_kv_len);
size_t attention_lds_bytes(int k_sub_dim, int v_sub_dim, int head_dim, int group);
hipError_t launch_attention(const AttnLayout &l, hipStream_t stream);
// Address of the static attention scratch (VQ_ATTN_STATIC_SCRATCH_BYTES) on
// the current device, resolved once per device.
hipError_t attention_static_scratch(void **ptr);

}  // namespace vqk
