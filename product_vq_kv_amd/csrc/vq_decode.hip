// vq_decode.hip -- gather of codebook rows by index, used to check encode.
//
// Row n of the output is centroid idx[n] of the codebook slot of n's group,
// copied bit for bit; an index >= n_centroids or a bad slot gives zero bits
// (VeloxQuant-MLX blog, "I Wrote a Metal Kernel to Stop My Mac From OOMing",
// section "Mistake 1: I Wrote the Dequant Kernel First": dequantization is a
// plain gather, which is why it is kept simple here).  One lane per row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vq_launch.h"

namespace vqk {
namespace {

constexpr int kBlock = 256;

template <int SD>
__global__ void __launch_bounds__(kBlock)
decode_kernel(const uint32_t *__restrict__ idx, const uint16_t *__restrict__ codebook, int64_t n,
              int n_c, int64_t cb_stride, int64_t n_codebooks, int64_t group_len,
              const int32_t *__restrict__ group_map, uint16_t *__restrict__ out) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (row >= n) return;
  const int64_t g = row / group_len;
  const int64_t slot = group_map ? static_cast<int64_t>(group_map[g]) : g;
  const uint32_t c = idx[row];
  uint16_t *dst = out + row * SD;
  if (slot < 0 || slot >= n_codebooks || c >= static_cast<uint32_t>(n_c)) {
#pragma unroll
    for (int i = 0; i < SD; ++i) dst[i] = 0;
    return;
  }
  const uint16_t *src = codebook + slot * cb_stride + static_cast<int64_t>(c) * SD;
#pragma unroll
  for (int i = 0; i < SD; ++i) dst[i] = src[i];
}

}  // namespace

hipError_t launch_decode(const uint32_t *idx, const void *codebook, const int32_t *group_map,
                         void *out_x, const Layout &l, hipStream_t stream) {
  const int64_t grid = (l.n + kBlock - 1) / kBlock;
  const uint16_t *cb = static_cast<const uint16_t *>(codebook);
  uint16_t *out = static_cast<uint16_t *>(out_x);
  if (l.sub_dim == 4) {
    hipLaunchKernelGGL(decode_kernel<4>, dim3(static_cast<uint32_t>(grid)), dim3(kBlock), 0,
                       stream, idx, cb, l.n, l.n_centroids, l.codebook_stride, l.n_codebooks,
                       l.group_len, group_map, out);
  } else {
    hipLaunchKernelGGL(decode_kernel<8>, dim3(static_cast<uint32_t>(grid)), dim3(kBlock), 0,
                       stream, idx, cb, l.n, l.n_centroids, l.codebook_stride, l.n_codebooks,
                       l.group_len, group_map, out);
  }
  return hipGetLastError();
}

}  // namespace vqk
