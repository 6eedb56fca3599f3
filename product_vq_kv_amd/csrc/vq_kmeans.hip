// vq_kmeans.hip -- K-means codebook calibration on the device (gfx950).
//
// The codebook of VecInfer product VQ is a set of K-means centroids trained
// on calibration data (VeloxQuant-MLX blog, "I Wrote a Metal Kernel to Stop
// My Mac From OOMing", section "What Even Is a KV Cache And Why Should You
// Care", step 2).  Lloyd's algorithm, every codebook slot trained on the
// sub-vectors of its own groups:
//   assignment: the encode (nearest centroid, exact) -> out_idx
//   update:     centroid = exact member mean rounded once to fp16 (round to
//               nearest even); a centroid without members keeps its value.
// fp16 values are integer multiples of 2^-24, so member sums are exact int64
// (|sum| < 2^40 * n); the sums are accumulated per workgroup in LDS with
// 64-bit integer atomics and flushed with 64-bit global atomics, so the
// result does not depend on the order of the additions, and the rounding of
// sum / count is done exactly in integer arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vq_launch.h"

namespace vqk {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerTile = 4096;      // rows per accumulate workgroup
constexpr int kLdsMaxCentroids = 512;   // beyond: accumulate straight to global

// x * 2^24 as an exact integer (fp16 x; non-finite values count as 0).
__device__ __forceinline__ int64_t units(uint16_t bits) {
  const float v = static_cast<float>(__builtin_bit_cast(_Float16, bits));
  if (!(__builtin_fabsf(v) <= 65504.0f)) return 0;
  return static_cast<int64_t>(v * 16777216.0f);  // exact: 11 significant bits
}

// fp16 bits of S / (n * 2^24) rounded to nearest even (n >= 1, |S| < 2^63).
__device__ uint16_t round_mean_f16(int64_t S, uint32_t n) {
  const uint16_t sign = S < 0 ? 0x8000u : 0u;
  const uint64_t A = S < 0 ? static_cast<uint64_t>(-(S + 1)) + 1u : static_cast<uint64_t>(S);
  if (A == 0) return 0;
  // f = floor(log2(A / n))
  const int la = 63 - __clzll(static_cast<long long>(A));
  const int ln = 31 - __clz(static_cast<int>(n));
  int f = la - ln;
  const bool ge = (f >= 0) ? ((A >> f) >= n) : ((A << (-f)) >= n);
  if (!ge) --f;
  // exponent of the result: floor(log2(A / (n 2^24))) clamped to subnormals
  int e = f - 24;
  if (e < -14) e = -14;
  if (e > 15) return sign | 0x7C00u;
  // m = round(A / (n 2^(e+14))), the 11-bit significand (or subnormal digits)
  const uint64_t den = static_cast<uint64_t>(n) << (e + 14);  // <= 2^60
  uint64_t m = A / den;
  const uint64_t rem = A - m * den;
  if (2 * rem > den || (2 * rem == den && (m & 1u))) ++m;
  if (m == 2048) {
    m = 1024;
    ++e;
    if (e > 15) return sign | 0x7C00u;
  }
  if (m < 1024) return sign | static_cast<uint16_t>(m);  // subnormal (e == -14)
  return sign | static_cast<uint16_t>(((e + 15) << 10) | (m - 1024));
}

struct KmArgs {
  const uint16_t *x;
  const uint32_t *idx;
  uint16_t *codebook;
  const int32_t *group_map;
  unsigned long long *sums;    // [n_codebooks][n_c][sd], two's complement
  unsigned int *counts;        // [n_codebooks][n_c]
  int64_t n, cb_stride, n_codebooks, group_len, tiles_per_group;
  int sd, n_c;
};

// Member sums and counts of one tile of rows (one group, so one slot).
template <int SD>
__global__ void __launch_bounds__(kThreads) km_accumulate(const KmArgs a) {
  extern __shared__ unsigned long long lsum[];  // [n_c][SD] then counts [n_c] (as u64)
  const int64_t tile = blockIdx.x;
  const int64_t g = tile / a.tiles_per_group;
  const int64_t gstart = g * a.group_len;
  const int64_t gend = min(gstart + a.group_len, a.n);
  const int64_t tbase = gstart + (tile - g * a.tiles_per_group) * kRowsPerTile;
  if (tbase >= gend) return;  // whole workgroup
  const int64_t slot = a.group_map ? static_cast<int64_t>(a.group_map[g]) : g;
  if (slot < 0 || slot >= a.n_codebooks) return;  // whole workgroup: no centroid to train
  const int64_t tend = min(tbase + kRowsPerTile, gend);
  unsigned long long *gs = a.sums + slot * a.n_c * SD;
  unsigned int *gc = a.counts + slot * a.n_c;
  const bool use_lds = a.n_c <= kLdsMaxCentroids;
  unsigned long long *lcnt = lsum + a.n_c * SD;
  if (use_lds) {
    for (int e = threadIdx.x; e < a.n_c * (SD + 1); e += kThreads) lsum[e] = 0;
    __syncthreads();
  }
  for (int64_t r = tbase + threadIdx.x; r < tend; r += kThreads) {
    const uint32_t c = a.idx[r];
    if (c >= static_cast<uint32_t>(a.n_c)) continue;
    const uint16_t *xr = a.x + r * SD;
#pragma unroll
    for (int i = 0; i < SD; ++i) {
      const unsigned long long u = static_cast<unsigned long long>(units(xr[i]));
      if (use_lds) {
        atomicAdd(&lsum[c * SD + i], u);
      } else {
        atomicAdd(&gs[c * SD + i], u);
      }
    }
    if (use_lds) {
      atomicAdd(&lcnt[c], 1ull);
    } else {
      atomicAdd(&gc[c], 1u);
    }
  }
  if (use_lds) {
    __syncthreads();
    for (int e = threadIdx.x; e < a.n_c * SD; e += kThreads)
      if (lsum[e]) atomicAdd(&gs[e], lsum[e]);
    for (int c = threadIdx.x; c < a.n_c; c += kThreads)
      if (lcnt[c]) atomicAdd(&gc[c], static_cast<unsigned int>(lcnt[c]));
  }
}

// New centroids from the sums (one thread per (slot, centroid)); the sums
// and counts are cleared for the next iteration.
template <int SD>
__global__ void __launch_bounds__(kThreads) km_update(const KmArgs a) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (e >= a.n_codebooks * a.n_c) return;
  const int64_t slot = e / a.n_c;
  const int c = static_cast<int>(e - slot * a.n_c);
  const unsigned int cnt = a.counts[e];
  uint16_t *cw = a.codebook + slot * a.cb_stride + static_cast<int64_t>(c) * SD;
#pragma unroll
  for (int i = 0; i < SD; ++i) {
    const int64_t S = static_cast<int64_t>(a.sums[e * SD + i]);
    if (cnt > 0) cw[i] = round_mean_f16(S, cnt);
    a.sums[e * SD + i] = 0;
  }
  a.counts[e] = 0;
}

__global__ void __launch_bounds__(kThreads) km_clear(const KmArgs a) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t nc = a.n_codebooks * a.n_c;
  if (e < nc * a.sd) a.sums[e] = 0;
  if (e < nc) a.counts[e] = 0;
}

template <int SD>
hipError_t launch_km(const KmArgs &a, const Layout &l, int iterations, hipStream_t stream) {
  const int64_t cells = a.n_codebooks * a.n_c;
  const int64_t clear_blocks = (cells * SD + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(km_clear, dim3(static_cast<uint32_t>(clear_blocks)), dim3(kThreads), 0,
                     stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t tiles = a.tiles_per_group * ((a.n + a.group_len - 1) / a.group_len);
  const size_t lds = a.n_c <= kLdsMaxCentroids
                         ? static_cast<size_t>(a.n_c) * (SD + 1) * sizeof(unsigned long long)
                         : 0;
  const int64_t upd_blocks = (cells + kThreads - 1) / kThreads;
  for (int it = 0; it < iterations; ++it) {
    err = encode_mfma_supported(l)
              ? launch_encode_mfma(a.x, a.codebook, a.group_map, const_cast<uint32_t *>(a.idx), l,
                                   plain_codes(l), stream)
              : launch_encode(a.x, a.codebook, a.group_map, const_cast<uint32_t *>(a.idx), l,
                              plain_codes(l), stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(km_accumulate<SD>, dim3(static_cast<uint32_t>(tiles)), dim3(kThreads), lds,
                       stream, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(km_update<SD>, dim3(static_cast<uint32_t>(upd_blocks)), dim3(kThreads), 0,
                       stream, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace

size_t kmeans_workspace_bytes(int sub_dim, int n_centroids, int64_t n_codebooks) {
  return static_cast<size_t>(n_codebooks) * n_centroids * (sub_dim * sizeof(unsigned long long) +
                                                           sizeof(unsigned int));
}

int64_t kmeans_grid(const Layout &l) {
  const int64_t span = l.group_len < l.n ? l.group_len : l.n;
  return (span + kRowsPerTile - 1) / kRowsPerTile * l.n_groups;
}

hipError_t launch_kmeans(const void *x, void *codebook, const int32_t *group_map, uint32_t *out_idx,
                         const Layout &l, int iterations, void *workspace, hipStream_t stream) {
  KmArgs a;
  a.x = static_cast<const uint16_t *>(x);
  a.idx = out_idx;
  a.codebook = static_cast<uint16_t *>(codebook);
  a.group_map = group_map;
  a.sums = static_cast<unsigned long long *>(workspace);
  a.counts = reinterpret_cast<unsigned int *>(a.sums + l.n_codebooks * l.n_centroids * l.sub_dim);
  a.n = l.n;
  a.cb_stride = l.codebook_stride;
  a.n_codebooks = l.n_codebooks;
  a.group_len = l.group_len;
  const int64_t span = l.group_len < l.n ? l.group_len : l.n;
  a.tiles_per_group = (span + kRowsPerTile - 1) / kRowsPerTile;
  a.sd = l.sub_dim;
  a.n_c = l.n_centroids;
  return l.sub_dim == 4 ? launch_km<4>(a, l, iterations, stream)
                        : launch_km<8>(a, l, iterations, stream);
}

}  // namespace vqk
