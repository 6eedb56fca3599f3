// vq_encode.hip -- product-VQ encode for gfx950 (CDNA4).
//
// Computes, for every sub-vector, the index of its nearest codebook centroid
// by squared L2 distance (VeloxQuant-MLX blog, "I Wrote a Metal Kernel to Stop
// My Mac From OOMing", sections "What quantize_vq Was Doing Wrong" and "The
// Kernel: 18 Lines of MSL").  The distance is evaluated exactly as the page's
// kernel states it, in fp32: d = x_i - c_i (one rounding), dist += d*d taken as
// one fused multiply-add, components in order; strict-< argmin from
// (+inf, 0), so ties keep the lowest index.
//
// Design (MI355X-first, not a translation of the Metal kernel):
//   * one workgroup = 256 lanes (4 wave64) encodes a tile of 256*S
//     sub-vectors of one group; a tile never straddles groups, so the whole
//     workgroup shares one codebook slot (per-(layer, head) select);
//   * the codebook slot is widened to fp32 once per workgroup and staged in
//     LDS (in chunks of at most kChunkMax centroids); every lane reads the same
//     centroid at the same time, so each LDS read is a broadcast;
//   * each lane keeps S sub-vectors in fp32 registers (coalesced loads of
//     2*sub_dim bytes per sub-vector, consecutive lanes on consecutive rows);
//   * the [N, n_centroids, sub_dim] difference tensor of the pure-array path
//     never exists: each distance lives in one register for a few cycles;
//   * argmin: instead of a compare + two selects per centroid, a running
//     minimum (v_min3_f32 folds two new distances per instruction) and, every
//     G centroids, one compare + select that remembers the last group in which
//     the minimum strictly decreased.  That group holds the first occurrence
//     of the minimum; it is recomputed from LDS with the identical instruction
//     sequence (so the same bits) and the lowest index whose distance equals
//     the minimum is the answer -- exactly the strict-< scan's result;
//   * smoothed keys (SCALED): each component is multiplied by its channel's
//     fp32 factor (staged in LDS per slot) right after widening, and the
//     search runs on those fp32 values with the same instruction sequence.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vq_codes.h"
#include "vq_launch.h"

namespace vqk {
namespace {

constexpr int kBlock = 256;      // lanes per workgroup
constexpr int kChunkMax = 1024;  // centroids staged in LDS at a time
constexpr int kGroup = 8;        // centroids per argmin tracking group

template <bool BF16>
__device__ __forceinline__ float widen(uint16_t v) {
  if constexpr (BF16) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
  } else {
    return static_cast<float>(__builtin_bit_cast(_Float16, v));
  }
}

// Fixed-order fp32 squared distance.  The first step is d*d, which equals
// fma(d, d, +0) bit for bit.
template <int SD>
__device__ __forceinline__ float sqdist(const float (&xv)[SD], const float (&c)[SD]) {
  float d = xv[0] - c[0];
  float acc = d * d;
#pragma unroll
  for (int i = 1; i < SD; ++i) {
    d = xv[i] - c[i];
    acc = __builtin_fmaf(d, d, acc);
  }
  return acc;
}

template <int SD>
__device__ __forceinline__ void lds_row(const float *lds, int c, float (&v)[SD]) {
  const float4 *p = reinterpret_cast<const float4 *>(lds + c * SD);
#pragma unroll
  for (int q = 0; q < SD / 4; ++q) {
    float4 t = p[q];
    v[4 * q + 0] = t.x;
    v[4 * q + 1] = t.y;
    v[4 * q + 2] = t.z;
    v[4 * q + 3] = t.w;
  }
}

template <int SD, bool BF16>
__device__ __forceinline__ void load_x(const uint16_t *__restrict__ x, int64_t row, float (&v)[SD]) {
  if constexpr (SD == 4) {
    uint2 w = *reinterpret_cast<const uint2 *>(x + row * 4);
    v[0] = widen<BF16>(static_cast<uint16_t>(w.x));
    v[1] = widen<BF16>(static_cast<uint16_t>(w.x >> 16));
    v[2] = widen<BF16>(static_cast<uint16_t>(w.y));
    v[3] = widen<BF16>(static_cast<uint16_t>(w.y >> 16));
  } else {
    uint4 w = *reinterpret_cast<const uint4 *>(x + row * 8);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q + 0] = widen<BF16>(static_cast<uint16_t>(u[q]));
      v[2 * q + 1] = widen<BF16>(static_cast<uint16_t>(u[q] >> 16));
    }
  }
}

template <int SD, int S, bool BF16, bool SCALED>
__global__ void __launch_bounds__(kBlock)
encode_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ codebook,
              int64_t n, int n_c, int64_t cb_stride, int64_t n_codebooks, int64_t group_len,
              uint32_t tiles_per_group, const int32_t *__restrict__ group_map,
              uint8_t *__restrict__ out, int chunk, const float *__restrict__ scale,
              int64_t scale_stride, int head_dim, int code_bits) {
  extern __shared__ float4 lds4[];
  float *lds = reinterpret_cast<float *>(lds4);
  float *lds_scale = lds + chunk * SD;  // smoothed keys: the slot's factors
  constexpr int kTile = kBlock * S;

  const uint32_t b = blockIdx.x;
  const uint32_t g = b / tiles_per_group;
  const uint32_t t = b - g * tiles_per_group;
  const int64_t gstart = static_cast<int64_t>(g) * group_len;
  const int64_t gend = min(gstart + group_len, n);
  const int64_t tbase = gstart + static_cast<int64_t>(t) * kTile;
  if (tbase >= gend) return;  // whole workgroup: tile past its group's end
  const int tid = threadIdx.x;
  const int64_t half0 = tbase + (tid & ~31);  // first row of this lane's half-wave

  const int64_t slot = group_map ? static_cast<int64_t>(group_map[g]) : static_cast<int64_t>(g);
  if (slot < 0 || slot >= n_codebooks) {
#pragma unroll
    for (int s = 0; s < S; ++s) store_codes32(0xFFFFFFFFu, half0 + s * kBlock, gend, code_bits, true, out);
    return;  // whole workgroup
  }
  const uint16_t *__restrict__ cb = codebook + slot * cb_stride;

  float xv[S][SD];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t row = tbase + s * kBlock + tid;
    if (row < gend) {
      load_x<SD, BF16>(x, row, xv[s]);
    } else {
#pragma unroll
      for (int i = 0; i < SD; ++i) xv[s][i] = 0.0f;
    }
  }
  if constexpr (SCALED) {
    const float *__restrict__ f = scale + slot * scale_stride;
    for (int i = tid; i < head_dim; i += kBlock) lds_scale[i] = f[i];
    __syncthreads();
    const int n_sub = head_dim / SD;
    const float inv_n_sub = 1.0f / static_cast<float>(n_sub);
    const int tmod = static_cast<int>(tbase % n_sub);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int m = mod_small(tmod + s * kBlock + tid, n_sub, inv_n_sub);
#pragma unroll
      for (int i = 0; i < SD; ++i) xv[s][i] = xv[s][i] * lds_scale[m * SD + i];
    }
  }

  float m[S], mp[S];
  uint32_t bg[S], res[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    m[s] = __builtin_inff();
    mp[s] = __builtin_inff();
    bg[s] = 0;
    res[s] = 0;
  }

  for (int cbase = 0; cbase < n_c; cbase += chunk) {
    const int clen = min(chunk, n_c - cbase);
    const int cpad = (clen + kGroup - 1) / kGroup * kGroup;
    __syncthreads();  // every lane is done with the previous chunk
    for (int e = tid; e < cpad * SD; e += kBlock) {
      const int c = e / SD;
      lds[e] = (c < clen) ? widen<BF16>(cb[static_cast<int64_t>(cbase) * SD + e]) : __builtin_inff();
    }
    __syncthreads();

    float mstart[S];
#pragma unroll
    for (int s = 0; s < S; ++s) mstart[s] = m[s];

    for (int gb = 0; gb < cpad; gb += kGroup) {
#pragma unroll
      for (int j = 0; j < kGroup; j += 2) {
        float c0[SD], c1[SD];
        lds_row<SD>(lds, gb + j, c0);
        lds_row<SD>(lds, gb + j + 1, c1);
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const float d0 = sqdist<SD>(xv[s], c0);
          const float d1 = sqdist<SD>(xv[s], c1);
          m[s] = fminf(m[s], fminf(d0, d1));
        }
      }
      const uint32_t grp = static_cast<uint32_t>(cbase + gb) / kGroup;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        bg[s] = (m[s] < mp[s]) ? grp : bg[s];
        mp[s] = m[s];
      }
    }

    // Resolve, for sub-vectors whose minimum fell inside this chunk, the
    // lowest index in the remembered group whose distance equals it.
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (m[s] < mstart[s]) {
        const int lb = static_cast<int>(bg[s]) * kGroup - cbase;
        uint32_t r = 0;
#pragma unroll
        for (int j = kGroup - 1; j >= 0; --j) {
          float c[SD];
          lds_row<SD>(lds, lb + j, c);
          const float d = sqdist<SD>(xv[s], c);
          r = (d == m[s]) ? static_cast<uint32_t>(cbase + lb + j) : r;
        }
        res[s] = r;
      }
    }
  }

#pragma unroll
  for (int s = 0; s < S; ++s) store_codes32(res[s], half0 + s * kBlock, gend, code_bits, true, out);
}

template <int SD>
constexpr int sub_vectors_per_lane() { return 4; }

template <int SD, bool BF16, bool SCALED>
hipError_t launch_t(const void *x, const void *codebook, const int32_t *group_map, void *out,
                    const Layout &l, const Codes &codes, hipStream_t stream) {
  constexpr int S = sub_vectors_per_lane<SD>();
  constexpr int kTile = kBlock * S;
  const int64_t span = l.group_len < l.n ? l.group_len : l.n;
  const int64_t tiles_per_group = (span + kTile - 1) / kTile;
  const int64_t grid = tiles_per_group * l.n_groups;
  const int chunk_raw = l.n_centroids < kChunkMax ? l.n_centroids : kChunkMax;
  const int chunk = (chunk_raw + kGroup - 1) / kGroup * kGroup;
  const size_t lds_bytes =
      (static_cast<size_t>(chunk) * SD + (SCALED ? codes.head_dim : 0)) * sizeof(float);
  hipLaunchKernelGGL((encode_kernel<SD, S, BF16, SCALED>), dim3(static_cast<uint32_t>(grid)),
                     dim3(kBlock), lds_bytes, stream,
                     static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(codebook),
                     l.n, l.n_centroids, l.codebook_stride, l.n_codebooks, l.group_len,
                     static_cast<uint32_t>(tiles_per_group), group_map,
                     static_cast<uint8_t *>(out), chunk, codes.scale, codes.scale_stride,
                     codes.head_dim, codes.code_bits);
  return hipGetLastError();
}

template <int SD, bool BF16>
hipError_t launch_scaled(const void *x, const void *codebook, const int32_t *group_map, void *out,
                         const Layout &l, const Codes &codes, hipStream_t stream) {
  return codes.scale ? launch_t<SD, BF16, true>(x, codebook, group_map, out, l, codes, stream)
                     : launch_t<SD, BF16, false>(x, codebook, group_map, out, l, codes, stream);
}

}  // namespace

int64_t encode_grid(const Layout &l) {
  const int S = 4;
  const int64_t tile = static_cast<int64_t>(kBlock) * S;
  const int64_t span = l.group_len < l.n ? l.group_len : l.n;
  return (span + tile - 1) / tile * l.n_groups;
}

hipError_t launch_encode(const void *x, const void *codebook, const int32_t *group_map,
                         void *out, const Layout &l, const Codes &codes, hipStream_t stream) {
  if (l.sub_dim == 4) {
    return l.bf16 ? launch_scaled<4, true>(x, codebook, group_map, out, l, codes, stream)
                  : launch_scaled<4, false>(x, codebook, group_map, out, l, codes, stream);
  }
  return l.bf16 ? launch_scaled<8, true>(x, codebook, group_map, out, l, codes, stream)
                : launch_scaled<8, false>(x, codebook, group_map, out, l, codes, stream);
}

}  // namespace vqk
