// vq_kmeans.hip -- K-means codebook calibration on the device (gfx950).
//
// The codebook of VecInfer product VQ is a set of K-means centroids trained
// on calibration data (VeloxQuant-MLX blog, "I Wrote a Metal Kernel to Stop
// My Mac From OOMing", section "What Even Is a KV Cache And Why Should You
// Care", step 2).  Lloyd's algorithm, every codebook slot trained on the
// sub-vectors of its own groups:
//   assignment: the encode (nearest centroid, exact) -> out_idx
//   update:     centroid = exact member mean rounded once to the element type
//               (round to nearest even); a centroid without members keeps
//               its value.
// fp16: every value is an integer multiple of 2^-24, so member sums are exact
// int64 (|sum| < 2^40 * n).  Up to 512 centroids the encode itself adds every
// sub-vector to its centroid's sums (fp64 LDS atomics, exact for the at most
// 8192 rows a workgroup adds before it flushes, see vq_encode_mfma.hip).
// bf16: every finite value is an integer multiple of 2^-133 below 2^261, so a
// member sum is an integer below 2^285.  It is kept as kLimbs signed int64
// limbs, limb j weighing 2^(32 j): a member whose value is m 2^p units (m <
// 2^8) adds m 2^(p mod 32) < 2^39 to limb p / 32, so a limb stays below
// 2^23 * 2^39 = 2^62 in magnitude for up to 2^23 members (limbs carry past
// 32 bits).  The update propagates the carries into one 320-bit integer and
// divides it by the count.
// Otherwise (bf16, or fp16 above 512 centroids) km_accumulate reads the rows
// and codes back: a workgroup takes a tile of rows of one group and a range
// of centroids whose sums fit in LDS, adds the members in that range with
// 64-bit LDS atomics, and flushes the nonzero sums with 64-bit global atomics.
// The flushes go into one of kReplicas copies (fewer workgroups contend for
// one address), which the update adds up.
// Integer addition is associative, so the result does not depend on the order
// of the additions, and the rounding of sum / count is done exactly in
// integer arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "vq_launch.h"

namespace vqk {
namespace {

constexpr int kThreads = 256;        // update and clear workgroups
constexpr int kAccThreads = 1024;    // accumulate workgroups
constexpr int kRowsPerThread = 4;
constexpr int kRowsPerBatch = kAccThreads * kRowsPerThread;  // rows per accumulate round
constexpr int64_t kAccMaxTileRows = 1 << 16;  // rows per accumulate workgroup at most
constexpr size_t kAccLdsBytes = 144 * 1024;   // LDS of an accumulate workgroup at most
constexpr int kReplicas = kKmReplicas;  // copies of the sums the flush is spread over
constexpr int kLimbs = kKmBf16Limbs;    // int64 limbs (weight 2^(32 j)) of a bf16 member sum

// x * 2^24 as an exact integer (fp16 x; non-finite values count as 0): a
// normal value (1024 + m) 2^(e - 25) gives (1024 + m) 2^(e - 1), a
// subnormal m 2^-24 gives m.
__device__ __forceinline__ int64_t units(uint16_t bits) {
  const uint32_t e = (bits >> 10) & 31u, m = bits & 1023u;
  uint64_t mag = (e == 0) ? m : (static_cast<uint64_t>(1024u | m) << (e - 1));
  mag = (e == 31) ? 0 : mag;
  return (bits & 0x8000u) ? -static_cast<int64_t>(mag) : static_cast<int64_t>(mag);
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

// bf16 bits of A / (n * 2^133) rounded to nearest even, A = the magnitude
// of an exact sum as 10 little-endian 32-bit words, n >= 1 (the count).
__device__ uint16_t round_mean_bf16(uint32_t (&A)[10], uint32_t n, uint16_t sign) {
  // Q = floor(A / n), r = A mod n, one word at a time from the top
  uint32_t Q[10];
  uint64_t rem = 0;
#pragma unroll
  for (int w = 9; w >= 0; --w) {
    const uint64_t cur = (rem << 32) | A[w];
    Q[w] = static_cast<uint32_t>(cur / n);
    rem = cur - static_cast<uint64_t>(Q[w]) * n;
  }
  const uint32_t r = static_cast<uint32_t>(rem);
  int bl = 0;  // bit length of Q
#pragma unroll
  for (int w = 0; w < 10; ++w)
    if (Q[w]) bl = 32 * w + 32 - __clz(static_cast<int>(Q[w]));
  // value = (Q + r / n) 2^-133; significand m = the value in ulps of its
  // binade (2^(e - 7), e >= -126), which is Q / 2^k with k = max(bl - 8, 0)
  const int k = bl > 8 ? bl - 8 : 0;
  auto bit = [&](int i) -> uint32_t { return (Q[i >> 5] >> (i & 31)) & 1u; };
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (k + i < 320) m |= bit(k + i) << i;
  bool up;
  if (k == 0) {
    up = 2ull * r > n || (2ull * r == n && (m & 1u));
  } else {
    bool sticky = r != 0;
    for (int i = 0; i < k - 1; ++i) sticky = sticky || bit(i);
    up = bit(k - 1) && (sticky || (m & 1u));
  }
  m += up ? 1u : 0u;
  int e = k - 126;  // exponent of the binade (-126 for subnormals)
  if (m == 256) {
    m = 128;
    ++e;
  }
  if (e > 127) return sign | 0x7F80u;
  if (m < 128) return sign | static_cast<uint16_t>(m);  // subnormal (or zero)
  return sign | static_cast<uint16_t>(((e + 127) << 7) | (m - 128));
}

struct KmArgs {
  const uint16_t *x;
  const uint32_t *idx;
  uint16_t *codebook;
  const int32_t *group_map;
  unsigned long long *sums;    // [kReplicas][n_codebooks][n_c][sd], two's complement
  unsigned int *counts;        // [kReplicas][n_codebooks][n_c]
  int64_t n, cb_stride, n_codebooks, group_len, tiles_per_group;
  int sd, n_c;
  int limbs;  // 1 (fp16) or kLimbs (bf16) int64 words per (slot, centroid, component)
  int64_t tile_rows;  // rows per accumulate workgroup (a multiple of kAccThreads * kRowsPerThread)
  int range;          // centroids per accumulate workgroup (their sums fit in LDS)
};

// Member sums of one tile of rows (one group, so one slot) for one range of
// centroids [c0, c0 + range), in LDS, then flushed.  A component with bits
// (sign, exponent field E, fraction F) adds, for fp16, its exact value in
// units of 2^-24 to its one word; for bf16 it is m 2^p units of 2^-133 with
// m = 128 + F, p = E - 1 when E > 0 and m = F, p = 0 when E = 0, and m 2^(p
// mod 32) goes to limb p / 32.  Non-finite components add 0.  A workgroup
// adds at most kAccMaxTileRows rows, so an LDS word stays below 2^16 2^40 =
// 2^56 (fp16) or 2^16 2^39 (bf16) in magnitude.
template <int SD, bool BF16>
__global__ void __launch_bounds__(kAccThreads) km_accumulate(const KmArgs a) {
  constexpr int L = BF16 ? kLimbs : 1;   // words per (centroid, component)
  extern __shared__ unsigned long long tab[];  // [range][SD][L], then counts [range] (u32)
  const int64_t tile = blockIdx.x;
  const int64_t g = tile / a.tiles_per_group;
  const int64_t gstart = g * a.group_len;
  const int64_t gend = min(gstart + a.group_len, a.n);
  const int64_t tbase = gstart + (tile - g * a.tiles_per_group) * a.tile_rows;
  if (tbase >= gend) return;  // whole workgroup
  const int64_t slot = a.group_map ? static_cast<int64_t>(a.group_map[g]) : g;
  if (slot < 0 || slot >= a.n_codebooks) return;  // whole workgroup: no centroid to train
  const int64_t tend = min(tbase + a.tile_rows, gend);
  const int c0 = static_cast<int>(blockIdx.y) * a.range;
  const int nr = min(a.range, a.n_c - c0);  // centroids of this range (>= 1)
  unsigned int *cnt = reinterpret_cast<unsigned int *>(tab + static_cast<int64_t>(a.range) * SD * L);
  for (int e = threadIdx.x; e < nr * SD * L; e += kAccThreads) tab[e] = 0;
  for (int e = threadIdx.x; e < nr; e += kAccThreads) cnt[e] = 0;
  __syncthreads();
  using Row = std::conditional_t<SD == 4, uint2, uint4>;
  const Row *xrows = reinterpret_cast<const Row *>(a.x);
  for (int64_t b0 = tbase + threadIdx.x; b0 < tend; b0 += kAccThreads * kRowsPerThread) {
    // every load of the batch first: the codes, then the rows (a row outside
    // the range loads the tile's first row instead, one shared address)
    uint32_t rel[kRowsPerThread];
    Row xr[kRowsPerThread];
#pragma unroll
    for (int k = 0; k < kRowsPerThread; ++k) {
      const int64_t r = min(b0 + static_cast<int64_t>(k) * kAccThreads, tend - 1);
      rel[k] = a.idx[r] - static_cast<uint32_t>(c0);  // in range: < nr (unsigned)
    }
#pragma unroll
    for (int k = 0; k < kRowsPerThread; ++k) {
      const int64_t r = b0 + static_cast<int64_t>(k) * kAccThreads;
      const bool in = r < tend && rel[k] < static_cast<uint32_t>(nr);
      xr[k] = xrows[in ? r : tbase];
    }
#pragma unroll
    for (int k = 0; k < kRowsPerThread; ++k) {
      const int64_t r = b0 + static_cast<int64_t>(k) * kAccThreads;
      if (r >= tend || rel[k] >= static_cast<uint32_t>(nr)) continue;
      uint32_t w[SD / 2];
      w[0] = xr[k].x;
      w[1] = xr[k].y;
      if constexpr (SD == 8) {
        w[2] = xr[k].z;
        w[3] = xr[k].w;
      }
      unsigned long long *t = tab + static_cast<int64_t>(rel[k]) * SD * L;
#pragma unroll
      for (int i = 0; i < SD; ++i) {
        const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
        if constexpr (BF16) {
          const uint32_t E = (bits >> 7) & 0xFFu, F = bits & 0x7Fu;
          const uint32_t m = (E == 0) ? F : (128u | F);
          if (E == 255u || m == 0) continue;  // non-finite adds 0
          const uint32_t p = (E == 0) ? 0u : E - 1u;
          const uint64_t v = static_cast<uint64_t>(m) << (p & 31u);
          atomicAdd(t + i * L + (p >> 5), (bits & 0x8000u) ? 0ull - v : v);
        } else {
          const unsigned long long u = static_cast<unsigned long long>(units(static_cast<uint16_t>(bits)));
          if (u) atomicAdd(t + i, u);
        }
      }
      atomicAdd(cnt + rel[k], 1u);
    }
  }
  __syncthreads();
  const int64_t cells = a.n_codebooks * a.n_c;
  const int rep = static_cast<int>(blockIdx.x % kReplicas);
  unsigned long long *gs = a.sums + ((rep * cells + slot * a.n_c + c0) * SD) * L;
  unsigned int *gc = a.counts + rep * cells + slot * a.n_c + c0;
  for (int e = threadIdx.x; e < nr * SD * L; e += kAccThreads)
    if (tab[e]) atomicAdd(gs + e, tab[e]);
  for (int e = threadIdx.x; e < nr; e += kAccThreads)
    if (cnt[e]) atomicAdd(gc + e, cnt[e]);
}

// New bf16 centroids from the limbs, one thread per (slot, centroid,
// component); the workgroup then clears what it read (as km_update).
template <int SD>
__global__ void __launch_bounds__(kThreads) km_update_bf16(const KmArgs a) {
  const int64_t cells = a.n_codebooks * a.n_c;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * (kThreads / SD) + threadIdx.x / SD;
  const int i = threadIdx.x % SD;
  const bool live = e < cells;
  if (live) {
    unsigned int cnt = 0;
#pragma unroll
    for (int r = 0; r < kReplicas; ++r) cnt += a.counts[r * cells + e];
    if (cnt > 0) {
      // limb sums over the replicas (together below 2^62 in magnitude: the
      // members are split between the replicas), then the carries into 10
      // words of a 320-bit two's complement integer
      uint32_t W[10];
      int64_t carry = 0;
#pragma unroll
      for (int j = 0; j < kLimbs; ++j) {
        int64_t L = 0;
#pragma unroll
        for (int r = 0; r < kReplicas; ++r)
          L += static_cast<int64_t>(a.sums[((r * cells + e) * SD + i) * kLimbs + j]);
        const int64_t t = L + carry;
        W[j] = static_cast<uint32_t>(t);
        carry = t >> 32;  // arithmetic: floor(t / 2^32)
      }
#pragma unroll
      for (int j = kLimbs; j < 10; ++j) {  // the carry's words, sign-extended
        W[j] = static_cast<uint32_t>(carry);
        carry >>= 32;
      }
      const bool neg = carry < 0;
      if (neg) {  // magnitude: invert and add one
        uint64_t c1 = 1;
#pragma unroll
        for (int j = 0; j < 10; ++j) {
          const uint64_t t = static_cast<uint64_t>(~W[j]) + c1;
          W[j] = static_cast<uint32_t>(t);
          c1 = t >> 32;
        }
      }
      const int64_t slot = e / a.n_c;
      const int64_t c = e - slot * a.n_c;
      a.codebook[slot * a.cb_stride + c * SD + i] =
          round_mean_bf16(W, cnt, neg ? static_cast<uint16_t>(0x8000u) : static_cast<uint16_t>(0));
    }
  }
  __syncthreads();
  if (live) {
#pragma unroll
    for (int r = 0; r < kReplicas; ++r) {
#pragma unroll
      for (int j = 0; j < kLimbs; ++j) a.sums[((r * cells + e) * SD + i) * kLimbs + j] = 0;
      if (i == 0) a.counts[r * cells + e] = 0;
    }
  }
}

// New centroids from the sums, one thread per (slot, centroid, component);
// a workgroup holds whole centroids, and clears their sums and counts for
// the next iteration once all of its threads have read them.
template <int SD>
__global__ void __launch_bounds__(kThreads) km_update(const KmArgs a) {
  const int64_t cells = a.n_codebooks * a.n_c;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * (kThreads / SD) + threadIdx.x / SD;
  const int i = threadIdx.x % SD;
  const bool live = e < cells;
  unsigned int cnt = 0;
  unsigned long long S = 0;  // two's complement: the sum wraps like int64
  if (live) {
#pragma unroll
    for (int r = 0; r < kReplicas; ++r) {
      cnt += a.counts[r * cells + e];
      S += a.sums[(r * cells + e) * SD + i];
    }
    if (cnt > 0) {
      const int64_t slot = e / a.n_c;
      const int64_t c = e - slot * a.n_c;
      a.codebook[slot * a.cb_stride + c * SD + i] = round_mean_f16(static_cast<int64_t>(S), cnt);
    }
  }
  __syncthreads();
  if (live) {
#pragma unroll
    for (int r = 0; r < kReplicas; ++r) {
      a.sums[(r * cells + e) * SD + i] = 0;
      if (i == 0) a.counts[r * cells + e] = 0;
    }
  }
}

__global__ void __launch_bounds__(kThreads) km_clear(const KmArgs a) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t nc = kReplicas * a.n_codebooks * a.n_c;
  if (e < nc * a.sd * a.limbs) a.sums[e] = 0;
  if (e < nc) a.counts[e] = 0;
}

// LDS of an accumulate workgroup: the sums of `range` centroids, then their
// counts.
size_t acc_lds_bytes(int sd, int limbs, int range) {
  return static_cast<size_t>(range) * (sd * limbs * sizeof(unsigned long long) + sizeof(unsigned int));
}

// Centroids per accumulate workgroup: all of them when their sums fit, else
// the largest power of two that does.
int acc_range(int sd, int limbs, int n_c) {
  if (acc_lds_bytes(sd, limbs, n_c) <= kAccLdsBytes) return n_c;
  int r = 1;
  while (acc_lds_bytes(sd, limbs, 2 * r) <= kAccLdsBytes) r *= 2;
  return r;
}

// Rows per accumulate workgroup: about one workgroup per CU over all tiles
// and ranges, in whole rounds of kRowsPerBatch, at most kAccMaxTileRows.
int64_t acc_tile_rows(int64_t span, int64_t n_groups, int ranges) {
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const int64_t target = (span * n_groups * ranges + cus - 1) / cus;
  int64_t rows = (target + kRowsPerBatch - 1) / kRowsPerBatch * kRowsPerBatch;
  const int64_t span_rounded = (span + kRowsPerBatch - 1) / kRowsPerBatch * kRowsPerBatch;
  rows = std::min(rows, std::min(kAccMaxTileRows, span_rounded));
  return std::max<int64_t>(rows, kRowsPerBatch);
}

template <int SD>
hipError_t launch_km(const KmArgs &a, const Layout &l, int iterations, hipStream_t stream) {
  const int64_t cells = a.n_codebooks * a.n_c;
  const int64_t clear_blocks = (kReplicas * cells * SD * a.limbs + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(km_clear, dim3(static_cast<uint32_t>(clear_blocks)), dim3(kThreads), 0,
                     stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t tiles = a.tiles_per_group * ((a.n + a.group_len - 1) / a.group_len);
  const int ranges = (a.n_c + a.range - 1) / a.range;
  const dim3 acc_grid(static_cast<uint32_t>(tiles), static_cast<uint32_t>(ranges));
  const size_t lds = acc_lds_bytes(SD, a.limbs, a.range);
  auto acc = l.bf16 ? km_accumulate<SD, true> : km_accumulate<SD, false>;
  if (lds > 65536) {
    err = hipFuncSetAttribute(reinterpret_cast<const void *>(acc),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (err != hipSuccess) return err;
  }
  const int64_t upd_blocks = (cells * SD + kThreads - 1) / kThreads;
  if (l.bf16) {
    for (int it = 0; it < iterations; ++it) {
      err = encode_mfma_supported(l)
                ? launch_encode_mfma(a.x, a.codebook, a.group_map, const_cast<uint32_t *>(a.idx),
                                     l, plain_codes(l), stream)
                : launch_encode(a.x, a.codebook, a.group_map, const_cast<uint32_t *>(a.idx), l,
                                plain_codes(l), stream);
      if (err != hipSuccess) return err;
      hipLaunchKernelGGL(acc, acc_grid, dim3(kAccThreads), lds, stream, a);
      err = hipGetLastError();
      if (err != hipSuccess) return err;
      hipLaunchKernelGGL(km_update_bf16<SD>, dim3(static_cast<uint32_t>(upd_blocks)),
                         dim3(kThreads), 0, stream, a);
      err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    return hipSuccess;
  }
  // up to 512 fp16 centroids the encode adds the member sums itself
  const bool fused = encode_mfma_kmeans_supported(l);
  for (int it = 0; it < iterations; ++it) {
    if (fused) {
      err = launch_encode_mfma_kmeans(a.x, a.codebook, a.group_map, const_cast<uint32_t *>(a.idx),
                                      l, KmSums{a.sums, a.counts}, stream);
      if (err != hipSuccess) return err;
      hipLaunchKernelGGL(km_update<SD>, dim3(static_cast<uint32_t>(upd_blocks)), dim3(kThreads), 0,
                         stream, a);
      err = hipGetLastError();
      if (err != hipSuccess) return err;
      continue;
    }
    err = encode_mfma_supported(l)
              ? launch_encode_mfma(a.x, a.codebook, a.group_map, const_cast<uint32_t *>(a.idx), l,
                                   plain_codes(l), stream)
              : launch_encode(a.x, a.codebook, a.group_map, const_cast<uint32_t *>(a.idx), l,
                              plain_codes(l), stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(acc, acc_grid, dim3(kAccThreads), lds, stream, a);
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

size_t kmeans_workspace_bytes(int sub_dim, int n_centroids, int64_t n_codebooks, bool bf16) {
  const int limbs = bf16 ? kLimbs : 1;
  const uint64_t cell = sub_dim * limbs * sizeof(unsigned long long) + sizeof(unsigned int);
  uint64_t r = 0;
  // 0 when the size does not fit in 63 bits (the caller rejects it)
  if (n_codebooks < 1 || n_centroids < 1 ||
      __builtin_mul_overflow(static_cast<uint64_t>(n_codebooks), static_cast<uint64_t>(n_centroids), &r) ||
      __builtin_mul_overflow(r, cell * kReplicas, &r) || r > static_cast<uint64_t>(INT64_MAX))
    return 0;
  return static_cast<size_t>(r);
}

int64_t kmeans_grid(const Layout &l) {
  // upper bound on the accumulate workgroups along x (tiles of at least
  // kRowsPerBatch rows)
  const int64_t span = l.group_len < l.n ? l.group_len : l.n;
  return (span + kRowsPerBatch - 1) / kRowsPerBatch * l.n_groups;
}

hipError_t launch_kmeans(const void *x, void *codebook, const int32_t *group_map, uint32_t *out_idx,
                         const Layout &l, int iterations, void *workspace, hipStream_t stream) {
  KmArgs a;
  a.x = static_cast<const uint16_t *>(x);
  a.idx = out_idx;
  a.codebook = static_cast<uint16_t *>(codebook);
  a.group_map = group_map;
  a.sums = static_cast<unsigned long long *>(workspace);
  a.limbs = l.bf16 ? kLimbs : 1;
  a.counts = reinterpret_cast<unsigned int *>(a.sums + kReplicas * l.n_codebooks * l.n_centroids *
                                                           l.sub_dim * a.limbs);
  a.n = l.n;
  a.cb_stride = l.codebook_stride;
  a.n_codebooks = l.n_codebooks;
  a.group_len = l.group_len;
  const int64_t span = l.group_len < l.n ? l.group_len : l.n;
  a.sd = l.sub_dim;
  a.n_c = l.n_centroids;
  a.range = acc_range(l.sub_dim, a.limbs, l.n_centroids);
  a.tile_rows = acc_tile_rows(span, l.n_groups, (l.n_centroids + a.range - 1) / a.range);
  a.tiles_per_group = (span + a.tile_rows - 1) / a.tile_rows;
  return l.sub_dim == 4 ? launch_km<4>(a, l, iterations, stream)
                        : launch_km<8>(a, l, iterations, stream);
}

}  // namespace vqk
