// vq_encode_mfma.hip -- product-VQ encode on gfx950 matrix cores, exact result.
//
// The operation (VeloxQuant-MLX blog, "I Wrote a Metal Kernel to Stop My Mac
// From OOMing", sections "What quantize_vq Was Doing Wrong" and "The Kernel: 18
// Lines of MSL") is the strict-< argmin over centroids of the fp32 distance
// d = x_i - c_i, dist = fma(d, d, dist) (components in order).  This kernel
// returns exactly that index; it uses the matrix cores only to find, cheaply,
// the few centroids that can possibly win.
//
// Stage 1 (one v_mfma_f32_32x32x8 per 32 centroids x 32 sub-vectors):
//   M(c) = C(c) - x.c, with C(c) = |c|^2/2 shrunk by the error bound below.
//   Products of fp16/bf16 inputs are exact in fp32; the matrix unit's
//   accumulation of the m = sub_dim + 1 nonzero terms errs by at most
//   eta_m (sum |terms|), eta_m = 2 (m + 1) u, u = 2^-24 (one rounding of at
//   most 2u per addition, in any order; measured below 5u on gfx950).  Each
//   lane holds 16 of the 32 rows of a block: one "group" of 16 rows, or, for
//   codebooks of up to 256 centroids, two groups of 8.  The group minimum of
//   M minus a(g) b(x), with a(g) >= kappa max_{c in g} |c| and b(x) >= |x|,
//   bounds every centroid of the group from below:
//       L(g) <= s(c) = |c|^2/2 - x.c   for all c in g,
//   and |x - c|^2 = |x|^2 + 2 s(c), so ranking by s is ranking by distance.
//   Per sub-vector the lanes keep the smallest group bound m1, its group g1
//   and the second smallest group bound m2.  With 8-row groups (at most 16
//   per lane) the index of g1 rides in the 4 low mantissa bits of the bound
//   itself, so one min and one med3 keep all three: writing those bits moves
//   a bound by less than 2^-19 of its magnitude plus 15 subnormal steps, and
//   the bounds of this form are built with that much more slack (C shrunk
//   and kappa grown by 2^-19 (1 + 2^-10) more, one more 2^-140 off C).
// Stage 2 (exact): the rows of g1 are evaluated in the fixed fp32
//   arithmetic above (8 or 4 rows on each lane of the pair that shares the
//   sub-vector).  With D the smallest such distance, the oracle's winner c*
//   satisfies s(c*) <= U = (D (1 + 2 gamma) - |x|^2_low) / 2, gamma = (sub_dim
//   + 2) u (rounding bound of the fp32 distance), so its group's bound is
//   <= U.  If m2 > U no centroid outside g1 can be c*, and the lowest-index
//   minimum over g1 is the answer, bit for bit.  Otherwise the sub-vector is
//   ambiguous: every group whose bound is <= U is recomputed exactly (the
//   bounds are recomputed on the matrix cores), which again contains c*.
//   Non-finite or huge values take a full exact strict-< scan.
// Exact duplicate rows: a row bit-identical to an earlier row has the same
//   fp32 distance and can never win the strict-< scan; such rows are found
//   with an LDS hash table per workgroup and excluded from stage 1 (C = +inf),
//   so they do not make every nearby sub-vector ambiguous.
// Smoothed keys (SCALED): the search runs on x~ = x * f (fp32, per-channel
//   factors f).  x~ is not an fp16/bf16 value, so stage 1 splits it exactly
//   as x~ = hi + lo + e with hi = rn(x~), lo = rn(x~ - hi) in the element
//   type (both subtractions are exact) and multiplies [hi, lo] by [-c, -c]:
//   2 sub_dim products, which fill the K = 8 slots at sub_dim 4 and take the
//   K = 16 instruction (same issue cost) at sub_dim 8.  The bound uses
//   eta for 2 sub_dim + 1 terms and |x| replaced by |(|hi| + |lo|)|, and the
//   residual adds |e . c| <= max|c| sum|e_i|.  Stage 2 recomputes x~ in fp32
//   and is unchanged.  (Measured on gfx950 for both instruction shapes: the
//   accumulation error stays below 4 u sum|terms| plus a fraction of the
//   smallest subnormal.)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

#include "vq_codes.h"
#include "vq_launch.h"

namespace vqk {
namespace {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMfmaMaxCentroids = 4096;    // whole codebook slot resident in LDS
constexpr int kRows32MaxCentroids = 1024;  // up to here an fp32 copy is kept too
// K-means sums: rows a workgroup adds up before it flushes.  Every fp16 value
// is a multiple of 2^-24 below 2^16 in magnitude, so a sum of at most 2^13 of
// them is a multiple of 2^-24 below 2^29: exact in fp64 in any order.
constexpr int kAccMaxRows = 8192;
constexpr float kU = 5.9604644775390625e-08f;       // 2^-24
constexpr float kTau = 7.174648137343064e-43f;      // 2^-140: absolute slack
constexpr float kNormCap = 1.2676506002282294e30f;  // 2^100: beyond it, exact path
constexpr float kNormUp = 1.0000038146972656f;      // 1 + 2^-18: upward norm margin
constexpr float kNegMax = -3.4028234663852886e38f;  // med3(a, b, kNegMax) = min(a, b)
constexpr float kFltMax = 3.4028234663852886e38f;
constexpr float kBnUp = 1.0000019073486328f;        // 1 + 2^-19

// SD: sub-vector length; NT: products per matrix-core dot (SD, or 2 SD for
// the hi/lo split of smoothed keys).
template <int SD, int NT>
struct Consts {
  static constexpr float kEta = (2.0f * (NT + 2) + 2.0f) * kU;  // eta_m + 2u (final fma)
  static constexpr float kKappa = 1.125f * kEta;                // > eta / (1 - u)
  static constexpr float kInvKappaUp = (1.0f / kKappa) * 1.0000152587890625f;  // >= 1/kappa
  static constexpr float kHalfShrink = 0.5f * (1.0f - kEta - 9.5367431640625e-07f);
  static constexpr float kGamma2 = 2.0f * (SD + 2) * kU * 1.01f;  // >= 1/(1-gamma) - 1
  // U = fma(best, kUA, fma(n2x, -kUB, kTau)) >= (best (1 + kGamma2) - |x|^2_low) / 2
  // with |x|^2_low = n2x (1 - (SD + 2) u) <= |x|^2: kUB carries 8u less than
  // the exact factor and kUA 8u more, which covers the two roundings (each at
  // most u of its result's magnitude, plus 2^-150 absolute, inside kTau) and
  // the rounding of the constants themselves.
  static constexpr float kUA = 0.5f * (1.0f + kGamma2) * (1.0f + 8.0f * kU);
  static constexpr float kUB = 0.5f * (1.0f - (SD + 2) * kU) * (1.0f - 8.0f * kU);
  // Small codebooks carry the group index in the 4 low bits of a bound,
  // which moves it by at most 15 ulps: less than 2^-19 = 32 u of its
  // magnitude for a normal bound, at most 15 2^-149 otherwise.  The bound is
  // built with 32 u (1 + 2^-10) more relative slack in both C and kappa
  // (which covers 32 u (1 + eta) of |C| + |x||c| + a'b', the largest the
  // bound can be), and one more kTau of absolute slack in C.
  static constexpr float kEtaIdx = kEta + 32.0f * kU * 1.0009765625f;
  static constexpr float kKappaIdx = 1.125f * kEtaIdx;
  static constexpr float kInvKappaIdxUp = (1.0f / kKappaIdx) * 1.0000152587890625f;
  static constexpr float kHalfShrinkIdx = 0.5f * (1.0f - kEtaIdx - 9.5367431640625e-07f);
};

// Codebooks of up to kSmallMaxCentroids (8 blocks of 32 rows) use groups of
// 8 rows and keep the group index in the bound itself (SMALL); larger ones
// use groups of 16 rows and keep the index in a register of its own.
constexpr int kSmallMaxCentroids = 256;
constexpr uint32_t kIdxMask = 15u;  // 2 groups per block and lane, <= 8 blocks

// Sub_dim 4 leaves K slots of the matrix-core dot empty; they carry C and
// the error term instead ("folded").  Plain keys (K = 8): A = [-c, C_hi,
// C_lo, -a', 0], B = [x, 1, 1, b', 0].  Smoothed keys (K = 16, the split
// x~ = hi + lo + e): A = [-c, -c, C_hi, C_lo, -a', 0 x 5], B = [hi, lo, 1, 1,
// b', 0 x 5].  a' >= kFoldScale a(g) (g the row's group) and b' >= b(x) /
// kFoldScale are element-type values rounded up, so a' b' >= a(g) b(x) and
// the dot is already the group's lower bound: the accumulator input is
// zero, and neither C nor a(g) is loaded per block.
template <int SD, bool SCALED>
constexpr bool kFold = (SD == 4);
// In fp16 a folded slot has C_hi finite, so |c| <= 362 and a(g) < 2^-11,
// and fp16 keys have |x| < 2^18: with the scale, a' < 1 and b' < 2^8.  In
// bf16 both stay far inside the range (|c|, |x| < 2^50).
constexpr float kFoldScale = 1024.0f;

// Products per matrix-core dot for the error bound (one more term, the
// accumulator input or the folded error term, is counted by Consts).
template <int SD, bool SCALED>
constexpr int kTerms = (SCALED ? 2 * SD : SD) + (kFold<SD, SCALED> ? 2 : 0);

template <bool BF16>
constexpr uint16_t kInfBits = BF16 ? 0x7F80 : 0x7C00;
template <bool BF16>
constexpr uint32_t kOnePair = BF16 ? 0x3F803F80u : 0x3C003C00u;  // (1, 1)

// Matrix-core operands: 4 halves per lane (K = 8), or 8 (K = 16) for
// smoothed keys.
template <int SD, bool SCALED>
using Op = std::conditional_t<SCALED, uint4, uint2>;

template <bool BF16>
__device__ __forceinline__ float widen(uint16_t v) {
  if constexpr (BF16) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
  } else {
    return static_cast<float>(__builtin_bit_cast(_Float16, v));
  }
}

// fp32 -> element bits, rounded to nearest even (overflow gives +-inf).
template <bool BF16>
__device__ __forceinline__ uint16_t narrow(float v) {
  if constexpr (BF16) {
    const uint32_t u = __float_as_uint(v);
    return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
  } else {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
  }
}

// Upper bound of sqrt(v) for 0 <= v <= 2^100 (no correctly rounded square
// root is needed): the hardware square root is within 1 ulp for normal
// inputs, which kNormUp (1 + 2^-18) covers many times over, and below the
// normal range sqrt(v) < 2^-63, covered by the floor.
__device__ __forceinline__ float sqrt_up(float v) {
  return fmaxf(__builtin_amdgcn_sqrtf(v) * kNormUp, 2.168404344971009e-19f /* 2^-62 */);
}

// The B value b' >= b / kFoldScale of the folded error term (b >= 0).  fp16:
// one fused multiply-add rounded once to fp16; the 2^-10 relative and 2^-24
// absolute margins exceed fp16's rounding error in the normal (2^-11
// relative) and subnormal (2^-25 absolute) ranges.
template <bool BF16>
__device__ __forceinline__ uint16_t fold_b(float b);

// Smallest element-type value >= v, for v >= 0 (+inf when v exceeds the
// largest finite value).
template <bool BF16>
__device__ __forceinline__ uint16_t round_up(float v) {
  const uint16_t b = narrow<BF16>(v);
  return (widen<BF16>(b) < v) ? static_cast<uint16_t>(b + 1u) : b;
}

template <bool BF16>
__device__ __forceinline__ uint16_t fold_b(float b) {
  if constexpr (BF16) {
    return round_up<true>(b * (1.0f / kFoldScale));
  } else {
    constexpr float k = (1.0f / kFoldScale) * (1.0f + 1.0f / 1024.0f);
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(__builtin_fmaf(b, k, 5.960464477539063e-08f)));
  }
}

// C = hi + lo with hi = rn(C) and lo = C - hi rounded toward -inf (C - hi is
// exact), so hi + lo <= C and the folded bound stays a lower bound.  False
// when hi overflows the element type.
template <bool BF16>
__device__ __forceinline__ bool split_down(float c, uint16_t &hi, uint16_t &lo) {
  if (c == __builtin_inff()) {
    hi = kInfBits<BF16>;
    lo = 0;
    return true;
  }
  hi = narrow<BF16>(c);
  const float hf = widen<BF16>(hi);
  if (!(__builtin_fabsf(hf) <= kFltMax)) return false;
  const float r = c - hf;
  uint16_t l = narrow<BF16>(r);
  if (widen<BF16>(l) > r) {  // one step toward -inf
    if ((l & 0x7FFFu) == 0) {
      l = 0x8001u;            // -(smallest subnormal)
    } else if (l & 0x8000u) {
      l = static_cast<uint16_t>(l + 1u);
    } else {
      l = static_cast<uint16_t>(l - 1u);
    }
  }
  lo = l;
  return true;
}

template <int SD>
__device__ __forceinline__ float sqdist(const float (&xv)[SD], const float (&c)[SD]) {
  float d = xv[0] - c[0];
  float acc = d * d;  // = fma(d, d, +0)
#pragma unroll
  for (int i = 1; i < SD; ++i) {
    d = xv[i] - c[i];
    acc = __builtin_fmaf(d, d, acc);
  }
  return acc;
}

// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>): the body
// is instantiated once per index, so per-column arrays are indexed by
// constants (never moved to scratch) however large the body is.
template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F &&f) {
  unroll_seq(f, std::make_integer_sequence<int, N>{});
}

// Element j of the 16-bit values packed in w (two per word).
__device__ __forceinline__ uint16_t half_of(const uint32_t *w, int j) {
  return static_cast<uint16_t>((j & 1) ? (w[j >> 1] >> 16) : w[j >> 1]);
}

template <int SD, bool BF16>
__device__ __forceinline__ void widen_words(const uint32_t *w, uint16_t flip, float (&v)[SD]) {
#pragma unroll
  for (int i = 0; i < SD; ++i) v[i] = widen<BF16>(half_of(w, i) ^ flip);
}

template <int SD>
__device__ __forceinline__ uint32_t hash_row(const uint4 &q) {
  uint32_t h = 0x9e3779b9u;
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < SD / 2; ++i) {
    h ^= w[i];
    h *= 0x85ebca6bu;
    h ^= h >> 13;
  }
  return h * 0xc2b2ae35u;
}

template <int SD>
__device__ __forceinline__ bool same_row(const uint4 &a, const uint4 &b) {
  return (SD == 4) ? (a.x == b.x && a.y == b.y)
                   : (a.x == b.x && a.y == b.y && a.z == b.z && a.w == b.w);
}

template <bool BF16>
__device__ __forceinline__ f32x16 mfma(const uint2 &a, const uint2 &b, const f32x16 &c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(f16x4, a),
                                                __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
}

template <bool BF16>
__device__ __forceinline__ f32x16 mfma(const uint4 &a, const uint4 &b, const f32x16 &c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// An empty use of a value: the loads that produce it are issued before this
// point (the compiler may otherwise sink them past a branch to their use).
__device__ __forceinline__ void hold(float v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void hold(const uint2 &v) { asm volatile("" ::"v"(v.x), "v"(v.y)); }
__device__ __forceinline__ void hold(const uint4 &v) {
  asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w));
}

// Minimum of the 16 values (finite or +inf).  The first step is a med3 with
// -FLT_MAX, which equals min for such values and needs no NaN quieting.
__device__ __forceinline__ float min16(const f32x16 &v) {
  float a = __builtin_amdgcn_fmed3f(v[0], v[1], kNegMax);
  a = fminf(fminf(a, v[2]), v[3]);
  a = fminf(fminf(a, v[4]), v[5]);
  a = fminf(fminf(a, v[6]), v[7]);
  a = fminf(fminf(a, v[8]), v[9]);
  a = fminf(fminf(a, v[10]), v[11]);
  a = fminf(fminf(a, v[12]), v[13]);
  return fminf(fminf(a, v[14]), v[15]);
}

// Minimum of the 8 values v[LO] .. v[LO + 7], at most FLT_MAX (an infinite
// minimum, a group of marked rows only, becomes FLT_MAX: still a lower
// bound, and finite, so that writing index bits into it cannot make a NaN).
template <int LO>
__device__ __forceinline__ float min8(const f32x16 &v) {
  float a = __builtin_fminf(__builtin_fminf(v[LO], v[LO + 1]), kFltMax);
  a = fminf(fminf(a, v[LO + 2]), v[LO + 3]);
  a = fminf(fminf(a, v[LO + 4]), v[LO + 5]);
  return fminf(fminf(a, v[LO + 6]), v[LO + 7]);
}

// The two lanes of a pair are l and l + 32 (h = 0, 1): they sit in the two
// 32-lane halves of the wave.  v_permlane32_swap trades the upper half of one
// register with the lower half of another on the VALU; with both operands
// equal to v it gives, in every lane, v of the pair's lane 0 (first) and v
// of its lane 1 (second), without the LDS round trip of a ds_bpermute.
struct PairVals {
  uint32_t first, second;
};
__device__ __forceinline__ PairVals pair_vals(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return {static_cast<uint32_t>(r[0]), static_cast<uint32_t>(r[1])};
}
// v of the other lane of the pair
__device__ __forceinline__ uint32_t pair_other(uint32_t v, int h) {
  const PairVals p = pair_vals(v);
  return h ? p.first : p.second;
}
__device__ __forceinline__ float pair_other(float v, int h) {
  return __builtin_bit_cast(float, pair_other(__builtin_bit_cast(uint32_t, v), h));
}
__device__ __forceinline__ int pair_other(int v, int h) {
  return static_cast<int>(pair_other(static_cast<uint32_t>(v), h));
}
// v(lane 0) + v(lane 1), the same value in both lanes
__device__ __forceinline__ float pair_sum(float v) {
  const PairVals p = pair_vals(__builtin_bit_cast(uint32_t, v));
  return __builtin_bit_cast(float, p.first) + __builtin_bit_cast(float, p.second);
}

// Per-workgroup LDS (dynamic) for one codebook slot of n_c centroids, padded
// to n_cpad = roundup(n_c, 32):
//   rows [n_cpad] uint4     A operand: halves 0..7 = -c_0 .. -c_{SD-1}, zero
//                           padded (K = 8; lane half h reads halves 4h..4h+3);
//   cval [n_cpad] float     C operand: shrunk |c|^2/2, +inf for padding and
//                           duplicate rows;
//   gan  [groups] float     per group (16 rows, or 8 when n_cpad <= 256):
//                           kappa max |c| (rounded up);
//   c32                     the centroids in fp32 (ROWS32 only; +inf in the
//                           padding rows), row r at
//                           c32_offset(r): 16 bytes of padding after every
//                           4 rows and after every 16, so that the rows the
//                           lanes of a wave read together in the exact stage
//                           (same position in different groups) fall on
//                           different LDS banks;
//   hash [hash_slots] uint  duplicate detection while staging;
//   flags [16] int          per-wave staging flags, then the unit counter;
//   scale [head_dim] float  the slot's channel factors (smoothed keys only).
// gan is padded to a multiple of 4 floats so every region is 16-byte aligned.
template <int SD, bool ROWS32>
struct Lds {
  static constexpr int kFlags = 16;  // one per wave, at most 1024 threads
  static constexpr int kCounter = kFlags;  // flags[kCounter]: next unit of the segment
  uint4 *arows;  // smoothed sub_dim 4: the K = 16 A operand, one 16-byte half per lane half
  uint4 *rows;
  float *cval;
  float *gan;
  float *c32;
  uint32_t *hash;
  int *flags;
  float *scale;
  // (8-row groups only where n_cpad <= kSmallMaxCentroids)
  static constexpr int gan_len(int n_cpad) {
    return ((n_cpad <= kSmallMaxCentroids ? n_cpad / 8 : n_cpad / 16) + 3) & ~3;
  }
  // floats of the c32 region, and the float offset of row r in it
  static constexpr int c32_len(int n_cpad) {
    return ROWS32 ? SD * n_cpad + 4 * (n_cpad / 4 + n_cpad / 16 + 1) : 0;
  }
  static __device__ __forceinline__ int c32_offset(int r) { return SD * r + 4 * ((r >> 2) + (r >> 4)); }
  __device__ Lds(uint4 *base, int n_cpad, int hash_slots, int arows_len) {
    arows = base;
    rows = base + arows_len;
    cval = reinterpret_cast<float *>(rows + n_cpad);
    gan = cval + n_cpad;
    c32 = gan + gan_len(n_cpad);
    hash = reinterpret_cast<uint32_t *>(c32 + c32_len(n_cpad));
    flags = reinterpret_cast<int *>(hash + hash_slots);
    scale = reinterpret_cast<float *>(flags + kFlags + 4);
  }
  static size_t bytes(int n_cpad, int hash_slots, int scale_len, int arows_len) {
    return static_cast<size_t>(arows_len) * 16 + static_cast<size_t>(n_cpad) * (16 + 4) + static_cast<size_t>(c32_len(n_cpad)) * 4 +
           static_cast<size_t>(gan_len(n_cpad)) * 4 + static_cast<size_t>(hash_slots) * 4 +
           (kFlags + 4) * 4 + static_cast<size_t>(scale_len) * 4;
  }
};

// In the matrix-core result the lane of half hh holds rows 32 b + 8 j + 4 hh
// + i (j, i = 0..3) of block b.  Group of row r = 32 b + 16 q + 8 j' + 4 hh
// + i: 2 b + hh (16 rows: the lane's 16 values), or with SMALL 4 b + 2 q + hh
// (8 rows: the lane's first 8 values, q = 0, or its last 8, q = 1).
template <bool SMALL>
__device__ __forceinline__ int group_of(int r) {
  return SMALL ? 4 * (r >> 5) + 2 * ((r >> 4) & 1) + ((r >> 2) & 1)
               : 2 * (r >> 5) + ((r >> 2) & 1);
}

// Row i (0..3) of the 4-row set starting at c0 (a multiple of 4) as fp32,
// from the fp32 copy (the set is contiguous there) or widened from the
// staged -c bits.
template <int SD, bool BF16, bool ROWS32>
__device__ __forceinline__ void centroid_in_set(const Lds<SD, ROWS32> &s, int c0, int i,
                                                float (&v)[SD]) {
  if constexpr (ROWS32) {
    const float *base = s.c32 + s.c32_offset(c0) + SD * i;
#pragma unroll
    for (int q = 0; q < SD / 4; ++q) {
      const float4 w = *reinterpret_cast<const float4 *>(base + 4 * q);
      v[4 * q] = w.x;
      v[4 * q + 1] = w.y;
      v[4 * q + 2] = w.z;
      v[4 * q + 3] = w.w;
    }
  } else {
    const uint4 q = s.rows[c0 + i];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    widen_words<SD, BF16>(w, 0x8000u, v);
  }
}

// Centroid c as fp32.
template <int SD, bool BF16, bool ROWS32>
__device__ __forceinline__ void centroid(const Lds<SD, ROWS32> &s, int c, float (&v)[SD]) {
  centroid_in_set<SD, BF16, ROWS32>(s, c & ~3, c & 3, v);
}

// Maximum over the lanes that hold the rows of one group, where lane l of a
// staging pass holds row base + l: the lanes that agree on bits 2 and 5 of
// the lane index (16 rows), and on bit 4 too with SMALL (8 rows).
// Non-negative floats order like their bit patterns.
template <bool SMALL>
__device__ __forceinline__ float group_max(float v) {
  int b = __float_as_int(v);
  b = max(b, __builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, false));   // lane ^ 1
  b = max(b, __builtin_amdgcn_update_dpp(0, b, 0x4E, 0xF, 0xF, false));   // lane ^ 2
  b = max(b, __builtin_amdgcn_update_dpp(0, b, 0x128, 0xF, 0xF, false));  // lane ^ 8
  if constexpr (SMALL) return __int_as_float(b);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);     // lane ^ 16
  return __int_as_float(max(static_cast<int>(r[0]), static_cast<int>(r[1])));
}

// Stage one codebook slot (and, for smoothed keys, its channel factors).
// Returns true when some centroid has a non-finite or huge norm: then every
// sub-vector of the slot takes the full exact scan.  One barrier, after the
// rows are written; duplicate rows are marked after it.
template <int SD, int NT, bool BF16, bool ROWS32, int BLOCK, bool FOLD, bool AROWS, bool SMALL>
__device__ bool stage_codebook(const uint16_t *__restrict__ cb, int n_c, int n_cpad,
                               const Lds<SD, ROWS32> &s, int hash_slots,
                               const float *__restrict__ scale, int scale_len, bool last_waves,
                               bool &fold_ok) {
  using K = Consts<SD, NT>;
  constexpr uint32_t kEmpty = 0xFFFFFFFFu;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int i = tid; i < hash_slots; i += BLOCK) s.hash[i] = kEmpty;
  for (int i = tid; i < scale_len; i += BLOCK) s.scale[i] = scale ? scale[i] : 1.0f;
  int flag = 0, nofold = 0;
  // whole waves per pass (n_cpad is a multiple of 32, so a group never
  // straddles the end), which keeps the group maximum's lane exchanges
  // uniform.  With fewer units than waves (last_waves) the last waves of
  // the workgroup stage the rows and mark the duplicates below, so that the
  // first waves, which take the units, start right after the barrier;
  // otherwise the first waves do it (the issue arbiter favours them, and
  // the last waves would end late).
  const int rwave = last_waves ? BLOCK / 64 - 1 - wave : wave;
  for (int base = rwave * 64; base < n_cpad; base += BLOCK) {
    const int r = base + lane;
    uint16_t k8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // padding rows (r >= n_c) keep +inf in the fp32 copy: their exact
    // distance is +inf, so the exact stage needs no row mask there
    float v[SD];
#pragma unroll
    for (int i = 0; i < SD; ++i) v[i] = __builtin_inff();
    float cv = __builtin_inff();
    float an = 0.0f;
    if (r < n_c) {
      // element loads: a slot only has to be 2-byte aligned
      const uint16_t *p = cb + static_cast<int64_t>(r) * SD;
#pragma unroll
      for (int i = 0; i < SD; ++i) {
        const uint16_t e = p[i];
        v[i] = widen<BF16>(e);
        k8[i] = e ^ 0x8000u;  // -c, exact
      }
      float n2c = v[0] * v[0];
#pragma unroll
      for (int i = 1; i < SD; ++i) n2c = __builtin_fmaf(v[i], v[i], n2c);
      if (!(n2c <= kNormCap)) {
        flag = 1;
      } else {
        cv = SMALL ? n2c * K::kHalfShrinkIdx - 3.0f * kTau : n2c * K::kHalfShrink - 2.0f * kTau;
        an = sqrt_up(n2c) * (SMALL ? K::kKappaIdx : K::kKappa);
      }
    }
    an = group_max<SMALL>(an);
    if (r < n_cpad) {
      if ((lane & (SMALL ? 0x0B : 0x1B)) == 0) s.gan[group_of<SMALL>(r)] = an;
      if constexpr (FOLD) {  // halves 4, 5 carry C, half 6 carries -a' (SD == 4)
        // C beyond the element type: the slot takes the unfolded form, which
        // adds C in fp32 and multiplies these halves by 0, so they must be
        // finite (an infinite half would make the row's product NaN, and the
        // minimum would drop the row)
        if (!split_down<BF16>(cv, k8[4], k8[5])) {
          nofold = 1;
          k8[4] = k8[5] = 0;
        }
        k8[6] = round_up<BF16>(an * kFoldScale) ^ 0x8000u;
      }
      const uint4 row = make_uint4(k8[0] | (static_cast<uint32_t>(k8[1]) << 16),
                                   k8[2] | (static_cast<uint32_t>(k8[3]) << 16),
                                   k8[4] | (static_cast<uint32_t>(k8[5]) << 16),
                                   k8[6] | (static_cast<uint32_t>(k8[7]) << 16));
      s.rows[r] = row;
      if constexpr (AROWS) {  // lane half 0: -c against hi and lo; half 1: C, -a'
        s.arows[2 * r] = make_uint4(row.x, row.y, row.x, row.y);
        s.arows[2 * r + 1] = make_uint4(row.z, row.w, 0u, 0u);
      }
      s.cval[r] = cv;
      if constexpr (ROWS32) {
#pragma unroll
        for (int q = 0; q < SD / 4; ++q)
          *reinterpret_cast<float4 *>(s.c32 + s.c32_offset(r) + 4 * q) =
              make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      }
    }
  }
  const int wflags = (__any(flag) ? 1 : 0) | (__any(nofold) ? 2 : 0);
  if (lane == 0) s.flags[wave] = wflags;
  __syncthreads();
  int all = 0;
#pragma unroll
  for (int w = 0; w < BLOCK / 64; ++w) all |= s.flags[w];
  all = __builtin_amdgcn_readfirstlane(all);  // uniform: the flags live in scalar registers
  const bool exact = (all & 1) != 0;
  fold_ok = FOLD && (all & 2) == 0;
  if (!exact) {
    // A row bit-identical to an earlier row can never win the strict-< scan.
    // Open addressing, at most half full; an entry is (tag << 12) | row with
    // the tag taken from hash bits the slot does not use (n_c <= 4096).  All
    // copies of one row value meet in one entry: the first to arrive claims
    // it, every later one lowers it to the smaller index with an atomic min,
    // and whichever of the two indices is larger is a duplicate.  So every
    // copy but the first is marked, and never the first.
    // No barrier follows: the marks may land while other waves already run
    // stage 1.  Either value of a marked word is valid there (a duplicate's
    // own C, or +inf, which drops a row that can never win), and every mark
    // is one 32-bit store; marks only make fewer sub-vectors ambiguous.  The
    // rows' x, y words (all the comparisons read at sub_dim 4) are never
    // written.
    const uint32_t mask = static_cast<uint32_t>(hash_slots - 1);
    for (int r = last_waves ? BLOCK - 1 - tid : tid; r < n_c; r += BLOCK) {
      const uint4 q = s.rows[r];
      const uint32_t hv = hash_row<SD>(q);
      const uint32_t key = ((hv >> 13) << 12) | static_cast<uint32_t>(r);
      uint32_t slot = hv & mask;
      for (int probe = 0; probe < hash_slots; ++probe) {
        const uint32_t old = atomicCAS(&s.hash[slot], kEmpty, key);
        if (old == kEmpty) break;
        if ((old >> 12) == (key >> 12) && same_row<SD>(s.rows[old & 0xFFFu], q)) {
          const uint32_t prev = atomicMin(&s.hash[slot], key);
          const int dup = max(static_cast<int>(prev & 0xFFFu), r);
          s.cval[dup] = __builtin_inff();
          // folded: C_hi = +inf, C_lo = 0 (an unfolded slot multiplies these
          // halves by 0 and takes C = +inf from cval alone)
          if (FOLD && fold_ok) {
            s.rows[dup].z = kInfBits<BF16>;
            if constexpr (AROWS) s.arows[2 * dup + 1].x = kInfBits<BF16>;
          }
          break;
        }
        slot = (slot + 1) & mask;
      }
    }
  }
  return exact;
}

// The 8 rows of group grp that lane half h evaluates in the exact stage:
// rows c0 .. c0 + 3 and c0 + 8 .. c0 + 11, c0 = 32 (grp / 2) + 16 h + 4 (grp
// mod 2), in ascending order.  best and bk are set to the minimum exact
// distance and the offset (0..3, 8..11) of its first row, the result of a
// strict-< scan from (+inf, 0) whenever that minimum is finite.  With MASK,
// rows >= n_c (the padding of the last block) are excluded; without it every
// row is < n_c, or a padding row of the fp32 copy (exact distance +inf).
template <int SD, bool BF16, bool ROWS32, bool MASK>
__device__ __forceinline__ void exact8(const Lds<SD, ROWS32> &s, const float (&xv)[SD], int grp,
                                       int h, int n_c, float &best, int &bk) {
  const int b = grp >> 1, hh = grp & 1;
  const int c0 = b * 32 + h * 16 + hh * 4;
  // c32_offset(c0), spelled out: the row set's padding is 4 (c0 / 4 + c0 / 16)
  const float *base = s.c32 + b * (32 * SD + 40) + h * (16 * SD + 20) + hh * (4 * SD + 4);
  float d[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k = (j & 3) + ((j & 4) << 1);
    const int c = c0 + k;
    float cv[SD];
    if constexpr (ROWS32) {
      // the second row set (k >= 8) is 2 sets further: 8 rows and 8 floats
      const float *row = base + SD * (k & 3) + ((k & 8) ? (8 * SD + 8) : 0);
#pragma unroll
      for (int q = 0; q < SD / 4; ++q) {
        const float4 w = *reinterpret_cast<const float4 *>(row + 4 * q);
        cv[4 * q] = w.x;
        cv[4 * q + 1] = w.y;
        cv[4 * q + 2] = w.z;
        cv[4 * q + 3] = w.w;
      }
    } else {
      centroid_in_set<SD, BF16, ROWS32>(s, c0 + (k & 8), k & 3, cv);
    }
    d[j] = sqdist<SD>(xv, cv);
    if (MASK) d[j] = (c < n_c) ? d[j] : __builtin_inff();
  }
  // the strict-< scan from (+inf, 0) keeps the first row of the minimum: take
  // the minimum, then the lowest row equal to it (rows after the first at an
  // infinite or NaN minimum differ from the scan; such a column takes the
  // full exact scan, which replaces this result)
  best = __builtin_fminf(__builtin_fminf(__builtin_fminf(d[0], d[1]), __builtin_fminf(d[2], d[3])),
                         __builtin_fminf(__builtin_fminf(d[4], d[5]), __builtin_fminf(d[6], d[7])));
  bk = 11;
#pragma unroll
  for (int j = 6; j >= 0; --j) bk = (d[j] == best) ? (j & 3) + ((j & 4) << 1) : bk;
}

// The 4 rows c0 .. c0 + 3 (c0 a multiple of 4) that one lane evaluates in the
// exact stage for an 8-row group; off = c32_offset(c0) (the caller knows
// c0 / 16).  best and bk are set as by exact8 (bk = offset 0..3).
template <int SD, bool BF16, bool ROWS32, bool MASK>
__device__ __forceinline__ void exact_rows4(const Lds<SD, ROWS32> &s, const float (&xv)[SD], int c0,
                                            int off, int n_c, float &best, int &bk) {
  float d[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float cv[SD];
    if constexpr (ROWS32) {
#pragma unroll
      for (int q = 0; q < SD / 4; ++q) {
        const float4 w = *reinterpret_cast<const float4 *>(s.c32 + off + SD * j + 4 * q);
        cv[4 * q] = w.x;
        cv[4 * q + 1] = w.y;
        cv[4 * q + 2] = w.z;
        cv[4 * q + 3] = w.w;
      }
    } else {
      centroid_in_set<SD, BF16, ROWS32>(s, c0, j, cv);
    }
    d[j] = sqdist<SD>(xv, cv);
    if (MASK) d[j] = (c0 + j < n_c) ? d[j] : __builtin_inff();
  }
  // (distances are >= 0, +inf or NaN; a NaN sends the column to the full
  // scan, and for the others med3 with -FLT_MAX is min without the NaN
  // quieting copy)
  best = __builtin_fminf(__builtin_fminf(__builtin_amdgcn_fmed3f(d[0], d[1], kNegMax), d[2]), d[3]);
  bk = 3;
#pragma unroll
  for (int j = 2; j >= 0; --j) bk = (d[j] == best) ? j : bk;
}

// Strict-< minimum of the exact distance over the 4 consecutive rows c0 ..
// c0 + 3 (c0 a multiple of 4, c0 + 3 < n_cpad: padding rows are staged too),
// visited in ascending order; the index recorded for row c0 + i is k0 + i.
// MASK as for exact8.
template <int SD, bool BF16, bool ROWS32, bool MASK>
__device__ __forceinline__ void exact4(const Lds<SD, ROWS32> &s, const float (&xv)[SD], int c0,
                                       int k0, int n_c, float &best, int &bk) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = c0 + i;
    float cv[SD];
    centroid_in_set<SD, BF16, ROWS32>(s, c0, i, cv);
    float d = sqdist<SD>(xv, cv);
    if (MASK) d = (c < n_c) ? d : __builtin_inff();
    const bool lt = d < best;
    best = lt ? d : best;
    bk = lt ? k0 + i : bk;
  }
}

// All rows of group grp (see group_of), in ascending order, into (best, bi)
// by strict <.
template <int SD, bool BF16, bool ROWS32, bool SMALL>
__device__ __forceinline__ void exact_group(const Lds<SD, ROWS32> &s, const float (&xv)[SD],
                                            int grp, int n_c, float &best, int &bi) {
  const int r0 = SMALL ? (grp >> 2) * 32 + ((grp >> 1) & 1) * 16 + 4 * (grp & 1)
                       : (grp >> 1) * 32 + 4 * (grp & 1);
#pragma unroll
  for (int j = 0; j < (SMALL ? 2 : 4); ++j)
    exact4<SD, BF16, ROWS32, !ROWS32>(s, xv, r0 + 8 * j, r0 + 8 * j, n_c, best, bi);
}

// Combine (distance, index) over the two lanes of a pair: smaller distance,
// then lower index.
__device__ __forceinline__ void pair_min(float &best, int &bi, int h) {
  const float ob = pair_other(best, h);
  const int oi = pair_other(bi, h);
  const bool take = ob < best || (ob == best && oi < bi);
  best = take ? ob : best;
  bi = take ? oi : bi;
}

// The full sub-vector of a column: lane 0 of the pair holds words 0, 1 and
// lane 1 words 2, 3 (sub_dim 8; at sub_dim 4 only lane 0's words are used).
template <int SD, bool BF16>
__device__ __forceinline__ void column_x(const uint2 &own, float (&xv)[SD]) {
  const PairVals p0 = pair_vals(own.x);
  const PairVals p1 = pair_vals(own.y);
  const uint32_t w[4] = {p0.first, p1.first, p0.second, p1.second};
  widen_words<SD, BF16>(w, 0, xv);
}

// Channel factors of sub-slot m (channels m*SD .. m*SD + SD - 1).
template <int SD, bool ROWS32>
__device__ __forceinline__ void factors(const Lds<SD, ROWS32> &s, int m, float (&f)[SD]) {
#pragma unroll
  for (int q = 0; q < SD / 4; ++q) {
    const float4 w = *reinterpret_cast<const float4 *>(s.scale + m * SD + 4 * q);
    f[4 * q] = w.x;
    f[4 * q + 1] = w.y;
    f[4 * q + 2] = w.z;
    f[4 * q + 3] = w.w;
  }
}

// Channel layout of smoothed keys: row r is sub-slot r mod n_sub of its key.
struct Smooth {
  int n_sub;
  float inv_n_sub;
  int mask;  // n_sub - 1 when n_sub is a power of two (every usual head_dim), else -1
};

// v mod n_sub for 0 <= v < 2^24 (a mask when n_sub is a power of two)
template <bool POW2>
__device__ __forceinline__ int sub_mod(int v, const Smooth &sm) {
  return POW2 ? (v & sm.mask) : mod_small(v, sm.n_sub, sm.inv_n_sub);
}

// Raw words of the T sub-vectors this lane loads for a unit: column t, row
// ubase + 32 t + lane mod 32 (zero past the group's end).
template <int SD, int T>
__device__ __forceinline__ void load_unit_x(const uint16_t *__restrict__ x, int64_t ubase,
                                            int64_t gend, uint32_t (&w)[T][4]) {
  const int lane = threadIdx.x & 63;
  // rows past the group end load the group's last row (their codes are
  // never stored); unconditional loads are not waited for one by one
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int64_t row = min(ubase + t * 32 + (lane & 31), gend - 1);
    if constexpr (SD == 4) {
      const uint2 q = *reinterpret_cast<const uint2 *>(x + row * 4);
      w[t][0] = q.x;
      w[t][1] = q.y;
      w[t][2] = w[t][3] = 0;
    } else {
      const uint4 q = *reinterpret_cast<const uint4 *>(x + row * 8);
      w[t][0] = q.x;
      w[t][1] = q.y;
      w[t][2] = q.z;
      w[t][3] = q.w;
    }
  }
}

// K-means: what a unit hands to the member sums (fp16 keys).  Lane h of a
// pair holds components h SD/2 .. h SD/2 + SD/2 - 1 of its column's row.
template <int SD, int T>
struct UnitSums {
  uint32_t code[T];
  uint32_t words[T][SD / 4];
  uint32_t check;  // bit t: column t took the full exact scan (may hold non-finite values)
};

// Adds a finished unit's rows to their centroids' member sums with fp64 LDS
// atomics (exact, see kAccMaxRows); lane 0 of a pair counts the member.
// Non-finite components count as 0.
template <int SD, int T>
__device__ __forceinline__ void add_unit_sums(const UnitSums<SD, T> &us, int64_t ubase,
                                              int64_t gend, double *lsum, uint32_t *lcnt) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int col = lane & 31;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (ubase + t * 32 + col < gend) {
      double *p = lsum + us.code[t] * SD + h * (SD / 2);
      const bool check = (us.check >> t) & 1u;
#pragma unroll
      for (int i = 0; i < SD / 2; ++i) {
        const uint32_t word = us.words[t][i >> 1];
        float v = widen<false>(static_cast<uint16_t>((i & 1) ? (word >> 16) : (word & 0xFFFFu)));
        if (check && !(__builtin_fabsf(v) <= kFltMax)) v = 0.0f;
        atomicAdd(p + i, static_cast<double>(v));
      }
      if (h == 0) atomicAdd(lcnt + us.code[t], 1u);
    }
  }
}

// One unit: the wave encodes T columns of 32 sub-vectors, rows ubase ..
// ubase + 32 T - 1 (raw words from load_unit_x).
template <int SD, int T, bool BF16, bool ROWS32, bool SCALED, bool ACC, bool POW2, bool SMALL>
__device__ void encode_unit(const uint32_t (&xin)[T][4], int64_t ubase, int64_t gend, int n_c,
                            int n_cpad, const Lds<SD, ROWS32> &s, bool exact_tile, bool fold,
                            const Smooth sm, int sub0, int code_bits, uint8_t *__restrict__ out,
                            UnitSums<SD, T> &us) {
  using K = Consts<SD, kTerms<SD, SCALED>>;
  using OpT = Op<SD, SCALED>;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;  // half of the block's rows / K slots this lane holds
  const int col = lane & 31;
  const int nblk = n_cpad / 32;
  // the last block has padding rows (uniform); with the fp32 copy their
  // exact distance is +inf and no mask is needed
  const bool padded = !ROWS32 && __builtin_amdgcn_readfirstlane(n_c & 31) != 0;

  OpT bop[T];    // this lane's K slots of its column
  uint2 xw[T];   // smoothed keys: the raw words stage 2 rebuilds x~ from
  float bn[T];   // upper bound of |x| (plus the split residual when smoothed)
  float nx2[T];  // plain keys: fp32 |x|^2 as the exact stage computes it
  float m1[T], m2[T];
  int g1[T];  // 16-row groups only; SMALL keeps the index in m1's low bits
  uint32_t codes[T];
  // smoothed keys: sub-slot of this lane's column 0 (sub0 = ubase mod n_sub)
  const int m0 = SCALED ? sub_mod<POW2>(sub0 + col, sm) : 0;
  uint32_t full_bits = 0;  // bit t: column t takes the full exact scan
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const uint32_t w[4] = {xin[t][0], xin[t][1], xin[t][2], xin[t][3]};
    if constexpr (SCALED) {
      // the pair splits the components: lane h smooths and splits components
      // h*E .. h*E + E - 1 (x~ = hi + lo + e exactly), then each lane trades
      // the half of the other operand for the half it lacks: h = 0 builds the
      // hi operand, h = 1 the lo operand
      constexpr int E = SD / 2;
      const int m = sub_mod<POW2>(m0 + 32 * t, sm);
      // this lane's E components: words 0 .. E/2-1 (h = 0) or E/2 .. E-1
      // (a mask select: a select between array elements becomes an indexed
      // load from private memory)
      const uint32_t upper = 0u - static_cast<uint32_t>(h);
      uint32_t ow[E / 2];
#pragma unroll
      for (int q = 0; q < E / 2; ++q) ow[q] = (w[q] & ~upper) | (w[E / 2 + q] & upper);
      float xo[E], f[E];
#pragma unroll
      for (int i = 0; i < E; ++i) {
        xo[i] = widen<BF16>(half_of(ow, i));
        f[i] = s.scale[m * SD + h * E + i];
      }
      uint32_t hw[E / 2], lw[E / 2];
      float nv2 = 0.0f, esum = 0.0f;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const float xt = xo[i] * f[i];
        const uint16_t hb = narrow<BF16>(xt);
        const float hf = widen<BF16>(hb);
        const float r = xt - hf;
        const uint16_t lb = narrow<BF16>(r);
        const float lf = widen<BF16>(lb);
        esum += __builtin_fabsf(r - lf);
        const float v = __builtin_fabsf(hf) + __builtin_fabsf(lf);
        nv2 = __builtin_fmaf(v, v, nv2);
        if (i & 1) {
          hw[i >> 1] |= static_cast<uint32_t>(hb) << 16;
          lw[i >> 1] |= static_cast<uint32_t>(lb) << 16;
        } else {
          hw[i >> 1] = hb;
          lw[i >> 1] = lb;
        }
      }
      uint32_t keep[E / 2], got[E / 2];
      if constexpr (SD == 8) {
#pragma unroll
        for (int q = 0; q < E / 2; ++q) {
          keep[q] = (h == 0) ? hw[q] : lw[q];
          got[q] = pair_other((h == 0) ? lw[q] : hw[q], h);
        }
      }
      nv2 = pair_sum(nv2);
      esum = pair_sum(esum);
      // a non-finite part (x~ beyond the element type, or not finite) makes
      // nv2 infinite or NaN, which sends the column to the full exact scan
      const bool ex = !(nv2 <= kNormCap) || exact_tile;
      full_bits |= (ex ? 1u : 0u) << t;
      bn[t] = ex ? 0.0f
                 : __builtin_fmaf(esum, SMALL ? K::kInvKappaIdxUp : K::kInvKappaUp, sqrt_up(nv2)) * kBnUp;
      // components 0 .. E-1 come from lane h = 0, E .. SD-1 from lane h = 1
      if constexpr (SD == 4) {
        // folded (K = 16): lane 0 of the pair holds [hi, lo], lane 1 the
        // slots of C and the error term
        const PairVals ph = pair_vals(hw[0]);
        const PairVals pl = pair_vals(lw[0]);
        bop[t] = (h == 0) ? make_uint4(ph.first, ph.second, pl.first, pl.second)
                          : make_uint4(fold ? kOnePair<BF16> : 0u,
                                       fold ? fold_b<BF16>(bn[t]) : 0u, 0u, 0u);
        xw[t] = make_uint2(w[0], w[1]);
      } else {
        bop[t] = (h == 0) ? make_uint4(keep[0], keep[1], got[0], got[1])
                          : make_uint4(got[0], got[1], keep[0], keep[1]);
        xw[t] = make_uint2((w[0] & ~upper) | (w[2] & upper), (w[1] & ~upper) | (w[3] & upper));
      }
    } else {
      float xv[SD];
      widen_words<SD, BF16>(w, 0, xv);
      float n2x = xv[0] * xv[0];
#pragma unroll
      for (int i = 1; i < SD; ++i) n2x = __builtin_fmaf(xv[i], xv[i], n2x);
      nx2[t] = n2x;
      const bool ex = !(n2x <= kNormCap) || exact_tile;
      full_bits |= (ex ? 1u : 0u) << t;
      bn[t] = ex ? 0.0f : sqrt_up(n2x);
      if constexpr (SD == 4) {
        // folded slots: the h = 1 half multiplies C_hi, C_lo by (1, 1)
        bop[t] = (h == 0) ? make_uint2(w[0], w[1])
                          : make_uint2(fold ? kOnePair<BF16> : 0u,
                                       fold ? fold_b<BF16>(bn[t]) : 0u);
      } else {
        bop[t] = (h == 0) ? make_uint2(w[0], w[1]) : make_uint2(w[2], w[3]);
      }
    }
    m1[t] = __builtin_inff();
    m2[t] = __builtin_inff();
    g1[t] = 0;
  }

  // A operand of block blk: -c for this lane's row; the plain form holds
  // the lane's half of the K slots, the smoothed form -c in both halves
  // (plain: from this lane's first entry, 64 entries per block)
  const uint2 *lane_rows = reinterpret_cast<const uint2 *>(s.rows) + 2 * col + h;
  auto a_operand = [&](int blk) -> OpT {
    if constexpr (SCALED && SD == 8) {
      return s.rows[blk * 32 + col];
    } else if constexpr (SCALED && ROWS32) {
      // K = 16, staged per lane half: -c twice (against hi and lo), or the
      // row's C_hi, C_lo, -a'
      return s.arows[(blk * 32 + col) * 2 + h];
    } else if constexpr (SCALED) {
      const uint2 q = reinterpret_cast<const uint2 *>(s.rows)[blk * 64 + 2 * col + h];
      return (h == 0) ? make_uint4(q.x, q.y, q.x, q.y) : make_uint4(q.x, q.y, 0u, 0u);
    } else {
      return lane_rows[blk * 64];
    }
  };
  auto c_operand = [&](int blk) {
    f32x16 cop;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 q = *reinterpret_cast<const float4 *>(&s.cval[blk * 32 + 8 * j + 4 * h]);
      cop[4 * j + 0] = q.x;
      cop[4 * j + 1] = q.y;
      cop[4 * j + 2] = q.z;
      cop[4 * j + 3] = q.w;
    }
    return cop;
  };

  // accumulator input of block blk: C from LDS, or zero when C is folded
  const f32x16 zero16 = {};
  // lower bounds of this lane's groups of block blk for column t
  // (recomputed): lo for group 2 blk + h, or with SMALL lo for 4 blk + h and
  // hi for 4 blk + 2 + h
  auto group_bounds = [&](int blk, int t, float &lo, float &hi) {
    const OpT aop = a_operand(blk);
    if constexpr (SMALL) {
      if (kFold<SD, SCALED> && fold) {
        const f32x16 a = mfma<BF16>(aop, bop[t], zero16);
        lo = min8<0>(a);
        hi = min8<8>(a);
      } else {
        const f32x16 a = mfma<BF16>(aop, bop[t], c_operand(blk));
        lo = __builtin_fmaf(-s.gan[4 * blk + h], bn[t], min8<0>(a));
        hi = __builtin_fmaf(-s.gan[4 * blk + 2 + h], bn[t], min8<8>(a));
      }
    } else {
      hi = __builtin_inff();
      if (kFold<SD, SCALED> && fold) {
        lo = min16(mfma<BF16>(aop, bop[t], zero16));
      } else {
        lo = __builtin_fmaf(-s.gan[2 * blk + h], bn[t],
                            min16(mfma<BF16>(aop, bop[t], c_operand(blk))));
      }
    }
  };

  // ---- stage 1: group lower bounds on the matrix cores ---------------------
  // With C folded into the product (no accumulator input) there are
  // registers for two accumulators: the matrix cores compute column t + 1
  // while the VALU reduces column t, and the next block's A operand and norm
  // bound are loaded one block ahead.  Otherwise one accumulator is reused.
  auto stage1 = [&](auto folded) {
    constexpr bool F = decltype(folded)::value;
    constexpr int kGpb = SMALL ? 4 : 2;  // groups per block
    OpT aop = a_operand(0);
    float an0 = F ? 0.0f : s.gan[h];
    float an1 = (F || !SMALL) ? 0.0f : s.gan[2 + h];
    for (int blk = 0; blk < nblk; ++blk) {
      const OpT a_cur = aop;
      const float an0_cur = an0, an1_cur = an1;
      const f32x16 cop = F ? zero16 : c_operand(blk);
      if constexpr (F) {
        aop = a_operand(min(blk + 1, nblk - 1));
      } else if (blk + 1 < nblk) {
        aop = a_operand(blk + 1);
        an0 = s.gan[kGpb * (blk + 1) + h];
        if constexpr (SMALL) an1 = s.gan[kGpb * (blk + 1) + 2 + h];
      }
      // 16-row groups: group 2 blk + h, its index kept in g1
      auto track = [&](int t, float mb) {
        m2[t] = __builtin_amdgcn_fmed3f(m1[t], m2[t], mb);
        g1[t] = (mb < m1[t]) ? 2 * blk + h : g1[t];
        m1[t] = __builtin_amdgcn_fmed3f(m1[t], mb, kNegMax);
      };
      // the bounds of this lane's groups from a product: lo (and hi, SMALL)
      auto reduce = [&](int t, const f32x16 &a, float &lo, float &hi) {
        if constexpr (SMALL) {
          lo = min8<0>(a);
          hi = min8<8>(a);
          if constexpr (!F) {
            lo = __builtin_fmaf(-an0_cur, bn[t], lo);
            hi = __builtin_fmaf(-an1_cur, bn[t], hi);
          }
        } else {
          lo = F ? min16(a) : __builtin_fmaf(-an0_cur, bn[t], min16(a));
        }
      };
      // (the index of the upper group is made a scalar of its own: folded into
      // the other's, it costs a second VALU instruction per key)
      const uint32_t k_lo = 2u * blk;
      const uint32_t k_hi = __builtin_amdgcn_readfirstlane(k_lo + 1u);
      auto track_all = [&](int t, float lo, float hi) {
        if constexpr (SMALL) {
          // 8-row groups: group 2 k + h with k = 2 blk + q, and k written
          // into the 4 low bits of the bound (see Consts), so keys of
          // different groups differ and min and med3 carry the index along
          // with the bound.  Both keys of the block at once: with m1 <= m2
          // and distinct keys a, b the new smallest is min3(m1, a, b) and the
          // new second smallest min(m2, med3(m1, a, b)): 3 instructions for 2
          // keys.  min3 and min are written out because keys with index bits
          // are not canonical floats to the compiler, which would quiet them
          // first (the keys are finite, so quieting changes nothing).
          const float ka = __uint_as_float((__float_as_uint(lo) & ~kIdxMask) | k_lo);
          const float kb = __uint_as_float((__float_as_uint(hi) & ~kIdxMask) | k_hi);
          const float mid = __builtin_amdgcn_fmed3f(m1[t], ka, kb);
          float n1, n2;
          asm("v_min3_f32 %0, %1, %2, %3" : "=v"(n1) : "v"(m1[t]), "v"(ka), "v"(kb));
          asm("v_min_f32 %0, %1, %2" : "=v"(n2) : "v"(m2[t]), "v"(mid));
          m1[t] = n1;
          m2[t] = n2;
        } else {
          track(t, lo);
        }
      };
      if constexpr (F) {
        // the error term is in the product: the group minimum is the bound
        f32x16 acc[2];
        acc[0] = mfma<BF16>(a_cur, bop[0], cop);
        if constexpr (T > 1) acc[1] = mfma<BF16>(a_cur, bop[1], cop);
        unroll<T>([&](auto tc) {
          constexpr int t = decltype(tc)::value;
          float lo, hi;
          reduce(t, acc[t & 1], lo, hi);
          if constexpr (t + 2 < T) acc[t & 1] = mfma<BF16>(a_cur, bop[t + 2], cop);
          track_all(t, lo, hi);
        });
      } else {
        unroll<T>([&](auto tc) {
          constexpr int t = decltype(tc)::value;
          float lo, hi;
          reduce(t, mfma<BF16>(a_cur, bop[t], cop), lo, hi);
          track_all(t, lo, hi);
        });
      }
    }
  };
  // The same block step as a function of the block index, for the forms
  // that run faster this way: with the blocks unrolled, sub_dim 8 with
  // 4-column units and 8-row groups (4-7% on the Llama shape, 3% on the full
  // cache) and smoothed sub_dim 4 keys with a power-of-two key length and
  // 8-row groups (1%); and the K-means forms (2.5%).  The other forms keep the loop above: the compiler schedules them
  // better in that shape (the Falcon shape runs 3% slower through this one).
  auto stage1_blocks = [&](auto folded) {
    constexpr bool F = decltype(folded)::value;
    constexpr int kGpb = SMALL ? 4 : 2;  // groups per block
    OpT aop = a_operand(0);
    float an0 = F ? 0.0f : s.gan[h];
    float an1 = (F || !SMALL) ? 0.0f : s.gan[2 + h];
    // 8-row groups (sub_dim 8 with 4-column units, or smoothed sub_dim 4 keys
    // with a power-of-two key length) with all
    // kSmallMaxCentroids / 32 blocks: the blocks are unrolled, so that the
    // operand reads take constant LDS offsets and the group indices are
    // constants
    constexpr bool kUnrolled = SMALL && ((SD == 8 && T == 4) || (SCALED && SD == 4 && POW2));
    auto block = [&](int blk) {
      const OpT a_cur = aop;
      const float an0_cur = an0, an1_cur = an1;
      const f32x16 cop = F ? zero16 : c_operand(blk);
      if constexpr (F) {
        aop = a_operand(min(blk + 1, nblk - 1));
      } else if (blk + 1 < nblk) {
        aop = a_operand(blk + 1);
        an0 = s.gan[kGpb * (blk + 1) + h];
        if constexpr (SMALL) an1 = s.gan[kGpb * (blk + 1) + 2 + h];
      }
      // 16-row groups: group 2 blk + h, its index kept in g1
      auto track = [&](int t, float mb) {
        m2[t] = __builtin_amdgcn_fmed3f(m1[t], m2[t], mb);
        g1[t] = (mb < m1[t]) ? 2 * blk + h : g1[t];
        m1[t] = __builtin_amdgcn_fmed3f(m1[t], mb, kNegMax);
      };
      // the bounds of this lane's groups from a product: lo (and hi, SMALL)
      auto reduce = [&](int t, const f32x16 &a, float &lo, float &hi) {
        if constexpr (SMALL) {
          lo = min8<0>(a);
          hi = min8<8>(a);
          if constexpr (!F) {
            lo = __builtin_fmaf(-an0_cur, bn[t], lo);
            hi = __builtin_fmaf(-an1_cur, bn[t], hi);
          }
        } else {
          lo = F ? min16(a) : __builtin_fmaf(-an0_cur, bn[t], min16(a));
        }
      };
      // (the index of the upper group is made a scalar of its own: folded into
      // the other's, it costs a second VALU instruction per key)
      const uint32_t k_lo = 2u * blk;
      const uint32_t k_hi = __builtin_amdgcn_readfirstlane(k_lo + 1u);
      auto track_all = [&](int t, float lo, float hi) {
        if constexpr (SMALL) {
          // 8-row groups: group 2 k + h with k = 2 blk + q, and k written
          // into the 4 low bits of the bound (see Consts), so keys of
          // different groups differ and min and med3 carry the index along
          // with the bound.  Both keys of the block at once: with m1 <= m2
          // and distinct keys a, b the new smallest is min3(m1, a, b) and the
          // new second smallest min(m2, med3(m1, a, b)): 3 instructions for 2
          // keys.  min3 and min are written out because keys with index bits
          // are not canonical floats to the compiler, which would quiet them
          // first (the keys are finite, so quieting changes nothing).
          const float ka = __uint_as_float((__float_as_uint(lo) & ~kIdxMask) | k_lo);
          const float kb = __uint_as_float((__float_as_uint(hi) & ~kIdxMask) | k_hi);
          const float mid = __builtin_amdgcn_fmed3f(m1[t], ka, kb);
          float n1, n2;
          asm("v_min3_f32 %0, %1, %2, %3" : "=v"(n1) : "v"(m1[t]), "v"(ka), "v"(kb));
          asm("v_min_f32 %0, %1, %2" : "=v"(n2) : "v"(m2[t]), "v"(mid));
          m1[t] = n1;
          m2[t] = n2;
        } else {
          track(t, lo);
        }
      };
      if constexpr (F) {
        // the error term is in the product: the group minimum is the bound
        f32x16 acc[2];
        acc[0] = mfma<BF16>(a_cur, bop[0], cop);
        if constexpr (T > 1) acc[1] = mfma<BF16>(a_cur, bop[1], cop);
        unroll<T>([&](auto tc) {
          constexpr int t = decltype(tc)::value;
          float lo, hi;
          reduce(t, acc[t & 1], lo, hi);
          if constexpr (t + 2 < T) acc[t & 1] = mfma<BF16>(a_cur, bop[t + 2], cop);
          track_all(t, lo, hi);
        });
      } else {
        unroll<T>([&](auto tc) {
          constexpr int t = decltype(tc)::value;
          float lo, hi;
          reduce(t, mfma<BF16>(a_cur, bop[t], cop), lo, hi);
          track_all(t, lo, hi);
        });
      }
      if constexpr (kUnrolled) {  // the next block's operands are read in this one
        hold(aop);
        if constexpr (!F) {
          hold(an0);
          hold(an1);
        }
      }
    };
    if (kUnrolled && nblk == kSmallMaxCentroids / 32) {  // uniform
      unroll<kSmallMaxCentroids / 32>([&](auto bc) { block(decltype(bc)::value); });
    } else {
      for (int blk = 0; blk < nblk; ++blk) block(blk);
    }
  };
  if (!exact_tile) {
    constexpr bool kBlockFn = (SMALL && SD == 8 && T == 4) || ACC || (SCALED && SMALL && SD == 4 && POW2);
    if (kFold<SD, SCALED> && fold) {
      if constexpr (kBlockFn) {
        stage1_blocks(std::true_type{});
      } else {
        stage1(std::true_type{});
      }
    } else {
      if constexpr (kBlockFn) {
        stage1_blocks(std::false_type{});
      } else {
        stage1(std::false_type{});
      }
    }
  }

  // the fp32 sub-vector of column t (smoothed keys: times the factors)
  auto column_value = [&](int t, float (&xv)[SD]) {
    if constexpr (SCALED) {
      if constexpr (SD == 4) {
        const uint32_t w[4] = {xw[t].x, xw[t].y, 0, 0};
        widen_words<SD, BF16>(w, 0, xv);
      } else {
        column_x<SD, BF16>(xw[t], xv);
      }
      float f[SD];
      factors<SD, ROWS32>(s, sub_mod<POW2>(m0 + 32 * t, sm), f);
#pragma unroll
      for (int i = 0; i < SD; ++i) xv[i] = xv[i] * f[i];
    } else {
      column_x<SD, BF16>(bop[t], xv);
    }
  };

  // ---- stage 2: exact resolution, one column at a time (lanes col and
  // col+32 share a column) ---------------------------------------------------
  unroll<T>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    float xv[SD];
    column_value(t, xv);
    // the pair's combined smallest group bound (lower group on equal bounds)
    // and second smallest bound: with a0 <= b0 and a1 <= b1 the second
    // smallest of {a0, b0, a1, b1} is med3(a0, a1, min(b0, b1))
    const PairVals pa = pair_vals(__float_as_uint(m1[t]));
    const PairVals pb = pair_vals(__float_as_uint(m2[t]));
    const float a0 = __uint_as_float(pa.first), a1 = __uint_as_float(pa.second);
    int cg1 = 0;
    [[maybe_unused]] int kk = 0, q1 = 0;  // 8-row groups: cg1 = 2 kk + q1
    if constexpr (SMALL) {
      // lane h's group is 2 k + h; equal keys hold equal k, and then lane
      // 0's group is the lower one
      const bool take1 = a1 < a0;
      const uint32_t key = take1 ? pa.second : pa.first;
      kk = static_cast<int>(key & kIdxMask);
      q1 = take1 ? 1 : 0;
    } else {
      const PairVals pg = pair_vals(static_cast<uint32_t>(g1[t]));
      const bool take1 =
          a1 < a0 || (a1 == a0 && static_cast<int>(pg.second) < static_cast<int>(pg.first));
      cg1 = static_cast<int>(take1 ? pg.second : pg.first);
    }
    const float cm2 = __builtin_amdgcn_fmed3f(
        a0, a1,
        __builtin_amdgcn_fmed3f(__uint_as_float(pb.first), __uint_as_float(pb.second), kNegMax));
    // the rows of group cg1 (see group_of) split over the pair so that every
    // row of lane 0 precedes every row of lane 1: 16-row groups, rows b*32 +
    // 8j + 4hh + i with j = 2h, 2h + 1; 8-row groups, rows 32 b + 16 q + 8 h
    // + 4 hh + i
    float best = __builtin_inff();
    int bk = 0;
    int bi;
    if constexpr (SMALL) {
      // c0 = 16 k + 8 h + 4 (cg1 mod 2) with k = cg1 / 2, so c0 / 16 = k and
      // its fp32 row set starts at (SD + 1) c0 + 4 k
      const int c0 = 16 * kk + 8 * h + 4 * q1;
      const int off = (16 * (SD + 1) + 4) * kk + (SD + 1) * (8 * h + 4 * q1);
      if (padded) {
        exact_rows4<SD, BF16, ROWS32, true>(s, xv, c0, off, n_c, best, bk);
      } else {
        exact_rows4<SD, BF16, ROWS32, false>(s, xv, c0, off, n_c, best, bk);
      }
      bi = c0 + bk;
    } else {
      if (padded) {
        exact8<SD, BF16, ROWS32, true>(s, xv, cg1, h, n_c, best, bk);
      } else {
        exact8<SD, BF16, ROWS32, false>(s, xv, cg1, h, n_c, best, bk);
      }
      bi = (cg1 >> 1) * 32 + 16 * h + 4 * (cg1 & 1) + bk;
    }
    {
      const PairVals pd = pair_vals(__float_as_uint(best));
      const PairVals pi = pair_vals(static_cast<uint32_t>(bi));
      const bool t1 = __uint_as_float(pd.second) < __uint_as_float(pd.first);
      best = __uint_as_float(t1 ? pd.second : pd.first);
      bi = static_cast<int>(t1 ? pi.second : pi.first);
    }
    float n2x;
    if constexpr (SCALED) {
      n2x = xv[0] * xv[0];
#pragma unroll
      for (int i = 1; i < SD; ++i) n2x = __builtin_fmaf(xv[i], xv[i], n2x);
    } else {
      n2x = nx2[t];
    }
    // s(c*) <= (best (1 + 2 gamma) - |x|^2) / 2 <= U
    const float U = __builtin_fmaf(best, K::kUA, __builtin_fmaf(n2x, -K::kUB, kTau));
    const bool full = ((full_bits >> t) & 1u) || !(best < __builtin_inff());
    // amb = !full && !(cm2 > U), as one compare: a column that is not full
    // has finite U and a cm2 that is not NaN, and a NaN fails <=
    const bool amb = (full ? __builtin_nanf("") : cm2) <= U;
    codes[t] = static_cast<uint32_t>(bi);

    // ambiguous: every group whose bound can reach U contains the oracle's
    // winner if any does; those groups are recomputed exactly.  The bounds
    // are recomputed on the matrix cores.  8-row groups: each lane marks its
    // qualifying groups in a mask and evaluates them in ascending order.
    // 16-row groups: each lane keeps the first two of its groups (its half
    // of every block) that qualify; lanes evaluate their own kept groups side
    // by side, and a lane with more than two takes a second pass over all of
    // its qualifying groups, which come after the kept two.
    if (__builtin_amdgcn_ballot_w64(amb) != 0) {
      float fb = __builtin_inff();
      int fi = 0x7fffffff;
      if constexpr (SMALL) {
        // at most 16 groups per lane: bit k of qmask marks group 2 k + h
        // (k = 2 blk + q, ascending rows); the blocks are unrolled so that
        // their products issue back to back, and the lane then visits its
        // qualifying groups in ascending order
        uint32_t qmask = 0;
        unroll<kSmallMaxCentroids / 32>([&](auto bc) {
          constexpr int blk = decltype(bc)::value;
          if (blk < nblk) {
            float lo, hi;
            group_bounds(blk, t, lo, hi);
            qmask |= (amb && lo <= U) ? (1u << (2 * blk)) : 0u;
            qmask |= (amb && hi <= U) ? (2u << (2 * blk)) : 0u;
          }
        });
        while (qmask != 0) {
          const int k = __builtin_ctz(qmask);
          qmask &= qmask - 1;
          exact_group<SD, BF16, ROWS32, SMALL>(s, xv, 2 * k + h, n_c, fb, fi);
        }
      } else {
        int q0 = -1, q1 = -1;
        bool over = false;
        // this lane's groups of block blk, 2 blk + h, in ascending row order
        auto keep = [&](float mb, int grp) {
          if (amb && mb <= U) {
            over = over || q1 >= 0;
            q1 = (q0 >= 0 && q1 < 0) ? grp : q1;
            q0 = (q0 < 0) ? grp : q0;
          }
        };
        // (nblk >= 1: bottom-tested loops, whose entry needs no test)
        int blk = 0;
        do {
          float lo, hi;
          group_bounds(blk, t, lo, hi);
          keep(lo, 2 * blk + h);
        } while (++blk < nblk);
        if (q0 >= 0) exact_group<SD, BF16, ROWS32, SMALL>(s, xv, q0, n_c, fb, fi);
        if (__any(q1 >= 0)) {
          if (q1 >= 0) exact_group<SD, BF16, ROWS32, SMALL>(s, xv, q1, n_c, fb, fi);
        }
        if (__any(over)) {
          blk = 0;
          do {
            float lo, hi;
            group_bounds(blk, t, lo, hi);
            if (over && lo <= U) exact_group<SD, BF16, ROWS32, SMALL>(s, xv, 2 * blk + h, n_c, fb, fi);
          } while (++blk < nblk);
        }
      }
      pair_min(fb, fi, h);
      codes[t] = amb ? static_cast<uint32_t>(fi) : codes[t];
    }
    // non-finite or huge values (or no distance below +inf): full exact
    // strict-< scan, split by parity; index 0 when nothing beats +inf
    if (__builtin_amdgcn_ballot_w64(full) != 0) {
      float fb = __builtin_inff();
      int fi = 0x7fffffff;
      // same trip count on both lanes of a pair; lane h takes rows r0 + h
      for (int r0 = 0; r0 < n_c; r0 += 2) {
        const int c = r0 + h;
        float cv[SD];
        centroid<SD, BF16, ROWS32>(s, min(c, n_c - 1), cv);
        float d = sqdist<SD>(xv, cv);
        d = (c < n_c) ? d : __builtin_inff();
        const bool lt = d < fb;
        fb = lt ? d : fb;
        fi = lt ? c : fi;
      }
      pair_min(fb, fi, h);
      codes[t] = full ? ((fi == 0x7fffffff) ? 0u : static_cast<uint32_t>(fi)) : codes[t];
    }
  });

  // ---- store: outside the column loop, one width branch ---------------------
  if constexpr (SCALED) {
#pragma unroll
    for (int t = 0; t < T; ++t)
      store_codes32(codes[t], ubase + t * 32, gend, code_bits, h == 0, out);
  } else if (h == 0) {
    const int64_t row0 = ubase + col;
    if (code_bits == 32) {
#pragma unroll
      for (int t = 0; t < T; ++t)
        if (row0 + 32 * t < gend) reinterpret_cast<uint32_t *>(out)[row0 + 32 * t] = codes[t];
    } else if (code_bits == 16) {
#pragma unroll
      for (int t = 0; t < T; ++t)
        if (row0 + 32 * t < gend)
          reinterpret_cast<uint16_t *>(out)[row0 + 32 * t] = static_cast<uint16_t>(codes[t]);
    } else {
#pragma unroll
      for (int t = 0; t < T; ++t)
        if (row0 + 32 * t < gend) out[row0 + 32 * t] = static_cast<uint8_t>(codes[t]);
    }
  }

  // ---- K-means: the codes and this lane's components for the member sums ---
  if constexpr (ACC) {
    static_assert(!SCALED && !BF16, "member sums are taken of plain fp16 keys");
    us.check = full_bits;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      us.code[t] = codes[t];
      if constexpr (SD == 4) {
        const uint32_t w1 = pair_vals(bop[t].y).first;  // lane 0 holds the whole row
        us.words[t][0] = h ? w1 : bop[t].x;
      } else {
        us.words[t][0] = bop[t].x;
        us.words[t][1] = bop[t].y;
      }
    }
  }
}

// One workgroup of BLOCK threads per CU.  Workgroup w owns units [w k,
// (w + 1) k) of the group-major unit sequence (a unit = 32 T consecutive
// sub-vectors of one group, encoded by one wave), split into segments of one
// group each.  Per segment the codebook slot is staged once, then the waves
// take units from a counter in LDS: a wave that runs ahead takes more units,
// so all waves of the CU finish close together (the issue arbiter favours
// the oldest waves, which would otherwise finish far ahead of the others).
template <int SD, int T, int BLOCK, bool BF16, bool ROWS32, bool SCALED, bool ACC, bool POW2,
          bool SMALL>
__global__ void __launch_bounds__(BLOCK, 1)
encode_mfma_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ codebook,
                   int64_t n, int n_c, int64_t cb_stride, int64_t n_codebooks, int64_t group_len,
                   int64_t units_per_group, int64_t total_units, int64_t units_per_wg,
                   const int32_t *__restrict__ group_map, uint8_t *__restrict__ out,
                   int hash_slots, const float *__restrict__ scale, int64_t scale_stride,
                   int head_dim, int code_bits, unsigned long long *__restrict__ acc_sums,
                   unsigned int *__restrict__ acc_counts) {
  constexpr int kWaves = BLOCK / 64;
  constexpr int kUnit = T * 32;
  extern __shared__ uint4 lds_raw[];
  const int n_cpad = (n_c + 31) & ~31;
  constexpr bool kARows = SCALED && SD == 4 && ROWS32;
  const Lds<SD, ROWS32> s(lds_raw, n_cpad, hash_slots, kARows ? 2 * n_cpad : 0);
  const int scale_len = SCALED ? head_dim : 0;
  Smooth sm{1, 1.0f, 0};
  if constexpr (SCALED) {
    sm.n_sub = head_dim / SD;
    sm.inv_n_sub = 1.0f / static_cast<float>(sm.n_sub);
    sm.mask = (sm.n_sub & (sm.n_sub - 1)) == 0 ? sm.n_sub - 1 : -1;
  }
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  int *counter = s.flags + s.kCounter;
  // K-means member sums of the current segment: [n_c][SD] fp64, then the
  // counts, after the staging areas (a plain encode stages no factors)
  double *lsum = nullptr;
  uint32_t *lcnt = nullptr;
  UnitSums<SD, T> us;
  if constexpr (ACC) {
    lsum = reinterpret_cast<double *>(s.scale);
    lcnt = reinterpret_cast<uint32_t *>(lsum + n_c * SD);
    for (int e = threadIdx.x; e < n_c * SD; e += BLOCK) lsum[e] = 0.0;
    for (int e = threadIdx.x; e < n_c; e += BLOCK) lcnt[e] = 0u;
  }

  const int64_t u_first = static_cast<int64_t>(blockIdx.x) * units_per_wg;
  const int64_t u_last = min(u_first + units_per_wg, total_units);
  bool first_seg = true;
  // the grid gives every workgroup at least one unit, so the first segment
  // is entered unconditionally
  int64_t seg = u_first;
  do {  // uniform
    const int64_t g = ((seg | units_per_group) >> 32) == 0
                          ? static_cast<int64_t>(static_cast<uint32_t>(seg) /
                                                 static_cast<uint32_t>(units_per_group))
                          : seg / units_per_group;
    const int64_t g_unit0 = g * units_per_group;
    const int64_t seg_end = min(u_last, g_unit0 + units_per_group);
    const int64_t gstart = g * group_len;
    const int64_t gend = min(gstart + group_len, n);
    const int seg_sub0 = SCALED ? static_cast<int>(gstart % sm.n_sub) : 0;
    const int64_t slot = group_map ? static_cast<int64_t>(group_map[g]) : g;
    const bool bad = slot < 0 || slot >= n_codebooks;
    // Plain keys in 4-column units with 16-row groups (codebooks of more
    // than 256 centroids, whose units are long: kMixed) take work in pieces
    // of half a unit: the youngest wave of each SIMD, which the issue
    // arbiter serves last, takes 2-column pieces and the others whole units
    // (two pieces), so the work a starved wave still holds when the others
    // run out is half as long.  A whole unit that starts on the segment's
    // last piece stores only the rows up to the segment's end (send).  (With
    // 8-row groups the 2-column form costs more than the shorter tail saves.)
    constexpr bool kMixed = !ACC && !SCALED && !SMALL && T == 4;
    if constexpr (kMixed) {
      constexpr int kSmallW = kWaves / 4;      // the youngest wave of each SIMD
      constexpr int kBigW = kWaves - kSmallW;
      constexpr int kPiece = kUnit / 2;        // half a unit: 2 columns
      const bool small = wave >= kBigW;        // uniform per wave
      const int take = small ? 1 : 2;          // pieces per take
      const int64_t p0 = 2 * seg, pend = 2 * seg_end, pg0 = 2 * g_unit0;
      const int64_t send = min(gend, gstart + (pend - pg0) * kPiece);
      // the first piece of every wave is fixed; its loads overlap the staging
      int64_t p = p0 + (small ? 2 * kBigW + (wave - kBigW) : 2 * wave);
      uint32_t xw[T][4];
      auto load_x = [&](int64_t piece) {
        const int64_t b = gstart + (piece - pg0) * kPiece;
        if (small) {
          load_unit_x<SD, 2>(x, b, send, reinterpret_cast<uint32_t(&)[2][4]>(xw));
        } else {
          load_unit_x<SD, T>(x, b, send, xw);
        }
      };
      if (!bad && p < pend) load_x(p);
      if (!first_seg) __syncthreads();  // every wave is done with the previous segment
      first_seg = false;
      if (threadIdx.x == 0) *counter = 2 * kBigW + kSmallW;
      bool exact_tile = false, fold = false;
      if (!bad) {
        // its barrier also publishes the counter
        exact_tile = stage_codebook<SD, kTerms<SD, SCALED>, BF16, ROWS32, BLOCK, kFold<SD, SCALED>,
                                    kARows, SMALL>(codebook + slot * cb_stride, n_c, n_cpad, s,
                                                   hash_slots, nullptr, 0, units_per_wg < kWaves,
                                                   fold);
      } else {
        __syncthreads();
      }
      while (p < pend) {  // uniform per wave
        const int64_t ubase = gstart + (p - pg0) * kPiece;
        if (bad) {  // a bad slot: all-one codes
          const int64_t bpc = code_bits / 8;
          const int64_t bend = min(ubase + kPiece * take, send) * bpc;
          for (int64_t b = ubase * bpc + lane; b < bend; b += 64) out[b] = 0xFFu;
        } else if (small) {
          UnitSums<SD, 2> none;
          encode_unit<SD, 2, BF16, ROWS32, false, false, false, SMALL>(
              reinterpret_cast<const uint32_t(&)[2][4]>(xw), ubase, send, n_c, n_cpad, s,
              exact_tile, fold, sm, 0, code_bits, out, none);
        } else {
          encode_unit<SD, T, BF16, ROWS32, false, false, false, SMALL>(
              xw, ubase, send, n_c, n_cpad, s, exact_tile, fold, sm, 0, code_bits, out, us);
        }
        int next = 0;
        if (lane == 0) next = atomicAdd(counter, take);
        p = p0 + __builtin_amdgcn_readfirstlane(next);
        if (!bad && p < pend) load_x(p);
      }
    } else {
      // the first unit of every wave is fixed; its loads overlap the staging
      int64_t u = seg + wave;
      uint32_t xw[T][4];
      if (!bad && u < seg_end) load_unit_x<SD, T>(x, gstart + (u - g_unit0) * kUnit, gend, xw);
      if (!first_seg) __syncthreads();  // every wave is done with the previous segment
      first_seg = false;
      if (threadIdx.x == 0) *counter = kWaves;
      bool exact_tile = false, fold = false;
      if (!bad) {
        // its barrier also publishes the counter
        exact_tile = stage_codebook<SD, kTerms<SD, SCALED>, BF16, ROWS32, BLOCK, kFold<SD, SCALED>,
                                    kARows, SMALL>(
            codebook + slot * cb_stride, n_c, n_cpad, s, hash_slots,
            (SCALED && scale) ? scale + slot * scale_stride : nullptr, scale_len,
            units_per_wg < kWaves, fold);
      } else {
        __syncthreads();
      }
      while (u < seg_end) {  // uniform per wave
        const int64_t ubase = gstart + (u - g_unit0) * kUnit;
        if (bad) {
          // a bad slot: all-one codes
          if constexpr (SCALED) {
#pragma unroll
            for (int t = 0; t < T; ++t)
              store_codes32(0xFFFFFFFFu, ubase + t * 32, gend, code_bits, h == 0, out);
          } else {
            const int64_t bpc = code_bits / 8;
            const int64_t bend = min(ubase + kUnit, gend) * bpc;
            for (int64_t b = ubase * bpc + lane; b < bend; b += 64) out[b] = 0xFFu;
          }
        } else {
          if constexpr (SCALED) {
            // sub-slot of the unit's first row: (group start + unit offset) mod
            // n_sub; the offset can pass 2^32 rows in one group
            const int64_t rel = (u - g_unit0) * kUnit;
            int sub0;
            if constexpr (POW2) {  // the host launches this form only for a power of two
              sub0 = (seg_sub0 + static_cast<int>(rel & sm.mask)) & sm.mask;
            } else {
              const uint32_t off = (rel >> 32) == 0
                                       ? static_cast<uint32_t>(rel) % static_cast<uint32_t>(sm.n_sub)
                                       : static_cast<uint32_t>(rel % sm.n_sub);
              sub0 = mod_small(seg_sub0 + static_cast<int>(off), sm.n_sub, sm.inv_n_sub);
            }
            encode_unit<SD, T, BF16, ROWS32, SCALED, ACC, POW2, SMALL>(
                xw, ubase, gend, n_c, n_cpad, s, exact_tile, fold, sm, sub0, code_bits, out, us);
          } else {
            encode_unit<SD, T, BF16, ROWS32, SCALED, ACC, false, SMALL>(
                xw, ubase, gend, n_c, n_cpad, s, exact_tile, fold, sm, 0, code_bits, out, us);
          }
        }
        // the next unit is taken (a returning LDS atomic, which would wait
        // behind the member-sum atomics) and its loads issued before this
        // unit's rows join the sums
        int next = 0;
        if (lane == 0) next = atomicAdd(counter, 1);
        u = seg + __builtin_amdgcn_readfirstlane(next);
        if (!bad && u < seg_end) load_unit_x<SD, T>(x, gstart + (u - g_unit0) * kUnit, gend, xw);
        if constexpr (ACC) {
          if (!bad) add_unit_sums<SD, T>(us, ubase, gend, lsum, lcnt);
        }
      }
    }
    if constexpr (ACC) {
      // flush the segment's sums into the workspace copy of this workgroup
      // (int64 units of 2^-24: the fp64 sums are exact multiples of 2^-24)
      // and clear them; the next segment adds only after its staging barrier
      __syncthreads();  // every wave has added its rows
      if (!bad) {
        const int64_t cell0 = (static_cast<int64_t>(blockIdx.x % kKmReplicas) * n_codebooks + slot) * n_c;
        for (int e = threadIdx.x; e < n_c * SD; e += BLOCK) {
          const double v = lsum[e];
          if (v != 0.0)
            atomicAdd(acc_sums + cell0 * SD + e,
                      static_cast<unsigned long long>(static_cast<int64_t>(v * 16777216.0)));
          lsum[e] = 0.0;
        }
        for (int e = threadIdx.x; e < n_c; e += BLOCK) {
          const uint32_t k = lcnt[e];
          if (k) atomicAdd(acc_counts + cell0 + e, k);
          lcnt[e] = 0u;
        }
      }
    }
    seg = seg_end;
  } while (seg < u_last);
}

template <int SD, int T, int BLOCK, bool BF16, bool ROWS32, bool SCALED, bool ACC, bool POW2,
          bool SMALL>
hipError_t launch_t(const void *x, const void *codebook, const int32_t *group_map, void *out,
                    const Layout &l, const Codes &codes, hipStream_t stream, int64_t cus,
                    const KmSums &acc = KmSums{nullptr, nullptr}) {
  constexpr int kUnit = T * 32;
  const int64_t span = l.group_len < l.n ? l.group_len : l.n;
  const int64_t units_per_group = (span + kUnit - 1) / kUnit;
  const int64_t total_units = units_per_group * l.n_groups;
  const int n_cpad = (l.n_centroids + 31) & ~31;
  int hash_slots = 64;
  while (hash_slots < 2 * l.n_centroids) hash_slots <<= 1;
  const int arows_len = (SCALED && SD == 4 && ROWS32) ? 2 * n_cpad : 0;
  const size_t lds =
      Lds<SD, ROWS32>::bytes(n_cpad, hash_slots, SCALED ? codes.head_dim : 0, arows_len) +
      (ACC ? static_cast<size_t>(l.n_centroids) * (SD * 8 + 4) : 0);
  static_assert(!SMALL || ROWS32, "small codebooks keep the fp32 rows");
  if (SMALL && l.n_centroids > kSmallMaxCentroids) return hipErrorInvalidValue;
  auto kern = encode_mfma_kernel<SD, T, BLOCK, BF16, ROWS32, SCALED, ACC, POW2, SMALL>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  // one workgroup per CU (small inputs: fewer units than waves per workgroup,
  // spread over more CUs)
  // (member sums: at most kAccMaxRows rows per workgroup)
  int64_t units_per_wg = (total_units + cus - 1) / cus;
  if (ACC && units_per_wg > kAccMaxRows / kUnit) units_per_wg = kAccMaxRows / kUnit;
  const int64_t grid = (total_units + units_per_wg - 1) / units_per_wg;
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(grid)), dim3(BLOCK), lds, stream,
                     static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(codebook),
                     l.n, l.n_centroids, l.codebook_stride, l.n_codebooks, l.group_len,
                     units_per_group, total_units, units_per_wg, group_map,
                     static_cast<uint8_t *>(out), hash_slots, codes.scale, codes.scale_stride,
                     codes.head_dim, codes.code_bits, acc.sums, acc.counts);
  return hipGetLastError();
}

// CUs of the current device (cached per device; safe to call from several
// host threads).
int cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  if (dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Columns per wave: the smoothed sub_dim 8 form holds twice the operand
// registers per column.
template <int SD, bool SCALED, bool ROWS32>
constexpr int columns() { return SCALED ? 2 : 4; }

template <int SD, bool BF16, bool SCALED, bool POW2>
hipError_t launch_sd_p(const void *x, const void *codebook, const int32_t *group_map, void *out,
                       const Layout &l, const Codes &codes, hipStream_t stream) {
  const int64_t cus = cu_count();
  if (l.n_centroids > kRows32MaxCentroids)
    return launch_t<SD, columns<SD, SCALED, false>(), 1024, BF16, false, SCALED, false, POW2, false>(
        x, codebook, group_map, out, l, codes, stream, cus);
  if (l.n_centroids > kSmallMaxCentroids)
    return launch_t<SD, columns<SD, SCALED, true>(), 1024, BF16, true, SCALED, false, POW2, false>(
        x, codebook, group_map, out, l, codes, stream, cus);
  if constexpr (!SCALED) {
    // fewer 4-column units than CUs: one column per unit, so that the work
    // spreads over 4 times as many waves (a unit runs on one wave, alone on
    // its CU, and its latency is the launch's)
    const int64_t span = l.group_len < l.n ? l.group_len : l.n;
    if ((span + 127) / 128 * l.n_groups < cus)
      return launch_t<SD, 1, 1024, BF16, true, false, false, false, true>(
          x, codebook, group_map, out, l, codes, stream, cus);
  }
  return launch_t<SD, columns<SD, SCALED, true>(), 1024, BF16, true, SCALED, false, POW2, true>(
      x, codebook, group_map, out, l, codes, stream, cus);
}

// Smoothed keys: the channel index is a mask when head_dim / sub_dim is a
// power of two (a form of its own, so that neither form holds the other's
// registers).
template <int SD, bool BF16, bool SCALED>
hipError_t launch_sd(const void *x, const void *codebook, const int32_t *group_map, void *out,
                     const Layout &l, const Codes &codes, hipStream_t stream) {
  if constexpr (SCALED) {
    const int n_sub = codes.head_dim / SD;
    if ((n_sub & (n_sub - 1)) == 0)
      return launch_sd_p<SD, BF16, true, true>(x, codebook, group_map, out, l, codes, stream);
  }
  return launch_sd_p<SD, BF16, SCALED, false>(x, codebook, group_map, out, l, codes, stream);
}

// The plain kernel handles unsmoothed keys with 8, 16 or 32-bit codes (one
// store per sub-vector); factors, or other code widths, take the fused
// kernel, which stages unit factors when none are given.
template <int SD, bool BF16>
hipError_t launch_scaled(const void *x, const void *codebook, const int32_t *group_map, void *out,
                         const Layout &l, const Codes &codes, hipStream_t stream) {
  const int b = codes.code_bits;
  const bool fused = codes.scale != nullptr || (b != 8 && b != 16 && b != 32);
  return fused ? launch_sd<SD, BF16, true>(x, codebook, group_map, out, l, codes, stream)
               : launch_sd<SD, BF16, false>(x, codebook, group_map, out, l, codes, stream);
}

}  // namespace

bool encode_mfma_supported(const Layout &l) { return l.n_centroids <= kMfmaMaxCentroids; }

bool encode_mfma_kmeans_supported(const Layout &l) {
  return !l.bf16 && l.n_centroids <= kKmFusedMaxCentroids &&
         (l.sub_dim == 4 || l.sub_dim == 8);
}

hipError_t launch_encode_mfma_kmeans(const void *x, const void *codebook,
                                     const int32_t *group_map, uint32_t *out, const Layout &l,
                                     const KmSums &acc, hipStream_t stream) {
  static_assert(kKmFusedMaxCentroids <= kRows32MaxCentroids, "the sums follow the fp32 rows");
  const int64_t cus = cu_count();
  const Codes codes = plain_codes(l);
  const bool small = l.n_centroids <= kSmallMaxCentroids;
  if (l.sub_dim == 4)
    return small ? launch_t<4, columns<4, false, true>(), 1024, false, true, false, true, false, true>(
                       x, codebook, group_map, out, l, codes, stream, cus, acc)
                 : launch_t<4, columns<4, false, true>(), 1024, false, true, false, true, false, false>(
                       x, codebook, group_map, out, l, codes, stream, cus, acc);
  return small ? launch_t<8, columns<8, false, true>(), 1024, false, true, false, true, false, true>(
                     x, codebook, group_map, out, l, codes, stream, cus, acc)
               : launch_t<8, columns<8, false, true>(), 1024, false, true, false, true, false, false>(
                     x, codebook, group_map, out, l, codes, stream, cus, acc);
}

int64_t encode_mfma_grid(const Layout &l) {
  // upper bound on the workgroups of any plan above (one 32-row unit each)
  const int64_t span = l.group_len < l.n ? l.group_len : l.n;
  return (span + 31) / 32 * l.n_groups;
}

hipError_t launch_encode_mfma(const void *x, const void *codebook, const int32_t *group_map,
                              void *out, const Layout &l, const Codes &codes,
                              hipStream_t stream) {
  if (l.sub_dim == 4) {
    return l.bf16 ? launch_scaled<4, true>(x, codebook, group_map, out, l, codes, stream)
                  : launch_scaled<4, false>(x, codebook, group_map, out, l, codes, stream);
  }
  return l.bf16 ? launch_scaled<8, true>(x, codebook, group_map, out, l, codes, stream)
                : launch_scaled<8, false>(x, codebook, group_map, out, l, codes, stream);
}

}  // namespace vqk
