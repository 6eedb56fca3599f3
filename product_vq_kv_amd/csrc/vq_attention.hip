// vq_attention.hip -- decode attention straight from VQ codes (gfx950).
//
// The operation (VeloxQuant-MLX blog, "I Wrote a Metal Kernel to Stop My Mac
// From OOMing", section "What's Next: Phase 2"; blog index, "The Kernel's
// Hot Path"): attention of one new query per sequence over a key/value cache
// stored as 8-bit product-VQ codes, computed from the codes without ever
// materializing the fp16 keys:
//   LUT[s][c] = q~_s . C_k[c]                  per query head, q~ = q / f
//   score_t   = sum_s LUT[s][k_code[t][s]]     (= q . k_t in exact arithmetic)
//   out       = sum_t softmax(scale * score)_t * v_t,  v_t from C_v[v_code[t][.]]
// with grouped-query heads (query head hq reads key/value head hq / g), a
// per-sequence length and an optional sliding window.
//
// Design (MI355X): the sequence is split into chunks of kChunk tokens so a
// batch of decode queries fills the chip; each workgroup handles one
// (sequence, kv head, chunk) for all g query heads of that kv head and writes
// an unnormalized partial (m, l, o) per head to the caller's workspace; a
// second launch merges the chunks (flash-decoding split).  Within a chunk:
//   * the codebooks are widened to fp32 in LDS once;
//   * per query head the LUT is built in LDS, 16 sub-spaces x 256 codes at a
//     time (16 KB, so several workgroups share a CU), and each lane gathers
//     the scores of its tokens from it (one LDS read per sub-space, the key
//     codes held in registers); softmax runs in base 2 with scale * log2(e)
//     folded into q~;
//   * the value sum maps lanes to (value sub-space, token group): a lane reads
//     one value-codebook row per token and feeds all g heads with it.
// For head_dim 64, 128 and 256 the scores and the value sum run on the
// matrix cores instead (attn_mfma_partial).  Large batches take a streaming
// form (attn_stream_partial): balanced ranges of 64-token slices per
// workgroup, a running softmax per wave and one partial per segment part.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "vq.h"
#include "vq_launch.h"

namespace vqk {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 512;     // tokens per workgroup
constexpr int kMaxGroup = 8;    // query heads per kv head
constexpr int kRows = 256;      // every 8-bit code has a table row (zero past n_c)
constexpr int kTokPerLane = kChunk / kThreads;  // score phase: tokens per lane
constexpr int kMaxKeyWords = 16;                // 4-code words per key row (<= 64 codes)
constexpr int kVPrefetch = 16;                  // value phase: code loads in flight per lane
constexpr int kLutBlock = 16;                   // sub-spaces per LUT block in LDS
constexpr int kVGroup = 4;                      // query heads per value pass
constexpr float kNegInf = -__builtin_inff();

template <bool BF16>
__device__ __forceinline__ float widen(uint16_t v) {
  if constexpr (BF16) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
  } else {
    return static_cast<float>(__builtin_bit_cast(_Float16, v));
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Workgroup-wide max / sum through `red` (kThreads / 64 floats).
__device__ __forceinline__ float block_max(float v, float *red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r += red[i];
  __syncthreads();
  return r;
}

struct AttnArgs {
  const uint16_t *q;        // [B][Hq][D]
  const uint8_t *k_codes;   // [B][Hkv][S][n_sub_k]
  const uint8_t *v_codes;   // [B][Hkv][S][n_sub_v]
  const uint16_t *k_cb;     // [Hkv][n_c][SDK]
  const uint16_t *v_cb;     // [Hkv][n_c][SDV]
  const float *k_scale;     // [Hkv][D] or null
  const int32_t *kv_len;    // [B] or null
  float *ws;                // [B][Hq][n_chunks][D + 2]
  float *out;               // [B][Hq][D]
  int B, Hq, Hkv, D, S, n_c, window, n_chunks;
  int n_wg;                 // workgroups of the streaming partial launch
  float qmul;               // softmax_scale * log2(e)
};

// LDS: ck [256][SDK], cv [256][SDV], lut [kLutBlock][256], qt [D],
// p [g][kChunk], red (reduction / partial sums) [max(64, NG * D)].  The
// tables have a row for every byte value; rows past n_c are zero, so a code
// >= n_c decodes to a zero row (as vq_decode does for a bad index).  The LUT
// holds kLutBlock sub-spaces at a time (16 KB), so several workgroups share
// a CU.
template <int SDK, int SDV>
size_t attn_lds_bytes(int D, int g) {
  const int n_sub_v = D / SDV;
  const int ng = kThreads / n_sub_v;
  return sizeof(float) * (static_cast<size_t>(kRows) * (SDK + SDV) +
                          static_cast<size_t>(kLutBlock) * kRows + D +
                          static_cast<size_t>(g) * kChunk + std::max(64, ng * D));
}

template <int SDK, int SDV, bool BF16>
__global__ void __launch_bounds__(kThreads)
attn_partial(const AttnArgs a) {
  extern __shared__ float4 lds4[];
  float *lds = reinterpret_cast<float *>(lds4);
  const int n_c = a.n_c, D = a.D;
  const int n_sub_k = D / SDK, n_sub_v = D / SDV;
  const int g = a.Hq / a.Hkv;
  float *ck = lds;
  float *cv = ck + kRows * SDK;
  float *lut = cv + kRows * SDV;
  float *qt = lut + kLutBlock * kRows;
  float *p = qt + D;
  float *red = p + g * kChunk;

  // chunks rotate with (sequence, head): workgroup i runs on XCD i mod 8, so
  // a fixed chunk-to-x map would give the XCDs that hold late (often empty)
  // chunks of every sequence far less work than the others
  const int chunk = (blockIdx.x + blockIdx.y + gridDim.y * blockIdx.z) % gridDim.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  int L = a.kv_len ? a.kv_len[b] : a.S;
  L = min(max(L, 0), a.S);
  const int first = a.window > 0 ? max(0, L - a.window) : 0;
  const int t0 = chunk * kChunk;
  const int lo = max(first, t0), hi = min(L, t0 + kChunk);
  const int64_t part_stride = D + 2;
  float *part = a.ws + ((static_cast<int64_t>(b) * a.Hq + h * g) * a.n_chunks + chunk) * part_stride;
  if (lo >= hi) {  // nothing attended here (uniform)
    for (int j = 0; j < g; ++j) {
      float *pj = part + static_cast<int64_t>(j) * a.n_chunks * part_stride;
      for (int d = tid; d < D; d += kThreads) pj[d] = 0.0f;
      if (tid == 0) {
        pj[D] = kNegInf;
        pj[D + 1] = 0.0f;
      }
    }
    return;
  }

  // codebooks of kv head h, widened once.  (Loads are unconditional from
  // clamped in-bounds addresses: a load under a branch is waited for before
  // the next one is issued.)
  const uint16_t *kcb = a.k_cb + static_cast<int64_t>(h) * n_c * SDK;
  const uint16_t *vcb = a.v_cb + static_cast<int64_t>(h) * n_c * SDV;
  for (int e = tid; e < kRows * SDK; e += kThreads) {
    const float v = widen<BF16>(kcb[min(e, n_c * SDK - 1)]);
    ck[e] = (e < n_c * SDK) ? v : 0.0f;
  }
  for (int e = tid; e < kRows * SDV; e += kThreads) {
    const float v = widen<BF16>(vcb[min(e, n_c * SDV - 1)]);
    cv[e] = (e < n_c * SDV) ? v : 0.0f;
  }

  const int64_t row0 = (static_cast<int64_t>(b) * a.Hkv + h) * a.S;
  const uint8_t *kc = a.k_codes + row0 * n_sub_k;
  const uint8_t *vc = a.v_codes + row0 * n_sub_v;

  // this lane's key-code rows (tokens t0 + tid + kThreads*i), loaded once
  // with every load in flight and reused by all g query heads
  const int kwords = n_sub_k / 4;
  uint32_t kw[kTokPerLane][kMaxKeyWords];
#pragma unroll
  for (int i = 0; i < kTokPerLane; ++i) {
    const int t = min(max(t0 + tid + kThreads * i, lo), hi - 1);
    const uint32_t *crow = reinterpret_cast<const uint32_t *>(kc + static_cast<int64_t>(t) * n_sub_k);
#pragma unroll
    for (int w = 0; w < kMaxKeyWords; ++w) kw[i][w] = crow[min(w, kwords - 1)];
  }

  for (int j = 0; j < g; ++j) {
    const int hq = h * g + j;
    const uint16_t *qrow = a.q + (static_cast<int64_t>(b) * a.Hq + hq) * D;
    __syncthreads();  // the previous head is done with qt and the LUT
    for (int d = tid; d < D; d += kThreads) {
      float v = widen<BF16>(qrow[d]);
      if (a.k_scale) v = v / a.k_scale[static_cast<int64_t>(h) * D + d];
      qt[d] = v * a.qmul;
    }
    // scores (base-2 units): LUT gathers, sub-spaces in ascending order, the
    // LUT built kLutBlock sub-spaces at a time
    float acc[kTokPerLane];
#pragma unroll
    for (int i = 0; i < kTokPerLane; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int sb = 0; sb < kMaxKeyWords * 4 / kLutBlock; ++sb) {
      if (sb * kLutBlock < n_sub_k) {  // uniform
        __syncthreads();  // qt is written; the previous block's LUT is no longer read
        // LUT[s][c] = sum_i qt[s*SDK + i] * ck[c][i], i ascending
        for (int e = tid; e < kLutBlock * kRows; e += kThreads) {
          const int sl = e / kRows, c = e % kRows;
          const int sg = min(sb * kLutBlock + sl, n_sub_k - 1);
          const float *qs = qt + sg * SDK;
          const float *cc = ck + c * SDK;
          float x = qs[0] * cc[0];
#pragma unroll
          for (int i = 1; i < SDK; ++i) x = __builtin_fmaf(qs[i], cc[i], x);
          lut[e] = x;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kTokPerLane; ++i) {
#pragma unroll
          for (int k4 = 0; k4 < kLutBlock / 4; ++k4) {
            const int w = sb * (kLutBlock / 4) + k4;
            if (w < kwords) {
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                const int sl = 4 * k4 + k;
                const float l = lut[sl * kRows + ((kw[i][w] >> (8 * k)) & 0xFFu)];
                acc[i] = (w == 0 && k == 0) ? l : acc[i] + l;
              }
            }
          }
        }
      }
    }
    float sc[kTokPerLane];
    float mloc = kNegInf;
#pragma unroll
    for (int i = 0; i < kTokPerLane; ++i) {
      const int t = t0 + tid + kThreads * i;
      sc[i] = (t >= lo && t < hi) ? acc[i] : kNegInf;
      mloc = fmaxf(mloc, sc[i]);
    }
    const float m = block_max(mloc, red);
    float lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < kTokPerLane; ++i) {
      const float e = exp2f(sc[i] - m);  // masked: exp2(-inf) = 0
      p[j * kChunk + tid + kThreads * i] = e;
      lsum += e;
    }
    const float l = block_sum(lsum, red);
    if (tid == 0) {
      float *pj = part + static_cast<int64_t>(j) * a.n_chunks * part_stride;
      pj[D] = m;
      pj[D + 1] = l;
    }
  }
  __syncthreads();  // all weights are in p

  // value sum, kVGroup heads per pass: lane (s, grp) walks tokens lo + grp,
  // lo + grp + ng, ...; one value-codebook row read feeds every head
  const int ng = kThreads / n_sub_v;
  const int s = tid % n_sub_v, grp = tid / n_sub_v;
  for (int j0 = 0; j0 < g; j0 += kVGroup) {
    float vacc[kVGroup][SDV];
#pragma unroll
    for (int j = 0; j < kVGroup; ++j)
#pragma unroll
      for (int i = 0; i < SDV; ++i) vacc[j][i] = 0.0f;
    if (grp < ng) {
      // codes of kVPrefetch tokens per batch; the next batch's loads are in
      // flight while the current batch is summed
      int cs[kVPrefetch], nx[kVPrefetch];
#pragma unroll
      for (int u = 0; u < kVPrefetch; ++u)
        cs[u] = vc[static_cast<int64_t>(min(lo + grp + u * ng, hi - 1)) * n_sub_v + s];
      for (int tb = lo + grp; tb < hi; tb += ng * kVPrefetch) {
#pragma unroll
        for (int u = 0; u < kVPrefetch; ++u) {
          const int t = min(tb + (kVPrefetch + u) * ng, hi - 1);
          nx[u] = vc[static_cast<int64_t>(t) * n_sub_v + s];
        }
#pragma unroll
        for (int u = 0; u < kVPrefetch; ++u) {
          const int t = tb + u * ng;
          if (t >= hi) break;
          float v[SDV];
#pragma unroll
          for (int q4 = 0; q4 < SDV / 4; ++q4) {
            const float4 w = *reinterpret_cast<const float4 *>(cv + cs[u] * SDV + 4 * q4);
            v[4 * q4] = w.x;
            v[4 * q4 + 1] = w.y;
            v[4 * q4 + 2] = w.z;
            v[4 * q4 + 3] = w.w;
          }
#pragma unroll
          for (int j = 0; j < kVGroup; ++j) {
            if (j0 + j < g) {
              const float pw = p[(j0 + j) * kChunk + (t - t0)];
#pragma unroll
              for (int i = 0; i < SDV; ++i) vacc[j][i] = __builtin_fmaf(pw, v[i], vacc[j][i]);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < kVPrefetch; ++u) cs[u] = nx[u];
      }
    }
    // sum the token groups, one head at a time
#pragma unroll
    for (int j = 0; j < kVGroup; ++j) {
      if (j0 + j < g) {  // uniform
        if (grp < ng) {
#pragma unroll
          for (int i = 0; i < SDV; ++i) red[grp * D + s * SDV + i] = vacc[j][i];
        }
        __syncthreads();
        float *pj = part + static_cast<int64_t>(j0 + j) * a.n_chunks * part_stride;
        for (int d = tid; d < D; d += kThreads) {
          float o = red[d];
          for (int r = 1; r < ng; ++r) o += red[r * D + d];
          pj[d] = o;
        }
        __syncthreads();
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core form (head_dim 128 or 256, 16-byte aligned code rows): the
// scores of 16 tokens for up to 16 rows of query parts are one
// v_mfma_f32_16x16x32 per 32 elements of the head dimension:
//   rows     (query head, part): the query q~ = q / f * scale * log2(e),
//            multiplied by 2^E (E per head, max |q~| 2^E in [2^13, 2^14)),
//            is split exactly into element-type parts, q~ 2^E = sum of parts
//            + e with |e| <= 2^-22 |q~ 2^E| + 2^-25 (fp16: hi, lo; bf16: four
//            parts, |e| <= 2^-32 |q~ 2^E|);
//   columns  16 tokens; the B operand of lane (token, quarter) is the key
//            codebook rows of its codes, gathered from LDS;
//   score    = 2^-E (sum of the head's part rows).
// Products of element-type values are exact in fp32 and the instruction's
// accumulation errs by less than 4 u (sum |terms| + |C|) (measured), so the
// score error stays below (4 head_dim/32 + 3) u sum_i |q_i k_i| -- inside the
// bound of the LUT form.  Each wave scores 64 tokens of the 256-token chunk;
// after one barrier the chunk maximum is known and the weights go to LDS;
// for the value sum every wave takes a quarter of the value sub-spaces over
// all 256 tokens, so its results go straight to the partial with no
// reduction across waves.
constexpr int kWaveTok = 64;
constexpr int kMChunk = kWaveTok * (kThreads / 64);  // 256 tokens per workgroup

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool BF16>
__device__ __forceinline__ f32x4 mfma16(const uint4 &a, const uint4 &b, const f32x4 &c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Round a finite fp32 value to the element type (nearest, ties to even).
template <bool BF16>
__device__ __forceinline__ uint16_t narrow_rn(float v) {
  if constexpr (BF16) {
    const uint32_t u = __float_as_uint(v);
    if (!(__builtin_fabsf(v) <= 3.4028234663852886e38f))
      return static_cast<uint16_t>((u >> 16) | ((v != v) ? 0x40u : 0u));
    return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
  } else {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Max / sum over the 16 lanes of a DPP row (xor 1, xor 2, half mirror,
// mirror); every lane of the row ends with the same value.
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  return fmaxf(v, dpp_f<0x140>(v));
}
__device__ __forceinline__ float row_sum16(float v) {
  v = v + dpp_f<0xB1>(v);
  v = v + dpp_f<0x4E>(v);
  v = v + dpp_f<0x141>(v);
  return v + dpp_f<0x140>(v);
}

// LDS of the matrix-core kernel for up to GC query heads per kv head.  All
// of it is static: the value codes are the target of asynchronous copies, and
// the compiler tells them apart from the other LDS objects only then.
template <int SDK, int SDV, bool BF16, int D, int GC>
struct MLayout {
  static constexpr int kNSK = D / SDK, kNSV = D / SDV;
  static constexpr int kParts = BF16 ? 4 : 2;  // element-type parts of a split fp32 value
  static constexpr int kHeadsPerBlock = 16 / kParts;
  static constexpr int kPieces = kNSV / 16;    // 16-byte pieces per value-code row
  static constexpr int kTokGroups = 4 / kPieces;
  // the value codes of the chunk, later the value sums of token groups > 0
  // (head_dim < 4 * 16 * SDV)
  static constexpr int kCodes = kMChunk * kNSV;
  static constexpr int kRed = (kTokGroups - 1) * GC * D * 4;
  static constexpr int kCodeBytes = kCodes > kRed ? kCodes : kRed;
  // query parts [GC * kParts][D] (scores), then the weights [GC * kParts][256]
  static constexpr int kRowElems = GC * kParts * (D > kMChunk ? D : kMChunk);
  static constexpr size_t kBytes = 2 * 256 * (SDK + SDV) + 2 * kRowElems + kCodeBytes +
                                   4 * (2 * kMaxGroup + 2 * 4 * kMaxGroup);
};

// Elements e of the rows r[0..7] (each row SDV element-type values in SDV/2
// words) as the 8 K values of a B operand: word m = (r[2m][e], r[2m+1][e]).
template <int SDV>
__device__ __forceinline__ uint4 column_of(const uint32_t (&r)[8][SDV / 2], int e) {
  const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high or low halves
  uint32_t o[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
    o[m] = __builtin_amdgcn_perm(r[2 * m + 1][e >> 1], r[2 * m][e >> 1], sel);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Asynchronous copy of 16 bytes per lane from global memory to LDS
// (global_load_lds_dwordx4): lane l of the wave writes lds + 16 l; `lds` is
// the same for every lane.  The target is an LDS object of its own, so the
// compiler does not make accesses to other LDS objects wait for the copy.
__device__ __forceinline__ void copy16_to_lds(const void *src, void *lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                   (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// Waits until every vector memory operation of the wave has completed.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Value codes of a chunk in LDS, token-major; piece p (16 bytes) of token t
// sits at position p ^ ((t / 8) mod VP) of its row, so that the rows of
// tokens 8 apart, read together by the value sum, start on different banks.
// Byte offset of the code of (token tc, sub-space s):
template <int VP, int NSV>
__device__ __forceinline__ int code_at(int tc, int s) {
  return tc * NSV + (((s >> 4) ^ ((tc >> 3) & (VP - 1))) << 4) + (s & 15);
}

// Waves per SIMD the register budget is set for (6 fit the LDS of the common
// fp16 shapes; the wider forms need more registers).
template <int SDV_, bool BF16_, int GC_>
constexpr int kMfmaWaves = BF16_ ? (SDV_ == 8 ? 3 : 4) : (SDV_ == 8 || GC_ == 8 ? 5 : 6);

template <int SDK, int SDV, bool BF16, int D, int GC>
__global__ void __launch_bounds__(kThreads, (kMfmaWaves<SDV, BF16, GC>))
attn_mfma_partial(const AttnArgs a) {
  using LY = MLayout<SDK, SDV, BF16, D, GC>;
  constexpr int NSK = LY::kNSK, NSV = LY::kNSV;
  constexpr int QB = NSK / 4;          // key-code bytes per lane quarter (4, 8 or 16)
  constexpr int NQW = QB / 4;          // their 32-bit words
  constexpr int NI = D / 32;           // score instructions per 16 tokens
  constexpr int P = LY::kParts;
  constexpr int GB = LY::kHeadsPerBlock;
  constexpr int HPL = 4 / P;           // heads per lane in the output layout
  constexpr int VP = LY::kPieces;      // 16-byte value-code pieces per thread and per row
  constexpr int WG = NSV / 16;         // waves covering all value sub-spaces (16 each)
  constexpr int TG = LY::kTokGroups;   // token groups of the value sum
  static_assert(QB % 4 == 0 && NSV % 16 == 0 && WG * TG == 4, "shape");
  constexpr float kPScale = 16384.0f;  // weights in (0, 1] are split as p 2^14

  __shared__ uint4 ktab_s[256 * SDK / 8];       // key codebook, element bits
  __shared__ uint4 vtab4[256 * SDV / 8];        // value codebook, element bits
  __shared__ uint4 rows4[LY::kRowElems / 8];    // query parts, then weights
  __shared__ uint4 codes4[LY::kCodeBytes / 16];  // value codes, then value sums
  __shared__ int qexp[kMaxGroup];               // E of each head
  __shared__ float cmax[kMaxGroup];             // chunk maximum per head
  __shared__ float wmax[4 * kMaxGroup];         // per wave and head
  __shared__ float wsum[4 * kMaxGroup];
  const int g = a.Hq / a.Hkv;
  const int nb = (g + GB - 1) / GB;
  const int nrows = g * P;             // rows (head, part) in use
  uint16_t *ktab = reinterpret_cast<uint16_t *>(ktab_s);
  uint16_t *vtab = reinterpret_cast<uint16_t *>(vtab4);
  uint16_t *qp = reinterpret_cast<uint16_t *>(rows4);
  uint16_t *pp = reinterpret_cast<uint16_t *>(rows4);  // after the scores
  uint8_t *codes = reinterpret_cast<uint8_t *>(codes4);
  float *red = reinterpret_cast<float *>(codes4);  // after the value sum

  // chunks rotate with (sequence, head): workgroup i runs on XCD i mod 8, so
  // a fixed chunk-to-x map would give the XCDs that hold late (often empty)
  // chunks of every sequence far less work than the others
  const int chunk = (blockIdx.x + blockIdx.y + gridDim.y * blockIdx.z) % gridDim.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int L = a.kv_len ? a.kv_len[b] : a.S;
  L = min(max(L, 0), a.S);
  const int first = a.window > 0 ? max(0, L - a.window) : 0;
  const int t0 = chunk * kMChunk;
  const int lo = max(first, t0), hi = min(L, t0 + kMChunk);
  const int64_t part_stride = D + 2;
  const int64_t head_stride = static_cast<int64_t>(a.n_chunks) * part_stride;
  float *part = a.ws + ((static_cast<int64_t>(b) * a.Hq + h * g) * a.n_chunks + chunk) * part_stride;
  if (lo >= hi) {  // nothing attended here (uniform)
    for (int j = 0; j < g; ++j) {
      float *pj = part + j * head_stride;
      for (int d = tid; d < D; d += kThreads) pj[d] = 0.0f;
      if (tid == 0) {
        pj[D] = kNegInf;
        pj[D + 1] = 0.0f;
      }
    }
    return;
  }

  // ---- every global load is issued here, in the order it is needed: the
  // codebooks, the query rows, then the codes (clamped token indices) --------
  const int n_c = a.n_c;
  const uint16_t *kcb = a.k_cb + static_cast<int64_t>(h) * n_c * SDK;
  const uint16_t *vcb = a.v_cb + static_cast<int64_t>(h) * n_c * SDV;
  uint16_t kv[SDK], vv[SDV];
#pragma unroll
  for (int k = 0; k < SDK; ++k) kv[k] = kcb[min(tid + kThreads * k, n_c * SDK - 1)];
#pragma unroll
  for (int k = 0; k < SDV; ++k) vv[k] = vcb[min(tid + kThreads * k, n_c * SDV - 1)];
  // query head slots w and w + 4 of this wave (slot < g), elements lane + 64 k
  uint16_t qv[2][D / 64];
  float ks[D / 64];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int hq = h * g + min(w + 4 * j, g - 1);
    const uint16_t *qrow = a.q + (static_cast<int64_t>(b) * a.Hq + hq) * D;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) qv[j][k] = qrow[lane + 64 * k];
  }
#pragma unroll
  for (int k = 0; k < D / 64; ++k)
    ks[k] = a.k_scale ? a.k_scale[static_cast<int64_t>(h) * D + lane + 64 * k] : 1.0f;

  const int64_t row0 = (static_cast<int64_t>(b) * a.Hkv + h) * a.S;
  const uint8_t *kc = a.k_codes + row0 * NSK;
  const uint8_t *vc = a.v_codes + row0 * NSV;
  const int col = lane & 15, kg = lane >> 4;
  uint32_t kw[4][NQW];  // key codes: quarter kg of token t0 + 64 w + 16 G + col
#pragma unroll
  for (int G = 0; G < 4; ++G) {
    const int t = min(max(t0 + w * kWaveTok + 16 * G + col, lo), hi - 1);
    const uint8_t *src = kc + static_cast<int64_t>(t) * NSK + kg * QB;
    if constexpr (NQW == 4) {
      const uint4 q = *reinterpret_cast<const uint4 *>(src);
      kw[G][0] = q.x;
      kw[G][1] = q.y;
      kw[G][2] = q.z;
      kw[G][3] = q.w;
    } else if constexpr (NQW == 2) {
      const uint2 q = *reinterpret_cast<const uint2 *>(src);
      kw[G][0] = q.x;
      kw[G][1] = q.y;
    } else {
      kw[G][0] = *reinterpret_cast<const uint32_t *>(src);
    }
  }
  // ---- codebooks of kv head h into LDS (rows past n_c are zero) -------------
#pragma unroll
  for (int k = 0; k < SDK; ++k) {
    const int e = tid + kThreads * k;
    ktab[e] = (e < n_c * SDK) ? kv[k] : static_cast<uint16_t>(0);
  }
#pragma unroll
  for (int k = 0; k < SDV; ++k) {
    const int e = tid + kThreads * k;
    vtab[e] = (e < n_c * SDV) ? vv[k] : static_cast<uint16_t>(0);
  }

  // ---- query parts: wave w splits heads w and w + 4 into rows h P + part ----
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int hs = w + 4 * j;
    if (hs < g) {  // uniform per wave
      uint16_t *rows = qp + static_cast<int64_t>(hs) * P * D;
      float x[D / 64];
      float mx = 0.0f;
#pragma unroll
      for (int k = 0; k < D / 64; ++k) {
        float v = widen<BF16>(qv[j][k]);
        if (a.k_scale) v = v / ks[k];
        v = v * a.qmul;
        x[k] = v;
        mx = fmaxf(mx, __builtin_fabsf(v));
      }
      mx = row_max16(mx);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      int E = 0;
      if (mx > 0.0f && mx <= 3.4028234663852886e38f) {
        int ex;
        (void)frexpf(mx, &ex);  // mx = f 2^ex, f in [0.5, 1)
        E = 14 - ex;            // max |q~| 2^E in [2^13, 2^14)
      }
      if (lane == 0) qexp[hs] = E;
#pragma unroll
      for (int k = 0; k < D / 64; ++k) {
        const int d = lane + 64 * k;
        float r = ldexpf(x[k], E);
#pragma unroll
        for (int q = 0; q < P; ++q) {  // r - part is exact in fp32
          const uint16_t pb = narrow_rn<BF16>(r);
          rows[q * D + d] = pb;
          r = r - widen<BF16>(pb);
        }
      }
    }
  }
  __syncthreads();

  // value codes of the chunk straight to LDS, in flight during the scores
  // (the key codes have landed first, so that their uses do not wait for
  // the copies): wave w fills pieces
  // 64 VP w .. 64 VP (w + 1) - 1 (slot e: token e / VP, position e % VP)
  wait_vm_all();
#pragma unroll
  for (int q = 0; q < VP; ++q) {
    const int e0 = 64 * VP * w + 64 * q, e = e0 + lane;
    const int tc = e / VP, pos = e % VP;
    const int t = min(max(t0 + tc, lo), hi - 1);
    copy16_to_lds(vc + static_cast<int64_t>(t) * NSV + 16 * (pos ^ ((tc >> 3) & (VP - 1))),
                  codes4 + e0);
  }

  // ---- scores on the matrix cores: wave w, tokens t0 + 64 w + 16 G + col ----
  // lane (col, kg): A = row col of a block at elements kg D/4 + 8 i .. + 7
  // (rows past g P are zero); B = the key rows of its codes for the same
  // elements; the result rows 4 kg .. 4 kg + 3 are (head, part) rows
  float sreg[2][4][HPL];  // blocks x groups x heads of the lane (bf16: 2 blocks)
  const uint2 *ktab2 = reinterpret_cast<const uint2 *>(ktab);
  const uint4 *ktab4 = reinterpret_cast<const uint4 *>(ktab);
#pragma unroll
  for (int hb = 0; hb < (BF16 ? 2 : 1); ++hb) {
    if (hb < nb) {  // uniform
      const int ar = hb * 16 + col;
      const uint16_t *arow = qp + static_cast<int64_t>(min(ar, nrows - 1)) * D + kg * (D / 4);
      uint4 areg[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const uint4 v = *reinterpret_cast<const uint4 *>(arow + 8 * i);
        areg[i] = ar < nrows ? v : make_uint4(0, 0, 0, 0);
      }
      int ex[HPL];
#pragma unroll
      for (int j = 0; j < HPL; ++j) ex[j] = qexp[min(hb * GB + kg * HPL + j, kMaxGroup - 1)];
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          uint4 bop;
          if constexpr (SDK == 4) {
            const uint32_t wd = kw[G][i >> 1];
            const uint32_t c0 = (wd >> (16 * (i & 1))) & 0xFFu;
            const uint32_t c1 = (wd >> (16 * (i & 1) + 8)) & 0xFFu;
            const uint2 r0 = ktab2[c0], r1 = ktab2[c1];
            bop = make_uint4(r0.x, r0.y, r1.x, r1.y);
          } else {
            const uint32_t c = (kw[G][i >> 2] >> (8 * (i & 3))) & 0xFFu;
            bop = ktab4[c];
          }
          acc = mfma16<BF16>(areg[i], bop, acc);
        }
        const int t = t0 + w * kWaveTok + 16 * G + col;
        const bool valid = t >= lo && t < hi;
        if constexpr (P == 2) {
          sreg[hb][G][0] = valid ? ldexpf(acc[0] + acc[1], -ex[0]) : kNegInf;
          sreg[hb][G][1] = valid ? ldexpf(acc[2] + acc[3], -ex[1]) : kNegInf;
        } else {
          sreg[hb][G][0] = valid ? ldexpf(((acc[3] + acc[2]) + acc[1]) + acc[0], -ex[0]) : kNegInf;
        }
      }
      // this wave's maximum per head
#pragma unroll
      for (int j = 0; j < HPL; ++j) {
        float m = kNegInf;
#pragma unroll
        for (int G = 0; G < 4; ++G) m = fmaxf(m, sreg[hb][G][j]);
        m = row_max16(m);
        const int hh = hb * GB + kg * HPL + j;
        if (col == 0 && hh < g) wmax[w * kMaxGroup + hh] = m;
      }
    }
  }
  __syncthreads();

  // ---- weights against the chunk maximum, stored split: rows h P + part of
  // pp hold the element-type parts of p 2^14 -----------------------------------
#pragma unroll
  for (int hb = 0; hb < (BF16 ? 2 : 1); ++hb) {
    if (hb < nb) {
#pragma unroll
      for (int j = 0; j < HPL; ++j) {
        const int hh = hb * GB + kg * HPL + j;
        const int hc = min(hh, g - 1);
        float M = wmax[hc];
#pragma unroll
        for (int v = 1; v < 4; ++v) M = fmaxf(M, wmax[v * kMaxGroup + hc]);
        float lsum = 0.0f;
#pragma unroll
        for (int G = 0; G < 4; ++G) {
          const float sv = sreg[hb][G][j];
          // v_exp_f32 directly: M is finite (the chunk attends a token) and
          // a masked score of -inf gives 2^-inf = 0; results below 2^-126
          // (flushed) are far below the split's resolution of 2^-38
          const float pv = __builtin_amdgcn_exp2f(sv - M);
          lsum += pv;
          if (hh < g) {
            const int tc = w * kWaveTok + 16 * G + col;
            float r = pv * kPScale;
#pragma unroll
            for (int q = 0; q < P; ++q) {
              const uint16_t pb = narrow_rn<BF16>(r);
              pp[(hh * P + q) * kMChunk + tc] = pb;
              r = r - widen<BF16>(pb);
            }
          }
        }
        lsum = row_sum16(lsum);
        if (col == 0 && hh < g) wsum[w * kMaxGroup + hh] = lsum;
        if (w == 0 && col == 0 && hh < g) cmax[hh] = M;
      }
    }
  }
  // every wave's value-code copies have landed before any wave reads them
  wait_vm_all();
  __syncthreads();

  // ---- value sum on the matrix cores: wave w takes sub-spaces 16 (w % WG)
  // .. + 15 (columns) over the 32-token blocks tg, tg + TG, ... (K), one
  // instruction per value element; lane (col, kg) gathers the rows of its
  // sub-space for 8 tokens and regroups them by element --------------------
  const int sb = w % WG, tg = w / WG;
  const int sv = sb * 16 + col;
  f32x4 vacc[2][SDV];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int e = 0; e < SDV; ++e) vacc[hb][e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  constexpr int kBlocks = kMChunk / 32 / TG;  // 32-token blocks per wave
#pragma unroll 2
  for (int m = 0; m < kBlocks; ++m) {
    const int tk = (tg + TG * m) * 32 + kg * 8;  // this lane's 8 tokens
    uint32_t rw[8][SDV / 2];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t c = codes[code_at<VP, NSV>(tk + j, sv)];
      if constexpr (SDV == 4) {
        const uint2 r = reinterpret_cast<const uint2 *>(vtab)[c];
        rw[j][0] = r.x;
        rw[j][1] = r.y;
      } else {
        const uint4 r = reinterpret_cast<const uint4 *>(vtab)[c];
        rw[j][0] = r.x;
        rw[j][1] = r.y;
        rw[j][2] = r.z;
        rw[j][3] = r.w;
      }
    }
#pragma unroll
    for (int hb = 0; hb < (BF16 ? 2 : 1); ++hb) {
      if (hb < nb) {
        const int ar = hb * 16 + col;
        const uint4 av =
            *reinterpret_cast<const uint4 *>(pp + min(ar, nrows - 1) * kMChunk + tk);
        const uint4 aop = ar < nrows ? av : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < SDV; ++e)
          vacc[hb][e] = mfma16<BF16>(aop, column_of<SDV>(rw, e), vacc[hb][e]);
      }
    }
  }
  // rows 4 kg .. 4 kg + 3 of column col: the (head, part) rows of heads
  // hb GB + kg HPL + j, element e of sub-space sv
  float o[2][HPL][SDV];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int e = 0; e < SDV; ++e) {
      const f32x4 v = vacc[hb][e];
      if constexpr (P == 2) {
        o[hb][0][e] = (v[0] + v[1]) * (1.0f / kPScale);
        o[hb][1][e] = (v[2] + v[3]) * (1.0f / kPScale);
      } else {
        o[hb][0][e] = (((v[3] + v[2]) + v[1]) + v[0]) * (1.0f / kPScale);
      }
    }
  if constexpr (TG > 1) {
    // token groups 1 .. TG-1 hand their sums to group 0 through LDS
    __syncthreads();  // every wave is done with the codes
    if (tg > 0) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int j = 0; j < HPL; ++j) {
          const int hh = hb * GB + kg * HPL + j;
          if (hb < nb && hh < g) {
#pragma unroll
            for (int e = 0; e < SDV; ++e) red[((tg - 1) * g + hh) * D + sv * SDV + e] = o[hb][j][e];
          }
        }
    }
    __syncthreads();
    if (tg == 0) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int j = 0; j < HPL; ++j) {
          const int hh = hb * GB + kg * HPL + j;
          if (hb < nb && hh < g) {
#pragma unroll
            for (int e = 0; e < SDV; ++e)
              for (int q = 1; q < TG; ++q) o[hb][j][e] += red[((q - 1) * g + hh) * D + sv * SDV + e];
          }
        }
    }
  }
  if (tg == 0) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int j = 0; j < HPL; ++j) {
        const int hh = hb * GB + kg * HPL + j;
        if (hb < nb && hh < g) {
          float *dst = part + hh * head_stride + sv * SDV;
#pragma unroll
          for (int q4 = 0; q4 < SDV / 4; ++q4)
            reinterpret_cast<float4 *>(dst)[q4] =
                make_float4(o[hb][j][4 * q4], o[hb][j][4 * q4 + 1], o[hb][j][4 * q4 + 2],
                            o[hb][j][4 * q4 + 3]);
        }
      }
  }
  if (tid < g) {
    float *pj = part + tid * head_stride;
    const float l = ((wsum[tid] + wsum[kMaxGroup + tid]) + wsum[2 * kMaxGroup + tid]) +
                    wsum[3 * kMaxGroup + tid];
    pj[D] = cmax[tid];
    pj[D + 1] = l;
  }
}

// Merge `count` partials of one (sequence, query head), `cstride` floats
// apart: thread d.  Partials are taken 16 at a time: lanes 0..15 load their
// (m, l) pairs and the threads their 16 o values, every load in flight
// (clamped indices); each batch is merged against the running maximum.  An
// empty partial has m = -inf (weight 0), l = 0 and o = 0.
__device__ __forceinline__ void merge_partials(const float *part, int count, int64_t cstride,
                                               int D, float *out) {
  constexpr int kBatch = 16;
  __shared__ float bm[kBatch], bl[kBatch];
  const int d = threadIdx.x, dc = min(d, D - 1);
  float M = kNegInf, l = 0.0f, acc = 0.0f;
  for (int c0 = 0; c0 < count; c0 += kBatch) {  // uniform
    float oc[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) oc[j] = part[min(c0 + j, count - 1) * cstride + dc];
    if (d < kBatch) {
      const float *pc = part + min(c0 + d, count - 1) * cstride;
      const float mj = pc[D], lj = pc[D + 1];
      bm[d] = c0 + d < count ? mj : kNegInf;
      bl[d] = lj;
    }
    __syncthreads();
    float m[kBatch], lc[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      m[j] = bm[j];
      lc[j] = bl[j];
    }
    __syncthreads();  // bm, bl are refilled by the next batch
    float Mb = M;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) Mb = fmaxf(Mb, m[j]);
    if (Mb != kNegInf) {
      const float r = exp2f(M - Mb);  // 0 while nothing is merged yet
      l *= r;
      acc *= r;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const float wj = exp2f(m[j] - Mb);
        l = __builtin_fmaf(lc[j], wj, l);
        acc = __builtin_fmaf(oc[j], wj, acc);
      }
      M = Mb;
    }
  }
  if (d < D) out[d] = M == kNegInf ? 0.0f : acc / l;
}

// Merge of the chunked form: the n_chunks partials of (sequence, query head)
// blockIdx.x.
__global__ void __launch_bounds__(kThreads)
attn_combine(const AttnArgs a) {
  const int bh = blockIdx.x;
  const int64_t part_stride = a.D + 2;
  merge_partials(a.ws + static_cast<int64_t>(bh) * a.n_chunks * part_stride, a.n_chunks,
                 part_stride, a.D, a.out + static_cast<int64_t>(bh) * a.D);
}

// ---- streaming form (matrix cores, balanced token ranges) -----------------
// The chunked form above gives every (sequence, kv head, 256-token chunk) a
// workgroup of its own: all of them are resident at once, so their loads,
// scores, softmax and value sums run in lockstep, and each writes a partial.
// Here the attended tokens of all (sequence, kv head) segments are cut into
// 64-token slices, laid end to end in (sequence, kv head, slice) order, and
// workgroup i of G takes slices [U i / G, U (i+1) / G) of the U in total
// (every workgroup reads the lengths and finds its range itself).  A
// workgroup works through the segment parts in its range; for each it stages
// the codebooks and the split query rows once, then its 4 waves take the
// part's slices in turn, each with a running softmax of its own (running
// maximum and sum per head, value sums rescaled when the maximum rises), the
// next slice's key codes (registers) and value codes (LDS, asynchronous)
// in flight while the current one is computed, and no barrier between
// slices.  At the end of a part the waves merge through LDS and write one
// partial per head into slot i + sigma (sigma = b Hkv + h: the slots of the
// (workgroup, segment) pairs along the range increase strictly, so they are
// distinct); the first and the last workgroup of each segment are recorded
// for the merge launch.  The arithmetic per slice is that of the chunked
// form: the query split exactly into element-type parts, scores
// and value sums on v_mfma_f32_16x16x32, weights p 2^14 split the same way.
constexpr int kSlice = 64;        // tokens per wave step
// Fourth word of a raw buffer resource on this target (untyped 32-bit data).
constexpr int kBufferWord3 = 0x00020000;
// Workgroups per CU the registers are budgeted for: 3, or 2 when the value
// sums take more than 8 accumulator blocks (bf16 or 8 heads per kv head at
// head_dim 256).
template <bool BF16, int D, int GC>
constexpr int kStreamPerCu = ((BF16 ? 4 : 2) * GC * 4 + 15) / 16 * (D / 64) > 8 ? 2 : 3;

// Attended slices of sequence b: tokens [first, L).
__device__ __forceinline__ int seq_slices(const AttnArgs &a, int b, int &first, int &L) {
  int len = a.kv_len ? a.kv_len[b] : a.S;
  len = min(max(len, 0), a.S);
  first = a.window > 0 ? max(0, len - a.window) : 0;
  L = len;
  return (len - first + kSlice - 1) / kSlice;
}

// Inclusive prefix sum of v over the workgroup (kThreads threads); `total`
// gets the sum of all.  `sc` holds kThreads / 64 words of LDS.
__device__ __forceinline__ int64_t block_scan(int64_t v, int64_t *sc, int64_t &total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  if (lane == 63) sc[w] = v;
  __syncthreads();
  int64_t off = 0;
  total = 0;
#pragma unroll
  for (int k = 0; k < kThreads / 64; ++k) {
    off += k < w ? sc[k] : 0;
    total += sc[k];
  }
  __syncthreads();  // sc is refilled by the next call
  return v + off;
}

// Waits until every LDS operation of the wave has completed.
__device__ __forceinline__ void wait_lgkm_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Waits until at most 4 vector memory operations of the wave are in flight
// (vmcnt(4)): the 4 key-code loads of the next slice.
__device__ __forceinline__ void wait_vm_keys() { __builtin_amdgcn_s_waitcnt(0x0F74); }

template <int SDK, int SDV, bool BF16, int D, int GC>
__global__ void __launch_bounds__(kThreads, (kStreamPerCu<BF16, D, GC>))
attn_stream_partial(const AttnArgs a) {
  constexpr int NSK = D / SDK, NSV = D / SDV;
  constexpr int QB = NSK / 4;          // key-code bytes per lane quarter (4, 8 or 16)
  constexpr int NQW = QB / 4;          // their 32-bit words
  constexpr int NI = D / 32;           // score instructions per 16 tokens
  constexpr int P = BF16 ? 4 : 2;      // element-type parts of a split fp32 value
  constexpr int HPL = 4 / P;           // heads per lane in the score layout
  constexpr int NR = GC * P;           // rows (head, part) at most
  constexpr int ZR = NR;               // the all-zero row
  constexpr int VP = NSV / 16;         // 16-byte pieces per value-code row
  constexpr int NCG = NSV / 16;        // 16-sub-space column groups of the value sum
  constexpr int NRB = (NR * 4 + 15) / 16;  // 16-row blocks (head, part, element)
  constexpr int CB = kSlice * NSV;     // value-code bytes of one slice
  constexpr int QS = D + 8;            // row stride of the query parts (halves)
  constexpr int PS = kSlice + 8;       // row stride of the weights (halves)
  constexpr float kPScale = 16384.0f;  // weights in (0, 1] are split as p 2^14
  static_assert(SDV == 4 && QB % 4 == 0 && NSV % 16 == 0 && NR <= 16, "shape");

  __shared__ uint4 ktab_s[256 * SDK / 8];         // key codebook, element bits
  __shared__ uint4 vtab_s[256 * SDV / 8];         // value codebook, element bits
  __shared__ uint4 qrow_s[(NR + 1) * QS / 8];     // query parts, rows (head, part); zero row
  __shared__ uint4 prow_s[4][(NR + 1) * PS / 8];  // per wave: weights, rows (head, part); zero row
  __shared__ uint4 vbuf_s[4][CB / 16];            // per wave: value codes of the next slice
  __shared__ float red[3 * GC * D];               // waves 1..3: scaled value sums
  __shared__ float wm[4][GC], wl[4][GC];          // per wave: running maximum, sum
  __shared__ float walpha[4][GC];                 // per wave: rescale factors
  __shared__ int qexp[GC];                        // E of each head
  __shared__ int64_t scan_s[kThreads / 64];
  __shared__ int found_b, found_first, found_len;
  __shared__ int64_t found_seq0;

  const int g = a.Hq / a.Hkv;
  const int nrows = g * P;             // rows (head, part) in use
  const int wg = blockIdx.x, G = gridDim.x;
  uint16_t *ktab = reinterpret_cast<uint16_t *>(ktab_s);
  uint16_t *vtab = reinterpret_cast<uint16_t *>(vtab_s);
  uint16_t *qp = reinterpret_cast<uint16_t *>(qrow_s);

  // the zero rows (read for the rows past g P of the matrix operands)
  for (int e = NR * QS / 8 + threadIdx.x; e < (NR + 1) * QS / 8; e += kThreads)
    qrow_s[e] = make_uint4(0, 0, 0, 0);
  for (int e = NR * PS / 8 + (threadIdx.x & 63); e < (NR + 1) * PS / 8; e += 64)
    prow_s[threadIdx.x >> 6][e] = make_uint4(0, 0, 0, 0);

  // ---- this workgroup's slice range --------------------------------------
  // (one pass over the lengths when they fit one round of threads: the
  // prefix sums that give the total also locate s_begin)
  int64_t U, s_begin, s_end;
  if (threadIdx.x == 0) {
    found_b = a.B;  // (not found: no part runs)
    found_seq0 = 0;
    found_first = found_len = 0;
  }
  if (a.B <= kThreads) {
    const int bb = threadIdx.x;
    int f = 0, L = 0;
    const int64_t v = bb < a.B ? seq_slices(a, bb, f, L) : 0;
    int64_t tot;
    const int64_t incl = block_scan(v, scan_s, tot);
    U = tot * a.Hkv;
    s_begin = U * wg / G;
    s_end = U * (wg + 1) / G;
    if (s_begin >= s_end) return;  // uniform
    const int64_t lo = (incl - v) * a.Hkv, hi = incl * a.Hkv;
    if (v > 0 && lo <= s_begin && s_begin < hi) {
      found_b = bb;
      found_seq0 = lo;
      found_first = f;
      found_len = L;
    }
    __syncthreads();
  } else {
    int64_t mine = 0;
    for (int b = threadIdx.x; b < a.B; b += kThreads) {
      int f, L;
      mine += seq_slices(a, b, f, L);
    }
    (void)block_scan(mine, scan_s, U);
    U *= a.Hkv;
    s_begin = U * wg / G;
    s_end = U * (wg + 1) / G;
    if (s_begin >= s_end) return;  // uniform
    int64_t run = 0;
    for (int base = 0; base < a.B; base += kThreads) {  // uniform
      const int bb = base + static_cast<int>(threadIdx.x);
      int f = 0, L = 0;
      const int64_t v = bb < a.B ? static_cast<int64_t>(a.Hkv) * seq_slices(a, bb, f, L) : 0;
      int64_t tot;
      const int64_t incl = block_scan(v, scan_s, tot);
      if (v > 0 && run + incl - v <= s_begin && s_begin < run + incl) {
        found_b = bb;
        found_seq0 = run + incl - v;
        found_first = f;
        found_len = L;
      }
      run += tot;
      __syncthreads();
      if (run > s_begin) break;
    }
  }
  // uniform values (scalar registers): the part loop and the buffer
  // resources derived from them are the same for every lane
  int b = __builtin_amdgcn_readfirstlane(found_b);
  const int b_found = b;
  const int first_found = __builtin_amdgcn_readfirstlane(found_first);
  const int len_found = __builtin_amdgcn_readfirstlane(found_len);
  int64_t seq0;
  {
    const uint64_t s0 = static_cast<uint64_t>(found_seq0);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(s0));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(s0 >> 32));
    seq0 = static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
  }
  int *tab_first = reinterpret_cast<int *>(
      a.ws + static_cast<int64_t>(G + a.B * a.Hkv - 1) * g * (D + 2));
  int *tab_last = tab_first + a.B * a.Hkv;

  int64_t pos = s_begin;
  while (pos < s_end && b < a.B) {  // uniform: one segment part per pass
    int first = first_found, L = len_found;
    const int ns = b == b_found ? (L - first + kSlice - 1) / kSlice : seq_slices(a, b, first, L);
    const int64_t span = static_cast<int64_t>(a.Hkv) * ns;
    if (pos >= seq0 + span) {
      seq0 += span;
      ++b;
      continue;
    }
    const int64_t r = pos - seq0;
    const int h = static_cast<int>(r / ns);
    const int j0 = static_cast<int>(r - static_cast<int64_t>(h) * ns);
    const int j1 = static_cast<int>(min<int64_t>(ns, s_end - seq0 - static_cast<int64_t>(h) * ns));
    pos = seq0 + static_cast<int64_t>(h) * ns + j1;
    const int sigma = b * a.Hkv + h;
    // the thread index, opaque to the optimizer per part: values derived from
    // it are computed where they are used instead of being kept in registers
    // across all parts
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int col = lane & 15, kg = lane >> 4;
    uint16_t *pp = reinterpret_cast<uint16_t *>(prow_s[w]);
    uint4 *vb = vbuf_s[w];

    __syncthreads();  // the previous part's readers of the tables and of red are done
    if (tid == 0) {
      if (j0 == 0) tab_first[sigma] = wg;
      if (j1 == ns) tab_last[sigma] = wg;
    }
    // the codes of segment (b, h) through buffer resources (base and size in
    // scalar registers, 32-bit offsets per lane)
    const int64_t row0 = (static_cast<int64_t>(b) * a.Hkv + h) * a.S;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.k_codes + row0 * NSK), 0, a.S * NSK, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.v_codes + row0 * NSV), 0, a.S * NSV, kBufferWord3);
    // key codes of slice j into kw (lane: quarter kg of token 16 G + col);
    // clamped token indices
    auto load_keys = [&](int j, uint32_t(&kw)[4][NQW]) {
      const int t0 = first + j * kSlice;
#pragma unroll
      for (int G4 = 0; G4 < 4; ++G4) {
        const int off = min(t0 + 16 * G4 + col, L - 1) * NSK + kg * QB;
        if constexpr (NQW == 4) {
          const auto q = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
          kw[G4][0] = q[0];
          kw[G4][1] = q[1];
          kw[G4][2] = q[2];
          kw[G4][3] = q[3];
        } else if constexpr (NQW == 2) {
          const auto q = __builtin_amdgcn_raw_buffer_load_b64(rk, off, 0, 0);
          kw[G4][0] = q[0];
          kw[G4][1] = q[1];
        } else {
          kw[G4][0] = __builtin_amdgcn_raw_buffer_load_b32(rk, off, 0, 0);
        }
      }
    };
    // value codes of slice j into the wave's buffer (slot e = 64 q + lane:
    // token e / VP, piece (e % VP) ^ ((token / 2) mod VP), so that the rows of
    // tokens 2 apart, read together by the value sum, start on different
    // banks); clamped token indices
    auto copy_values = [&](int j) {
      const int t0 = first + j * kSlice;
      wait_lgkm_all();  // earlier reads of the buffer have completed
#pragma unroll
      for (int q = 0; q < VP; ++q) {
        const int e = 64 * q + lane;
        const int tc = e / VP, pc = e % VP;
        const int off = min(t0 + tc, L - 1) * NSV + 16 * (pc ^ ((tc >> 1) & (VP - 1)));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (__attribute__((address_space(3))) void *)(vb + 64 * q), 16, off, 0, 0, 0);
      }
    };
    // Every step issues the same memory operations in the same order (the
    // key codes of the next slice after the scores, its value codes after the
    // value sum; past the wave's last slice the loads repeat that slice), so
    // the waits the compiler places count only what each use needs.
    // ---- codebooks of kv head h, query parts of its g heads: their loads
    // go out before the first slice's codes (they are few and cached) ------
    const int n_c = a.n_c;
    uint16_t kvr[SDK], vvr[SDV];
    {
      const uint16_t *kcb = a.k_cb + static_cast<int64_t>(h) * n_c * SDK;
      const uint16_t *vcb = a.v_cb + static_cast<int64_t>(h) * n_c * SDV;
#pragma unroll
      for (int k = 0; k < SDK; ++k) kvr[k] = kcb[min(tid + kThreads * k, n_c * SDK - 1)];
#pragma unroll
      for (int k = 0; k < SDV; ++k) vvr[k] = vcb[min(tid + kThreads * k, n_c * SDV - 1)];
    }
    constexpr int JH = GC > 4 ? 2 : 1;
    uint16_t qv[JH][D / 64];
    float ks[D / 64];
#pragma unroll
    for (int jh = 0; jh < JH; ++jh) {
      const int hq = h * g + min(w + 4 * jh, g - 1);
      const uint16_t *qrow = a.q + (static_cast<int64_t>(b) * a.Hq + hq) * D;
#pragma unroll
      for (int k = 0; k < D / 64; ++k) qv[jh][k] = qrow[lane + 64 * k];
    }
#pragma unroll
    for (int k = 0; k < D / 64; ++k)
      ks[k] = a.k_scale ? a.k_scale[static_cast<int64_t>(h) * D + lane + 64 * k] : 1.0f;
    __builtin_amdgcn_sched_barrier(0);
    uint32_t kw[4][NQW];
    int j = j0 + w;
    if (j < j1) {
      load_keys(j, kw);
      copy_values(j);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < SDK; ++k) {
      const int e = tid + kThreads * k;
      ktab[e] = (e < n_c * SDK) ? kvr[k] : static_cast<uint16_t>(0);
    }
#pragma unroll
    for (int k = 0; k < SDV; ++k) {
      const int e = tid + kThreads * k;
      vtab[e] = (e < n_c * SDV) ? vvr[k] : static_cast<uint16_t>(0);
    }
#pragma unroll
    for (int jh = 0; jh < JH; ++jh) {
      const int hs = w + 4 * jh;
      if (hs < g) {  // uniform per wave
        uint16_t *rows = qp + static_cast<int64_t>(hs) * P * QS;
        float x[D / 64];
        float mx = 0.0f;
#pragma unroll
        for (int k = 0; k < D / 64; ++k) {
          float v = widen<BF16>(qv[jh][k]);
          if (a.k_scale) v = v / ks[k];
          v = v * a.qmul;
          x[k] = v;
          mx = fmaxf(mx, __builtin_fabsf(v));
        }
        mx = row_max16(mx);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        int E = 0;
        if (mx > 0.0f && mx <= 3.4028234663852886e38f) {
          int ex;
          (void)frexpf(mx, &ex);  // mx = f 2^ex, f in [0.5, 1)
          E = 14 - ex;            // max |q~| 2^E in [2^13, 2^14)
        }
        if (lane == 0) qexp[hs] = E;
#pragma unroll
        for (int k = 0; k < D / 64; ++k) {
          const int d = lane + 64 * k;
          float rr = ldexpf(x[k], E);
#pragma unroll
          for (int q = 0; q < P; ++q) {  // rr - part is exact in fp32
            const uint16_t pb = narrow_rn<BF16>(rr);
            rows[q * QS + d] = pb;
            rr = rr - widen<BF16>(pb);
          }
        }
      }
    }
    __syncthreads();

    // A operand of the scores: row col of the query parts (the zero row past
    // g P), quarter kg
    uint4 areg[NI];
    {
      const uint16_t *arow = qp + (col < nrows ? col : ZR) * QS + kg * (D / 4);
#pragma unroll
      for (int i = 0; i < NI; ++i) areg[i] = *reinterpret_cast<const uint4 *>(arow + 8 * i);
    }
    int ex[HPL];
#pragma unroll
    for (int jj = 0; jj < HPL; ++jj) ex[jj] = qexp[min(kg * HPL + jj, g - 1)];
    float m_run[HPL], l_run[HPL];
#pragma unroll
    for (int jj = 0; jj < HPL; ++jj) {
      m_run[jj] = kNegInf;
      l_run[jj] = 0.0f;
    }
    // Value sum, rows (head, part, element): in block rb lane (col, kg) holds
    // rows 16 rb + 4 kg .. + 3 = elements 0..3 of weight row 4 rb + kg, for
    // sub-space 16 cg + col.  Its A operand is row 16 rb + col, i.e. weight row
    // (16 rb + col) / 4 placed at element e = col % 4 of its two tokens: word
    // e / 2 (first token) and 2 + e / 2 (second), half e % 2 (selectors).
    f32x4 vacc[NCG][NRB];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) vacc[cg][rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int ea = col & 3;
    const uint32_t zsel = 0x0C0C0C0Cu;
    const uint32_t lo_sel = (ea & 1) ? 0x01000C0Cu : 0x0C0C0100u;  // first token's half
    const uint32_t hi_sel = (ea & 1) ? 0x03020C0Cu : 0x0C0C0302u;  // second token's half
    const uint32_t sel0 = (ea >> 1) == 0 ? lo_sel : zsel, sel1 = (ea >> 1) == 1 ? lo_sel : zsel;
    const uint32_t sel2 = (ea >> 1) == 0 ? hi_sel : zsel, sel3 = (ea >> 1) == 1 ? hi_sel : zsel;
    int prow_off[NRB];  // the weight row of A row 16 rb + col (the zero row past g P)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int hp = (16 * rb + col) >> 2;
      prow_off[rb] = (hp < nrows ? hp : ZR) * PS + 2 * kg;
    }
    const uint8_t *codes = reinterpret_cast<const uint8_t *>(vb) + 2 * kg * NSV + col;
    const int swz = kg & (VP - 1);

    const uint2 *ktab2 = reinterpret_cast<const uint2 *>(ktab_s);
    const uint4 *ktab4 = reinterpret_cast<const uint4 *>(ktab_s);
    const uint2 *vtab2 = reinterpret_cast<const uint2 *>(vtab_s);
    // one 64-token slice: scores, running softmax, value sum
    auto slice = [&](int js) {
      const int t0 = first + js * kSlice;
      float sreg[4][HPL];
#pragma unroll
      for (int G4 = 0; G4 < 4; ++G4) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          uint4 bop;
          if constexpr (SDK == 4) {
            const uint32_t wd = kw[G4][i >> 1];
            const uint32_t c0 = (wd >> (16 * (i & 1))) & 0xFFu;
            const uint32_t c1 = (wd >> (16 * (i & 1) + 8)) & 0xFFu;
            const uint2 r0 = ktab2[c0], r1 = ktab2[c1];
            bop = make_uint4(r0.x, r0.y, r1.x, r1.y);
          } else {
            const uint32_t c = (kw[G4][i >> 2] >> (8 * (i & 3))) & 0xFFu;
            bop = ktab4[c];
          }
          acc = mfma16<BF16>(areg[i], bop, acc);
        }
        __builtin_amdgcn_sched_barrier(0);  // one 16-token group's gathers live at a time
        const bool valid = t0 + 16 * G4 + col < L;
        if constexpr (P == 2) {
          sreg[G4][0] = valid ? ldexpf(acc[0] + acc[1], -ex[0]) : kNegInf;
          sreg[G4][1] = valid ? ldexpf(acc[2] + acc[3], -ex[1]) : kNegInf;
        } else {
          sreg[G4][0] = valid ? ldexpf(((acc[3] + acc[2]) + acc[1]) + acc[0], -ex[0]) : kNegInf;
        }
      }
      // the key codes are consumed: the next slice's go into the same registers
      load_keys(min(js + 4, j1 - 1), kw);
      __builtin_amdgcn_sched_barrier(0);
      // This slice's value codes (the copy issued one step earlier, before
      // those 4 key loads) must have landed in LDS before the value sum reads
      // them; the compiler does not track the copy's LDS writes, so the wait
      // is explicit: at most the 4 key loads may still be in flight.
      wait_vm_keys();
      __builtin_amdgcn_sched_barrier(0);
      // running maximum per head; rescale the sums when it rises
      float alpha[HPL];
      bool grow = false;
#pragma unroll
      for (int jj = 0; jj < HPL; ++jj) {
        float m = fmaxf(fmaxf(sreg[0][jj], sreg[1][jj]), fmaxf(sreg[2][jj], sreg[3][jj]));
        m = row_max16(m);
        const float mn = fmaxf(m_run[jj], m);
        alpha[jj] = (mn == m_run[jj]) ? 1.0f : exp2f(m_run[jj] - mn);
        grow = grow || mn != m_run[jj];
        m_run[jj] = mn;
      }
      if (__builtin_amdgcn_ballot_w64(grow)) {  // uniform
#pragma unroll
        for (int jj = 0; jj < HPL; ++jj) {
          l_run[jj] *= alpha[jj];
          if (col == 0 && kg * HPL + jj < GC) walpha[w][kg * HPL + jj] = alpha[jj];
        }
        // value rows of block rb: weight row 4 rb + kg, head (4 rb + kg) / P
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const float f = walpha[w][min((4 * rb + kg) / P, GC - 1)];
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) vacc[cg][rb][rr] *= f;
        }
      }
      // weights p 2^14, split, as rows (head, part) x 64 tokens
#pragma unroll
      for (int jj = 0; jj < HPL; ++jj) {
        const int hh = kg * HPL + jj;
        float lsum = 0.0f;
#pragma unroll
        for (int G4 = 0; G4 < 4; ++G4) {
          const float sv = sreg[G4][jj];
          // v_exp_f32 directly (results below 2^-126 flush to 0, far below
          // the split's resolution of 2^-38)
          const float pv = (sv == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(sv - m_run[jj]);
          lsum += pv;
          if (hh < g) {
            float rr = pv * kPScale;
#pragma unroll
            for (int q = 0; q < P; ++q) {
              const uint16_t pb = narrow_rn<BF16>(rr);
              pp[(hh * P + q) * PS + 16 * G4 + col] = pb;
              rr = rr - widen<BF16>(pb);
            }
          }
        }
        l_run[jj] += row_sum16(lsum);
      }
      // value sum over 8-token groups: lane (col, kg) gathers the rows of
      // sub-space 16 cg + col for tokens 8 k8 + 2 kg, + 1 (one B operand,
      // elements in order); the A operand places the weights by element
#pragma unroll
      for (int k8 = 0; k8 < kSlice / 8; ++k8) {
        uint4 aop[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const uint32_t pv = *reinterpret_cast<const uint32_t *>(pp + prow_off[rb] + 8 * k8);
          aop[rb] = make_uint4(__builtin_amdgcn_perm(0u, pv, sel0), __builtin_amdgcn_perm(0u, pv, sel1),
                               __builtin_amdgcn_perm(0u, pv, sel2), __builtin_amdgcn_perm(0u, pv, sel3));
        }
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg) {
          const uint8_t *cc = codes + 8 * k8 * NSV + ((cg ^ swz) << 4);
          const uint2 r0 = vtab2[cc[0]], r1 = vtab2[cc[NSV]];
          const uint4 bop = make_uint4(r0.x, r0.y, r1.x, r1.y);
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) vacc[cg][rb] = mfma16<BF16>(aop[rb], bop, vacc[cg][rb]);
        }
      }
      // the value codes are consumed: the next slice's go into the buffer
      copy_values(min(js + 4, j1 - 1));
    };

    while (j < j1) {  // uniform per wave
      slice(j);
      j += 4;
    }
    wait_vm_all();  // the repeated loads past the last slice have landed

    // ---- merge the waves, write the part's partial -------------------------
    if (col == 0) {
#pragma unroll
      for (int jj = 0; jj < HPL; ++jj) {
        const int hh = kg * HPL + jj;
        if (hh < g) {
          wm[w][hh] = m_run[jj];
          wl[w][hh] = l_run[jj];
        }
      }
    }
    __syncthreads();
    // o of weight row 4 rb + kg (head (4 rb + kg) / P), elements 0..3 of
    // sub-space 16 cg + col: scaled to the part's maximum, parts summed across
    // the lanes that hold them (kg differs in its low log2(P) bits)
    float o[NRB][NCG][4];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int hc = min((4 * rb + kg) / P, g - 1);
      const float M = fmaxf(fmaxf(wm[0][hc], wm[1][hc]), fmaxf(wm[2][hc], wm[3][hc]));
      const float mine_m = wm[w][hc];
      const float f = (mine_m == kNegInf) ? 0.0f : exp2f(mine_m - M) * (1.0f / kPScale);
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = vacc[cg][rb][e];
          v = v + __shfl_xor(v, 16);
          if constexpr (P == 4) v = v + __shfl_xor(v, 32);
          o[rb][cg][e] = v * f;
        }
    }
    // lanes holding part 0 of a head in range write it
    const bool owner = (kg & (P - 1)) == 0;
    if (w > 0 && owner) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int hh = (4 * rb + kg) / P;
        if (hh < g) {
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              red[((w - 1) * GC + hh) * D + (cg * 16 + col) * 4 + e] = o[rb][cg][e];
        }
      }
    }
    __syncthreads();
    float *slot = a.ws + static_cast<int64_t>(wg + sigma) * g * (D + 2);
    if (w == 0 && owner) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int hh = (4 * rb + kg) / P;
        if (hh < g) {
          float *dst = slot + hh * (D + 2);
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg) {
            const int d0 = (cg * 16 + col) * 4;
            float s4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              s4[e] = ((o[rb][cg][e] + red[hh * D + d0 + e]) + red[(GC + hh) * D + d0 + e]) +
                      red[(2 * GC + hh) * D + d0 + e];
            *reinterpret_cast<float4 *>(dst + d0) = make_float4(s4[0], s4[1], s4[2], s4[3]);
          }
        }
      }
    }
    if (tid < g) {
      const float M = fmaxf(fmaxf(wm[0][tid], wm[1][tid]), fmaxf(wm[2][tid], wm[3][tid]));
      float l = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) l += wm[v][tid] == kNegInf ? 0.0f : wl[v][tid] * exp2f(wm[v][tid] - M);
      slot[tid * (D + 2) + D] = M;
      slot[tid * (D + 2) + D + 1] = l;
    }
  }
}

// Merge of the streaming form: the partials of (sequence, query head)
// blockIdx.x sit in slots i + sigma for the workgroups i from the first to
// the last one recorded for its segment sigma; a sequence with no attended
// token gets zeros.
__global__ void __launch_bounds__(kThreads)
attn_stream_combine(const AttnArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, hq = bh - b * a.Hq;
  const int g = a.Hq / a.Hkv, h = hq / g, jh = hq - h * g;
  float *out = a.out + static_cast<int64_t>(bh) * a.D;
  int first, L;
  if (seq_slices(a, b, first, L) == 0) {
    if (threadIdx.x < a.D) out[threadIdx.x] = 0.0f;
    return;
  }
  const int G = a.n_wg;
  const int sigma = b * a.Hkv + h;
  const int *tab_first = reinterpret_cast<const int *>(
      a.ws + static_cast<int64_t>(G + a.B * a.Hkv - 1) * g * (a.D + 2));
  // (clamped: the indices are always in range when the partial launch ran)
  const int i0 = min(max(tab_first[sigma], 0), G - 1);
  const int i1 = min(max(tab_first[a.B * a.Hkv + sigma], i0), G - 1);
  const int64_t cstride = static_cast<int64_t>(g) * (a.D + 2);
  merge_partials(a.ws + (static_cast<int64_t>(i0 + sigma) * g + jh) * (a.D + 2), i1 - i0 + 1,
                 cstride, a.D, out);
}

template <int SDK, int SDV, bool BF16>
hipError_t launch_attn_t(AttnArgs a, hipStream_t stream) {
  const int g = a.Hq / a.Hkv;
  const size_t lds = attn_lds_bytes<SDK, SDV>(a.D, g);
  auto kern = attn_partial<SDK, SDV, BF16>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  a.n_chunks = std::max(1, static_cast<int>((static_cast<int64_t>(a.S) + kChunk - 1) / kChunk));
  hipLaunchKernelGGL(kern, dim3(a.n_chunks, a.Hkv, a.B), dim3(kThreads), lds, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine, dim3(a.B * a.Hq), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// The matrix-core form takes head_dim 64, 128 or 256 with 16 or more codes
// per key and per value row.
constexpr bool mfma_shape(int sdk, int sdv, int d) {
  return (d == 64 || d == 128 || d == 256) && (d / sdk) % 16 == 0 && (d / sdv) % 16 == 0;
}

// Workgroups of the streaming form for this call: per_cu per CU, few enough
// that the partials (slots up to G + B Hkv - 1) and the segment table fit in
// the workspace the chunked form is sized for (attention_chunks(S) partials
// per sequence and query head).  0 = the chunked form runs instead: the
// streaming form pays a longer fixed latency per workgroup (length scan,
// staging, merge in sequence), which only a long enough range of slices per
// workgroup amortizes; below kStreamMinSlices slices per workgroup (counted
// on max_kv_len, the lengths being on the device) the chunked form is the
// faster one.
constexpr int64_t kStreamMinSlices = 32;
int stream_workgroups(const AttnArgs &a, int per_cu) {
  const int g = a.Hq / a.Hkv;
  const int64_t segs = static_cast<int64_t>(a.B) * a.Hkv;
  const int64_t row = static_cast<int64_t>(g) * (a.D + 2);  // floats per slot
  const int64_t avail = static_cast<int64_t>(a.B) * a.Hq * attention_chunks(a.S) * (a.D + 2);
  const int64_t gmax = (avail - 2 * segs) / row - segs + 1;
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  const int64_t G = static_cast<int64_t>(per_cu) * cus;
  const int64_t slices = segs * ((static_cast<int64_t>(a.S) + kSlice - 1) / kSlice);
  if (slices < kStreamMinSlices * G || G > gmax) return 0;
  // a segment's codes are addressed with 32-bit offsets (buffer resources)
  const int64_t row_bytes = a.D / 4;  // the most code bytes per token (sub_dim 4)
  if (static_cast<int64_t>(a.S) * row_bytes >= (int64_t{1} << 31)) return 0;
  return static_cast<int>(G);
}

template <int SDK, int SDV, bool BF16, int D>
hipError_t launch_attn_m(AttnArgs a, hipStream_t stream) {
  if constexpr (!mfma_shape(SDK, SDV, D)) {
    return hipErrorInvalidValue;
  } else {
    const int g = a.Hq / a.Hkv;
    // the streaming form (value sub-dim 4) holds one block of query rows:
    // g P <= 16
    if constexpr (SDV == 4) {
      const bool small = BF16 || g <= 4;
      constexpr int GC8 = BF16 ? 4 : kMaxGroup;
      a.n_wg = (g * (BF16 ? 4 : 2) <= 16)
                   ? stream_workgroups(a, small ? kStreamPerCu<BF16, D, 4> : kStreamPerCu<BF16, D, GC8>)
                   : 0;
      if (a.n_wg > 0) {
        auto kern = small ? attn_stream_partial<SDK, SDV, BF16, D, 4>
                          : attn_stream_partial<SDK, SDV, BF16, D, GC8>;
        hipLaunchKernelGGL(kern, dim3(a.n_wg), dim3(kThreads), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_stream_combine, dim3(a.B * a.Hq), dim3(kThreads), 0, stream, a);
        return hipGetLastError();
      }
    }
    auto kern = g <= 4 ? attn_mfma_partial<SDK, SDV, BF16, D, 4>
                       : attn_mfma_partial<SDK, SDV, BF16, D, kMaxGroup>;
    a.n_chunks = attention_chunks(a.S);
    hipLaunchKernelGGL(kern, dim3(a.n_chunks, a.Hkv, a.B), dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_combine, dim3(a.B * a.Hq), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
  }
}

template <int SDK, int SDV, bool BF16>
hipError_t launch_attn_d(const AttnArgs &a, bool mfma, hipStream_t stream) {
  if (mfma) {
    if (a.D == 256) return launch_attn_m<SDK, SDV, BF16, 256>(a, stream);
    if (a.D == 128) return launch_attn_m<SDK, SDV, BF16, 128>(a, stream);
    return launch_attn_m<SDK, SDV, BF16, 64>(a, stream);
  }
  return launch_attn_t<SDK, SDV, BF16>(a, stream);
}

template <bool BF16>
hipError_t launch_attn_dt(const AttnArgs &a, int sdk, int sdv, bool mfma, hipStream_t stream) {
  if (sdk == 4) {
    return sdv == 4 ? launch_attn_d<4, 4, BF16>(a, mfma, stream)
                    : launch_attn_d<4, 8, BF16>(a, mfma, stream);
  }
  return sdv == 4 ? launch_attn_d<8, 4, BF16>(a, mfma, stream)
                  : launch_attn_d<8, 8, BF16>(a, mfma, stream);
}

}  // namespace

// Chunk partials of vq_attention_decode_static, for callers that cannot
// allocate: one copy per GPU (the code object's device data), held until the
// process ends.  In host code `scratch` names a host-side stand-in, not device
// memory: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) uint8_t scratch[VQ_ATTN_STATIC_SCRATCH_BYTES];

hipError_t attention_static_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void *> addr[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

int attention_chunks(int max_kv_len) {
  // 64-bit: max_kv_len may be close to INT32_MAX
  return std::max(1, static_cast<int>((static_cast<int64_t>(max_kv_len) + kMChunk - 1) / kMChunk));
}

size_t attention_lds_bytes(int sdk, int sdv, int D, int g) {
  if (sdk == 4) return sdv == 4 ? attn_lds_bytes<4, 4>(D, g) : attn_lds_bytes<4, 8>(D, g);
  return sdv == 4 ? attn_lds_bytes<8, 4>(D, g) : attn_lds_bytes<8, 8>(D, g);
}

hipError_t launch_attention(const AttnLayout &l, hipStream_t stream) {
  AttnArgs a;
  a.q = static_cast<const uint16_t *>(l.q);
  a.k_codes = l.k_codes;
  a.v_codes = l.v_codes;
  a.k_cb = static_cast<const uint16_t *>(l.k_codebook);
  a.v_cb = static_cast<const uint16_t *>(l.v_codebook);
  a.k_scale = l.k_scale;
  a.kv_len = l.kv_len;
  a.ws = l.workspace;
  a.out = l.out;
  a.B = l.batch;
  a.Hq = l.n_q_heads;
  a.Hkv = l.n_kv_heads;
  a.D = l.head_dim;
  a.S = l.max_kv_len;
  a.n_c = l.n_centroids;
  a.window = l.window;
  a.n_chunks = 0;
  a.n_wg = 0;
  a.qmul = l.softmax_scale * 1.4426950408889634f;
  const bool mfma = mfma_shape(l.k_sub_dim, l.v_sub_dim, l.head_dim) &&
                    reinterpret_cast<uintptr_t>(l.k_codes) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(l.v_codes) % 16 == 0;
  return l.bf16 ? launch_attn_dt<true>(a, l.k_sub_dim, l.v_sub_dim, mfma, stream)
                : launch_attn_dt<false>(a, l.k_sub_dim, l.v_sub_dim, mfma, stream);
}

}  // namespace vqk
