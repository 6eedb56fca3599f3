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
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

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

  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
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

// Merge the chunk partials of one (sequence, query head): thread d.
__global__ void __launch_bounds__(kThreads)
attn_combine(const AttnArgs a) {
  const int bh = blockIdx.x;
  const int D = a.D;
  const int64_t part_stride = D + 2;
  const float *part = a.ws + static_cast<int64_t>(bh) * a.n_chunks * part_stride;
  float M = kNegInf;
  for (int c = 0; c < a.n_chunks; ++c) M = fmaxf(M, part[c * part_stride + D]);
  for (int d = threadIdx.x; d < D; d += kThreads) {
    float o = 0.0f;
    if (M != kNegInf) {
      float l = 0.0f, acc = 0.0f;
      for (int c = 0; c < a.n_chunks; ++c) {
        const float mc = part[c * part_stride + D];
        if (mc == kNegInf) continue;
        const float w = exp2f(mc - M);
        l = __builtin_fmaf(part[c * part_stride + D + 1], w, l);
        acc = __builtin_fmaf(part[c * part_stride + d], w, acc);
      }
      o = acc / l;
    }
    a.out[static_cast<int64_t>(bh) * D + d] = o;
  }
}

template <int SDK, int SDV, bool BF16>
hipError_t launch_attn_t(const AttnArgs &a, hipStream_t stream) {
  const int g = a.Hq / a.Hkv;
  const size_t lds = attn_lds_bytes<SDK, SDV>(a.D, g);
  auto kern = attn_partial<SDK, SDV, BF16>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(a.n_chunks, a.Hkv, a.B), dim3(kThreads), lds, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine, dim3(a.B * a.Hq), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_attn_dt(const AttnArgs &a, int sdk, int sdv, hipStream_t stream) {
  if (sdk == 4) {
    return sdv == 4 ? launch_attn_t<4, 4, BF16>(a, stream) : launch_attn_t<4, 8, BF16>(a, stream);
  }
  return sdv == 4 ? launch_attn_t<8, 4, BF16>(a, stream) : launch_attn_t<8, 8, BF16>(a, stream);
}

}  // namespace

int attention_chunks(int max_kv_len) { return std::max(1, (max_kv_len + kChunk - 1) / kChunk); }

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
  a.n_chunks = attention_chunks(l.max_kv_len);
  a.qmul = l.softmax_scale * 1.4426950408889634f;
  return l.bf16 ? launch_attn_dt<true>(a, l.k_sub_dim, l.v_sub_dim, stream)
                : launch_attn_dt<false>(a, l.k_sub_dim, l.v_sub_dim, stream);
}

}  // namespace vqk
