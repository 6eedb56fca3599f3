// Device helpers shared by the encode kernels: per-channel smoothing factors
// and the packed code stream.
//
// Code stream (VeloxQuant-MLX blog, "How I built VeloxQuant-MLX -- KV cache
// compression for LLMs running on your Mac", section "The Bit-Packing
// Problem"): b-bit codes back to back, least significant bit first; code r
// occupies stream bits r*b .. r*b + b - 1, stream bit k is bit (k mod 8) of
// byte k / 8.  With b = 8 this is one byte per code, the 16x (sub_dim 8) or
// 8x (sub_dim 4) key compression of "I Wrote a Metal Kernel to Stop My Mac
// From OOMing", section "What Even Is a KV Cache And Why Should You Care".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vqk {

// v mod d for 0 <= v < 2^20 and 1 <= d <= 4096, with inv_d = fp32(1/d): the
// float quotient is off by at most one either way, which the two fix-ups
// undo.
__device__ __forceinline__ int mod_small(int v, int d, float inv_d) {
  const int q = static_cast<int>(static_cast<float>(v) * inv_d);
  int r = v - q * d;
  r += (r < 0) ? d : 0;
  r -= (r >= d) ? d : 0;
  return r;
}

// Code widths written with one plain store per sub-vector.
__device__ __forceinline__ bool byte_width(int bits) {
  return bits == 8 || bits == 16 || bits == 32;
}

// Code of row `row` for a byte-multiple width (8, 16 or 32 bits).
__device__ __forceinline__ void store_code_bytes(uint8_t *__restrict__ out, int64_t row,
                                                 uint32_t code, int bits) {
  if (bits == 32) {
    reinterpret_cast<uint32_t *>(out)[row] = code;
  } else if (bits == 16) {
    reinterpret_cast<uint16_t *>(out)[row] = static_cast<uint16_t>(code);
  } else {
    out[row] = static_cast<uint8_t>(code);
  }
}

// Writes the codes of the 32 consecutive rows [row0, row0 + 32) held by the
// 32 lanes of one half of a wave (lane j of the half holds row row0 + j) into
// the stream at `out`.  Rows >= rend are not written (their code bits are
// zero in a partly covered word).  row0 * bits must be a multiple of 32, and
// a 32-bit word of the stream is shared with rows beyond rend only at the
// very end of the stream, where it is written byte by byte so that no byte
// past ceil(rend * bits / 8) is touched.  Only the half with store_half set
// writes.  Every lane of the wave must call this with the same bits (it
// exchanges codes across lanes).
__device__ __forceinline__ void store_codes32(uint32_t code, int64_t row0, int64_t rend, int bits,
                                              bool store_half, uint8_t *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 31;
  const int64_t left = rend - row0;
  const int nv = left <= 0 ? 0 : (left >= 32 ? 32 : static_cast<int>(left));
  if (byte_width(bits)) {
    if (store_half && j < nv)
      store_code_bytes(out, row0 + j, bits == 32 ? code : (code & ((1u << bits) - 1u)), bits);
    return;
  }
  const uint32_t mine = (j < nv) ? (code & ((1u << bits) - 1u)) : 0u;
  // lane k < bits assembles word k = stream bits [32k, 32k + 32) of these 32
  // codes: the codes first .. first + ceil(32 / bits) overlap it
  const int k = j;
  const int first = (32 * k) / bits;
  const int trips = (32 + bits - 1) / bits + 1;
  uint32_t word = 0;
  for (int s = 0; s < trips; ++s) {
    const int jj = first + s;
    const uint32_t cj = static_cast<uint32_t>(__shfl(static_cast<int>(mine), (lane & 32) + min(jj, 31)));
    const int off = jj * bits - 32 * k;  // > -bits
    if (jj < 32 && off < 32) word |= (off >= 0) ? (cj << off) : (cj >> (-off));
  }
  if (store_half && k < bits) {
    const int valid = nv * bits - 32 * k;  // bits of this word that belong to rows < rend
    if (valid >= 32) {
      reinterpret_cast<uint32_t *>(out)[((row0 * bits) >> 5) + k] = word;
    } else if (valid > 0) {
      uint8_t *p = out + ((row0 * bits) >> 3) + 4 * k;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (8 * q < valid) p[q] = static_cast<uint8_t>(word >> (8 * q));
    }
  }
}

}  // namespace vqk
