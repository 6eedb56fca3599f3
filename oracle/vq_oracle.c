/*
 * vq_oracle.c -- plain CPU oracle for the product-VQ encode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; only tests, the smoke check
 * and the CPU-baseline leg of the benchmark do.  It shares no code, header,
 * table or helper with the HIP library.
 *
 * What it computes (VeloxQuant-MLX blog, "I Wrote a Metal Kernel to Stop My
 * Mac From OOMing"):
 *   - section "What Even Is a KV Cache And Why Should You Care", steps 1-3:
 *     each key is cut into sub-vectors of length sub_dim and every sub-vector
 *     is replaced by the index of its nearest codebook centroid;
 *   - section "What quantize_vq Was Doing Wrong": nearest means the argmin
 *     over centroids of the summed squared component differences;
 *   - section "The Kernel: 18 Lines of MSL": components are promoted to fp32
 *     before the difference, the squared difference is accumulated in one
 *     fp32 register, the running best starts at +infinity with index 0, a
 *     centroid replaces the best only when its distance is strictly smaller
 *     (so ties keep the lowest index), and one uint32 index is written per
 *     sub-vector.
 *
 * Readings taken where the page is silent (each is listed in the design
 * notes of the repository):
 *   - the accumulation "dist += d*d" is evaluated as one fused multiply-add
 *     per component (fmaf, a single rounding), components summed in order
 *     i = 0 .. sub_dim-1, starting from +0;
 *   - fp16 and bf16 inputs widen to fp32 exactly; IEEE subnormals are kept;
 *   - a NaN distance never wins (the strict comparison is false), and a
 *     sub-vector with no distance below +infinity gets index 0;
 *   - batched caches: sub-vector n belongs to group n / group_len and uses
 *     codebook slot group_map[g] (or g when no map is given).  A slot outside
 *     [0, n_codebooks) yields the sentinel index 0xFFFFFFFF.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC, so that the
 * only fused operation is the explicit fmaf and every other operation is one
 * IEEE binary32 operation rounded to nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define VQO_F16 0
#define VQO_BF16 1
#define VQO_BAD_SLOT 0xFFFFFFFFu

/* IEEE 754 binary16 -> binary32, written out from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static float f16_bits_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    float mag;
    if (expo == 0) {
        mag = ldexpf((float)frac, -24);            /* subnormal: frac * 2^-24 */
    } else if (expo == 31) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexpf((float)(1024 + frac), expo - 25); /* (1.frac) * 2^(e-15) */
    }
    return sign ? -mag : mag;
}

/* bfloat16 is the upper half of a binary32 word. */
static float bf16_bits_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float widen(uint16_t v, int dtype)
{
    return dtype == VQO_BF16 ? bf16_bits_to_f32(v) : f16_bits_to_f32(v);
}

float vqo_to_f32(uint16_t v, int dtype) { return widen(v, dtype); }

/* Squared L2 distance of one sub-vector to one centroid, in the fixed fp32
 * arithmetic described above. */
float vqo_sqdist(const uint16_t *xrow, const uint16_t *crow, int sub_dim, int dtype)
{
    float dist = 0.0f;
    for (int i = 0; i < sub_dim; ++i) {
        float d = widen(xrow[i], dtype) - widen(crow[i], dtype);
        dist = fmaf(d, d, dist);
    }
    return dist;
}

static int slot_of(int64_t n, int64_t group_len, const int32_t *group_map,
                   int64_t n_codebooks, int64_t *slot)
{
    int64_t g = n / group_len;
    int64_t s = group_map ? (int64_t)group_map[g] : g;
    if (s < 0 || s >= n_codebooks) return 0;
    *slot = s;
    return 1;
}

static int args_ok(int64_t n, int sub_dim, int n_centroids, int dtype,
                   int64_t n_codebooks, int64_t group_len)
{
    return n >= 0 && sub_dim >= 1 && n_centroids >= 1 &&
           (dtype == VQO_F16 || dtype == VQO_BF16) && n_codebooks >= 1 &&
           group_len >= 1;
}

/*
 * Encode n sub-vectors.  x: [n][sub_dim] fp16/bf16 bits.  codebook slot s
 * starts at codebook + s*codebook_stride and holds [n_centroids][sub_dim].
 * out: [n] uint32.  Returns 0 on success, -1 on a bad argument.
 */
int vqo_encode(const uint16_t *x, const uint16_t *codebook, int64_t n, int sub_dim,
               int n_centroids, int dtype, int64_t codebook_stride, int64_t n_codebooks,
               int64_t group_len, const int32_t *group_map, uint32_t *out)
{
    if (!args_ok(n, sub_dim, n_centroids, dtype, n_codebooks, group_len)) return -1;
    for (int64_t r = 0; r < n; ++r) {
        int64_t slot;
        if (!slot_of(r, group_len, group_map, n_codebooks, &slot)) {
            out[r] = VQO_BAD_SLOT;
            continue;
        }
        const uint16_t *cb = codebook + slot * codebook_stride;
        const uint16_t *xr = x + r * sub_dim;
        float best = INFINITY;
        uint32_t best_idx = 0;
        for (int c = 0; c < n_centroids; ++c) {
            float dist = vqo_sqdist(xr, cb + (int64_t)c * sub_dim, sub_dim, dtype);
            if (dist < best) {
                best = dist;
                best_idx = (uint32_t)c;
            }
        }
        out[r] = best_idx;
    }
    return 0;
}

/*
 * Same search, also reporting the winning distance and the second-best
 * distance, i.e. the minimum over every centroid other than the winner (it
 * equals the best when an exact duplicate of the winner exists).  With one
 * centroid the second-best is +infinity.  These two numbers are what the
 * near-tie acceptance rule of the GPU comparison needs.
 */
int vqo_encode_top2(const uint16_t *x, const uint16_t *codebook, int64_t n, int sub_dim,
                    int n_centroids, int dtype, int64_t codebook_stride, int64_t n_codebooks,
                    int64_t group_len, const int32_t *group_map, uint32_t *out,
                    float *best_out, float *second_out)
{
    if (!args_ok(n, sub_dim, n_centroids, dtype, n_codebooks, group_len)) return -1;
    for (int64_t r = 0; r < n; ++r) {
        int64_t slot;
        if (!slot_of(r, group_len, group_map, n_codebooks, &slot)) {
            out[r] = VQO_BAD_SLOT;
            best_out[r] = NAN;
            second_out[r] = NAN;
            continue;
        }
        const uint16_t *cb = codebook + slot * codebook_stride;
        const uint16_t *xr = x + r * sub_dim;
        float best = INFINITY;
        uint32_t best_idx = 0;
        for (int c = 0; c < n_centroids; ++c) {
            float dist = vqo_sqdist(xr, cb + (int64_t)c * sub_dim, sub_dim, dtype);
            if (dist < best) {
                best = dist;
                best_idx = (uint32_t)c;
            }
        }
        float second = INFINITY;
        for (int c = 0; c < n_centroids; ++c) {
            if ((uint32_t)c == best_idx) continue;
            float dist = vqo_sqdist(xr, cb + (int64_t)c * sub_dim, sub_dim, dtype);
            if (dist < second) second = dist;
        }
        out[r] = best_idx;
        best_out[r] = best;
        second_out[r] = second;
    }
    return 0;
}

/*
 * Gather: row r of the output is centroid idx[r] of the codebook slot of r,
 * copied bit for bit.  An index >= n_centroids, or a bad slot, gives a row of
 * zero bits.  This is the reconstruction the page measures its MSE on
 * (section "Correctness: Bit-Exact on fp32, MSE-Identical on fp16").
 */
int vqo_decode(const uint32_t *idx, const uint16_t *codebook, int64_t n, int sub_dim,
               int n_centroids, int dtype, int64_t codebook_stride, int64_t n_codebooks,
               int64_t group_len, const int32_t *group_map, uint16_t *out_x)
{
    if (!args_ok(n, sub_dim, n_centroids, dtype, n_codebooks, group_len)) return -1;
    for (int64_t r = 0; r < n; ++r) {
        int64_t slot;
        uint16_t *dst = out_x + r * sub_dim;
        if (!slot_of(r, group_len, group_map, n_codebooks, &slot) ||
            idx[r] >= (uint32_t)n_centroids) {
            for (int i = 0; i < sub_dim; ++i) dst[i] = 0;
            continue;
        }
        const uint16_t *src = codebook + slot * codebook_stride + (int64_t)idx[r] * sub_dim;
        for (int i = 0; i < sub_dim; ++i) dst[i] = src[i];
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * The two steps on either side of the search in a VecInfer key cache.
 *
 * Smoothing (VeloxQuant-MLX blog, post introducing the library's nine
 * algorithms, section "VecInfer -- 16x with Metal acceleration": a scale per
 * channel tames the outlier channels that defeat plain VQ; "I Wrote a Metal
 * Kernel to Stop My Mac From OOMing", section "How to Use This Today": the
 * cache is configured with calibrated smooth factors, and section "What's
 * Next: Phase 2": the attention LUT is built from the correspondingly
 * transformed query q_tilde).  Reading taken: every channel of a key is
 * multiplied by its own fp32 factor (one IEEE multiply, rounded to nearest
 * even) before the search, and the search then runs on those fp32 values
 * exactly as in vqo_encode.  Smoothing by a divisor s is the multiplier 1/s.
 * The key cache is laid out [..][tokens][head_dim] and cut into sub-vectors
 * along head_dim, so component i of sub-vector r is channel
 * (r mod (head_dim / sub_dim)) * sub_dim + i.  The factor vector is chosen by
 * the codebook slot of the sub-vector: slot s uses
 * channel_scale[s * scale_stride .. + head_dim) (scale_stride 0 = one vector
 * for every slot).
 *
 * Packed codes ("I Wrote a Metal Kernel ...", section "What Even Is a KV
 * Cache And Why Should You Care": a 128-dim fp16 key becomes 16 indices of 8
 * bits; "How I built VeloxQuant-MLX -- KV cache compression for LLMs running
 * on your Mac", section "The Bit-Packing Problem": b-bit indices are packed
 * back to back into bytes, least significant bit first, an index may straddle
 * a byte boundary).  Code r occupies bits r*b .. r*b + b - 1 of the stream,
 * bit k of the stream being bit (k mod 8) of byte k / 8; the unused high bits
 * of the last byte are zero.  A sub-vector whose slot is out of range gets a
 * code of b one-bits (the low b bits of the 0xFFFFFFFF sentinel).
 * ------------------------------------------------------------------------ */

/* Distance from an fp32 sub-vector to one fp16/bf16 centroid: the same
 * sequence as vqo_sqdist with the sub-vector already in fp32. */
static float sqdist_f32(const float *xs, const uint16_t *crow, int sub_dim, int dtype)
{
    float dist = 0.0f;
    for (int i = 0; i < sub_dim; ++i) {
        float d = xs[i] - widen(crow[i], dtype);
        dist = fmaf(d, d, dist);
    }
    return dist;
}

/*
 * Smoothed sub-vectors: xs[r][i] = fp32(x[r][i]) * factor of its channel.
 * channel_scale NULL means every factor is 1 (xs is the exact widening).
 * Rows whose slot is out of range are filled with NaN.  head_dim must be a
 * positive multiple of sub_dim.  Returns 0, or -1 on a bad argument.
 */
int vqo_smooth(const uint16_t *x, int64_t n, int sub_dim, int dtype,
               const float *channel_scale, int head_dim, int64_t scale_stride,
               int64_t n_codebooks, int64_t group_len, const int32_t *group_map, float *xs)
{
    if (n < 0 || sub_dim < 1 || (dtype != VQO_F16 && dtype != VQO_BF16) ||
        n_codebooks < 1 || group_len < 1 || head_dim < sub_dim || head_dim % sub_dim ||
        scale_stride < 0)
        return -1;
    const int n_sub = head_dim / sub_dim;
    for (int64_t r = 0; r < n; ++r) {
        int64_t slot;
        float *dst = xs + r * sub_dim;
        if (!slot_of(r, group_len, group_map, n_codebooks, &slot)) {
            for (int i = 0; i < sub_dim; ++i) dst[i] = NAN;
            continue;
        }
        const int64_t ch0 = (r % n_sub) * sub_dim;
        for (int i = 0; i < sub_dim; ++i) {
            float v = widen(x[r * sub_dim + i], dtype);
            if (channel_scale) v = v * channel_scale[slot * scale_stride + ch0 + i];
            dst[i] = v;
        }
    }
    return 0;
}

/*
 * The search of vqo_encode over fp32 sub-vectors xs [n][sub_dim] against
 * fp16/bf16 codebook slots.  best_out and second_out may be NULL; when given
 * they receive the winning distance and the minimum over every other centroid
 * (as in vqo_encode_top2).
 */
int vqo_encode_f32(const float *xs, const uint16_t *codebook, int64_t n, int sub_dim,
                   int n_centroids, int dtype, int64_t codebook_stride, int64_t n_codebooks,
                   int64_t group_len, const int32_t *group_map, uint32_t *out,
                   float *best_out, float *second_out)
{
    if (!args_ok(n, sub_dim, n_centroids, dtype, n_codebooks, group_len)) return -1;
    for (int64_t r = 0; r < n; ++r) {
        int64_t slot;
        if (!slot_of(r, group_len, group_map, n_codebooks, &slot)) {
            out[r] = VQO_BAD_SLOT;
            if (best_out) best_out[r] = NAN;
            if (second_out) second_out[r] = NAN;
            continue;
        }
        const uint16_t *cb = codebook + slot * codebook_stride;
        const float *xr = xs + r * sub_dim;
        float best = INFINITY;
        uint32_t best_idx = 0;
        for (int c = 0; c < n_centroids; ++c) {
            float dist = sqdist_f32(xr, cb + (int64_t)c * sub_dim, sub_dim, dtype);
            if (dist < best) {
                best = dist;
                best_idx = (uint32_t)c;
            }
        }
        out[r] = best_idx;
        if (best_out) best_out[r] = best;
        if (second_out) {
            float second = INFINITY;
            for (int c = 0; c < n_centroids; ++c) {
                if ((uint32_t)c == best_idx) continue;
                float dist = sqdist_f32(xr, cb + (int64_t)c * sub_dim, sub_dim, dtype);
                if (dist < second) second = dist;
            }
            second_out[r] = second;
        }
    }
    return 0;
}

/* Bytes of a stream of n codes of code_bits bits. */
int64_t vqo_packed_bytes(int64_t n, int code_bits)
{
    return (n * code_bits + 7) / 8;
}

/*
 * Pack n codes into the LSB-first bit stream, one bit at a time: bit k of
 * code r goes to stream bit r*code_bits + k.  Only the low code_bits bits of
 * each code are kept.  out receives vqo_packed_bytes(n, code_bits) bytes.
 */
int vqo_pack(const uint32_t *codes, int64_t n, int code_bits, uint8_t *out)
{
    if (n < 0 || code_bits < 1 || code_bits > 32) return -1;
    memset(out, 0, (size_t)vqo_packed_bytes(n, code_bits));
    for (int64_t r = 0; r < n; ++r) {
        for (int k = 0; k < code_bits; ++k) {
            int64_t bit = r * code_bits + k;
            uint32_t b = (codes[r] >> k) & 1u;
            out[bit / 8] |= (uint8_t)(b << (bit % 8));
        }
    }
    return 0;
}

/* Inverse of vqo_pack. */
int vqo_unpack(const uint8_t *in, int64_t n, int code_bits, uint32_t *codes)
{
    if (n < 0 || code_bits < 1 || code_bits > 32) return -1;
    for (int64_t r = 0; r < n; ++r) {
        uint32_t c = 0;
        for (int k = 0; k < code_bits; ++k) {
            int64_t bit = r * code_bits + k;
            c |= (uint32_t)((in[bit / 8] >> (bit % 8)) & 1u) << k;
        }
        codes[r] = c;
    }
    return 0;
}

/*
 * Smooth, search, pack: the encode of a VecInfer key cache from raw keys to
 * stored codes.  Requires n_centroids <= 2^code_bits.  out_codes receives
 * vqo_packed_bytes(n, code_bits) bytes.  Returns 0, -1 on a bad argument, -2
 * when scratch memory cannot be had.
 */
int vqo_encode_packed(const uint16_t *x, const uint16_t *codebook, int64_t n, int sub_dim,
                      int n_centroids, int dtype, int64_t codebook_stride, int64_t n_codebooks,
                      int64_t group_len, const int32_t *group_map, const float *channel_scale,
                      int head_dim, int64_t scale_stride, int code_bits, uint8_t *out_codes)
{
    if (!args_ok(n, sub_dim, n_centroids, dtype, n_codebooks, group_len) ||
        code_bits < 1 || code_bits > 32 ||
        (code_bits < 32 && (int64_t)n_centroids > ((int64_t)1 << code_bits)))
        return -1;
    float *xs = malloc((size_t)(n > 0 ? n : 1) * sub_dim * sizeof(float));
    uint32_t *idx = malloc((size_t)(n > 0 ? n : 1) * sizeof(uint32_t));
    int rc = (xs && idx) ? 0 : -2;
    if (rc == 0)
        rc = vqo_smooth(x, n, sub_dim, dtype, channel_scale, head_dim, scale_stride,
                        n_codebooks, group_len, group_map, xs);
    if (rc == 0)
        rc = vqo_encode_f32(xs, codebook, n, sub_dim, n_centroids, dtype, codebook_stride,
                            n_codebooks, group_len, group_map, idx, NULL, NULL);
    if (rc == 0) rc = vqo_pack(idx, n, code_bits, out_codes);
    free(xs);
    free(idx);
    return rc;
}
