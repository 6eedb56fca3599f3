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
