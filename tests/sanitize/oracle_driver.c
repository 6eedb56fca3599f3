/* Runs the CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer
 * on seeded inputs (every fp16/bf16 bit pattern can occur: subnormals,
 * infinities, NaN), with invariants that need no second implementation:
 *   - the top-2 search returns the encode's index, and its best distance is
 *     the distance to that index;
 *   - the fp32 search over unscaled smoothed keys (an exact widening) returns
 *     the encode's indices;
 *   - unpacking a packed stream returns the low bits of every code;
 *   - decode of an index >= n_centroids gives a zero row.
 * Exit 0 when every invariant holds; the sanitizers abort on any fault. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int vqo_encode(const uint16_t *, const uint16_t *, int64_t, int, int, int, int64_t, int64_t,
               int64_t, const int32_t *, uint32_t *);
int vqo_encode_top2(const uint16_t *, const uint16_t *, int64_t, int, int, int, int64_t, int64_t,
                    int64_t, const int32_t *, uint32_t *, float *, float *);
int vqo_decode(const uint32_t *, const uint16_t *, int64_t, int, int, int, int64_t, int64_t,
               int64_t, const int32_t *, uint16_t *);
int vqo_smooth(const uint16_t *, int64_t, int, int, const float *, int, int64_t, int64_t, int64_t,
               const int32_t *, float *);
int vqo_encode_f32(const float *, const uint16_t *, int64_t, int, int, int, int64_t, int64_t,
                   int64_t, const int32_t *, uint32_t *, float *, float *);
float vqo_sqdist(const uint16_t *, const uint16_t *, int, int);
int64_t vqo_packed_bytes(int64_t, int);
int vqo_pack(const uint32_t *, int64_t, int, uint8_t *);
int vqo_unpack(const uint8_t *, int64_t, int, uint32_t *);
int vqo_encode_packed(const uint16_t *, const uint16_t *, int64_t, int, int, int, int64_t, int64_t,
                      int64_t, const int32_t *, const float *, int, int64_t, int, uint8_t *);

static uint64_t st = 0x243F6A8885A308D3ull;
static uint64_t rnd(void) {
  st ^= st << 13;
  st ^= st >> 7;
  st ^= st << 17;
  return st;
}

int main(void) {
  int bad = 0;
  for (int it = 0; it < 400; ++it) {
    const int sd = 1 + (int)(rnd() % 8), nc = 1 + (int)(rnd() % 40), dt = (int)(rnd() % 2);
    const int64_t n = (int64_t)(rnd() % 70), slots = 1 + (int64_t)(rnd() % 3);
    const int64_t glen = 1 + (int64_t)(rnd() % 30), stride = (int64_t)nc * sd + (int64_t)(rnd() % 3);
    const int64_t groups = n ? (n - 1) / glen + 1 : 1;
    uint16_t *x = malloc(sizeof(uint16_t) * (size_t)(n * sd + 1));
    uint16_t *cb = malloc(sizeof(uint16_t) * (size_t)(slots * stride));
    int32_t *map = malloc(sizeof(int32_t) * (size_t)groups);
    uint32_t *idx = malloc(sizeof(uint32_t) * (size_t)(n + 1));
    uint32_t *idx2 = malloc(sizeof(uint32_t) * (size_t)(n + 1));
    float *best = malloc(sizeof(float) * (size_t)(n + 1)), *second = malloc(sizeof(float) * (size_t)(n + 1));
    float *xs = malloc(sizeof(float) * (size_t)(n * sd + 1));
    uint16_t *rec = malloc(sizeof(uint16_t) * (size_t)(n * sd + 1));
    const int special = (int)(rnd() % 4);  /* 0: any bits; else finite moderate values */
    for (int64_t i = 0; i < n * sd; ++i)
      x[i] = special ? (uint16_t)((rnd() & 0x83FF) | (0x3000 + (rnd() % 0x0C00))) : (uint16_t)rnd();
    for (int64_t i = 0; i < slots * stride; ++i)
      cb[i] = special ? (uint16_t)((rnd() & 0x83FF) | (0x3000 + (rnd() % 0x0C00))) : (uint16_t)rnd();
    for (int64_t g = 0; g < groups; ++g) map[g] = (int32_t)(rnd() % (uint64_t)(slots + 1)) - (rnd() % 5 == 0);
    const int32_t *gm = (rnd() % 2) ? map : NULL;
    const int64_t ncb = gm ? slots : groups > slots ? groups : slots;
    uint16_t *cbu = cb;
    if (!gm && ncb > slots) {  /* identity slots: one codebook per group */
      cbu = malloc(sizeof(uint16_t) * (size_t)(ncb * stride));
      for (int64_t i = 0; i < ncb * stride; ++i) cbu[i] = cb[i % (slots * stride)];
    }
    if (vqo_encode(x, cbu, n, sd, nc, dt, stride, ncb, glen, gm, idx) != 0) bad++;
    if (vqo_encode_top2(x, cbu, n, sd, nc, dt, stride, ncb, glen, gm, idx2, best, second) != 0) bad++;
    for (int64_t r = 0; r < n; ++r) {
      if (idx[r] != idx2[r]) bad++;
      if (idx[r] < (uint32_t)nc) {
        const int64_t s = gm ? gm[r / glen] : r / glen;
        const float d = vqo_sqdist(x + r * sd, cbu + s * stride + (int64_t)idx[r] * sd, sd, dt);
        /* the winner's distance, or +inf kept when no distance is below it */
        if (!(d == best[r] || (best[r] == INFINITY && !(d < INFINITY)))) bad++;
      }
    }
    if (vqo_smooth(x, n, sd, dt, NULL, sd, 0, ncb, glen, gm, xs) != 0) bad++;
    if (vqo_encode_f32(xs, cbu, n, sd, nc, dt, stride, ncb, glen, gm, idx2, NULL, NULL) != 0) bad++;
    for (int64_t r = 0; r < n; ++r)
      if (idx[r] != idx2[r]) bad++;
    for (int64_t r = 0; r < n; ++r) idx2[r] = (uint32_t)(rnd() % (uint64_t)(nc + 3));
    if (vqo_decode(idx2, cbu, n, sd, nc, dt, stride, ncb, glen, gm, rec) != 0) bad++;
    for (int64_t r = 0; r < n; ++r)
      if (idx2[r] >= (uint32_t)nc)
        for (int i = 0; i < sd; ++i)
          if (rec[r * sd + i] != 0) bad++;
    const int bits = 1 + (int)(rnd() % 32);
    uint8_t *packed = malloc((size_t)vqo_packed_bytes(n, bits) + 1);
    for (int64_t r = 0; r < n; ++r) idx2[r] = (uint32_t)rnd();
    if (vqo_pack(idx2, n, bits, packed) != 0) bad++;
    if (vqo_unpack(packed, n, bits, idx) != 0) bad++;
    const uint32_t mask = bits == 32 ? 0xFFFFFFFFu : ((1u << bits) - 1u);
    for (int64_t r = 0; r < n; ++r)
      if (idx[r] != (idx2[r] & mask)) bad++;
    const int cbits = 6 + (int)(rnd() % 3);
    uint8_t *codes = malloc((size_t)vqo_packed_bytes(n, cbits) + 1);
    float *f = malloc(sizeof(float) * (size_t)(ncb * 2 * sd));
    for (int64_t i = 0; i < ncb * 2 * sd; ++i) f[i] = (float)((rnd() % 1000) + 1) / 250.0f;
    const int rc = vqo_encode_packed(x, cbu, n, sd, nc, dt, stride, ncb, glen, gm, f, 2 * sd,
                                     2 * sd, cbits, codes);
    if (rc != 0) bad++;  /* n_centroids <= 40 < 2^6 */
    free(codes);
    free(f);
    free(packed);
    if (cbu != cb) free(cbu);
    free(x); free(cb); free(map); free(idx); free(idx2); free(best); free(second); free(xs);
    free(rec);
  }
  /* bad arguments are rejected */
  if (vqo_encode(NULL, NULL, -1, 4, 4, 0, 16, 1, 1, NULL, NULL) != -1) bad++;
  if (vqo_pack(NULL, 5, 33, NULL) != -1) bad++;
  printf("oracle sanitizer run: %d invariant failures\n", bad);
  return bad ? 1 : 0;
}
