// Calls every C-ABI entry point with many argument combinations -- valid,
// invalid and extreme (sizes near INT64_MAX, negative counts, misaligned
// pointers) -- under AddressSanitizer and UndefinedBehaviorSanitizer.  The
// pointers are never dereferenced by the argument checks, and the stubbed
// launchers make a passing combination return VQ_ERR_DEVICE.  Exit 0 when
// every status is one the header defines; the sanitizers abort on any
// overflow, out-of-bounds access or other undefined behaviour.
#include <cstdint>
#include <cstdio>

#include "vq.h"

namespace {
uint64_t state = 0x9E3779B97F4A7C15ull;
uint64_t next() {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return state;
}
template <typename T>
T pick(const T *v, int n) { return v[next() % n]; }

const int64_t kI64[] = {0, 1, 2, 31, 32, 33, 1000, 4096, 131072, (int64_t(1) << 31) + 7,
                        (int64_t(1) << 40), INT64_MAX / 64, INT64_MAX / 8, INT64_MAX - 1,
                        INT64_MAX, -1, INT64_MIN};
const int32_t kI32[] = {0, 1, 2, 3, 4, 8, 16, 7, 64, 96, 128, 255, 256, 257, 4096, 65536, 65537,
                        INT32_MAX, -1, INT32_MIN};
const uintptr_t kPtr[] = {0, 0x10000, 0x10002, 0x10004, 0x10008, 0x10001};
const float kF[] = {0.0625f, 1.0f, -2.0f, 3.3e38f, -3.3e38f, __builtin_nanf(""), __builtin_inff()};

const void *P() { return reinterpret_cast<const void *>(pick(kPtr, 6)); }
bool known(int s) { return s <= 0 && s >= -5; }
}  // namespace

int main() {
  int bad = 0;
  for (int it = 0; it < 200000; ++it) {
    const int which = static_cast<int>(next() % 7);
    int s = 0;
    switch (which) {
      case 0:
        s = vq_encode(P(), P(), pick(kI64, 17), pick(kI32, 20), pick(kI32, 20),
                      static_cast<vq_dtype>(next() % 3), pick(kI64, 17), pick(kI64, 17),
                      pick(kI64, 17), static_cast<const int32_t *>(P()),
                      static_cast<uint32_t *>(const_cast<void *>(P())), nullptr);
        break;
      case 1:
        s = vq_encode_packed(P(), P(), pick(kI64, 17), pick(kI32, 20), pick(kI32, 20),
                             static_cast<vq_dtype>(next() % 3), pick(kI64, 17), pick(kI64, 17),
                             pick(kI64, 17), static_cast<const int32_t *>(P()),
                             static_cast<const float *>(P()), pick(kI32, 20), pick(kI64, 17),
                             pick(kI32, 20), const_cast<void *>(P()), nullptr);
        break;
      case 2:
        s = vq_decode(static_cast<const uint32_t *>(P()), P(), pick(kI64, 17), pick(kI32, 20),
                      pick(kI32, 20), static_cast<vq_dtype>(next() % 3), pick(kI64, 17),
                      pick(kI64, 17), pick(kI64, 17), static_cast<const int32_t *>(P()),
                      const_cast<void *>(P()), nullptr);
        break;
      case 3:
        s = vq_kmeans(P(), const_cast<void *>(P()), pick(kI64, 17), pick(kI32, 20), pick(kI32, 20),
                      static_cast<vq_dtype>(next() % 3), pick(kI64, 17), pick(kI64, 17),
                      pick(kI64, 17), static_cast<const int32_t *>(P()), pick(kI32, 20),
                      static_cast<uint32_t *>(const_cast<void *>(P())), const_cast<void *>(P()),
                      static_cast<size_t>(pick(kI64, 17)), nullptr);
        (void)vq_kmeans_workspace_bytes(pick(kI32, 20), pick(kI32, 20), pick(kI64, 17),
                                        static_cast<vq_dtype>(next() % 3));
        break;
      case 4:
      case 5: {
        const bool st = which == 5;
        const void *q = P();
        const uint8_t *kc = static_cast<const uint8_t *>(P()), *vc = static_cast<const uint8_t *>(P());
        const float *ks = static_cast<const float *>(P());
        const int32_t *kl = static_cast<const int32_t *>(P());
        float *out = static_cast<float *>(const_cast<void *>(P()));
        const int32_t B = pick(kI32, 20), Hq = pick(kI32, 20), Hkv = pick(kI32, 20),
                      D = pick(kI32, 20), S = pick(kI32, 20);
        (void)vq_attention_workspace_bytes(B, Hq, D, S);
        if (st) {
          s = vq_attention_decode_static(q, kc, vc, P(), P(), ks, kl, B, Hq, Hkv, D, S,
                                         pick(kI32, 20), pick(kI32, 20), pick(kI32, 20),
                                         static_cast<vq_dtype>(next() % 3), pick(kI32, 20),
                                         pick(kF, 7), out, nullptr);
        } else {
          s = vq_attention_decode(q, kc, vc, P(), P(), ks, kl, B, Hq, Hkv, D, S, pick(kI32, 20),
                                  pick(kI32, 20), pick(kI32, 20),
                                  static_cast<vq_dtype>(next() % 3), pick(kI32, 20), pick(kF, 7),
                                  out, const_cast<void *>(P()), static_cast<size_t>(pick(kI64, 17)),
                                  nullptr);
        }
        break;
      }
      default:
        s = 0;
        (void)vq_status_str(static_cast<int32_t>(next() % 9) - 6);
        (void)vq_last_hip_error();
        (void)vq_abi_version();
    }
    if (!known(s)) {
      if (++bad < 5) std::printf("call %d returned unknown status %d\n", which, s);
    }
  }
  std::printf("capi sanitizer run: %d unknown statuses\n", bad);
  return bad ? 1 : 0;
}
