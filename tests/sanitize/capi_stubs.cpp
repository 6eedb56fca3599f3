// Host-only stand-ins for the kernel launchers and the one HIP call of the
// C ABI, so that vq_capi.cpp's argument checks can run under AddressSanitizer
// and UndefinedBehaviorSanitizer on a machine without a GPU.  Every launcher
// reports failure; sizes follow the library's formulas closely enough for
// the checks (the checks, not these values, are what is under test).
#include <hip/hip_runtime.h>

#include "vq_launch.h"

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

namespace vqk {
int64_t encode_grid(const Layout &l) { return (l.n + 1023) / 1024; }
int64_t encode_mfma_grid(const Layout &) { return 256; }
bool encode_mfma_supported(const Layout &l) { return l.n_centroids <= 4096; }
int64_t kmeans_grid(const Layout &l) { return (l.n + 4095) / 4096; }
size_t kmeans_workspace_bytes(int sub_dim, int n_centroids, int64_t n_codebooks, bool bf16) {
  uint64_t r = 0;
  if (n_codebooks < 1 || n_centroids < 1 ||
      __builtin_mul_overflow(static_cast<uint64_t>(n_codebooks), static_cast<uint64_t>(n_centroids), &r) ||
      __builtin_mul_overflow(r, 8ull * (sub_dim * (bf16 ? 8 : 1) * 8 + 4), &r) || r > INT64_MAX)
    return 0;
  return r;
}
int attention_chunks(int max_kv_len) {
  return max_kv_len < 256 ? 1 : static_cast<int>((static_cast<int64_t>(max_kv_len) + 255) / 256);
}
size_t attention_lds_bytes(int, int, int, int) { return 1024; }
hipError_t launch_encode(const void *, const void *, const int32_t *, void *, const Layout &,
                         const Codes &, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_encode_mfma(const void *, const void *, const int32_t *, void *, const Layout &,
                              const Codes &, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_decode(const uint32_t *, const void *, const int32_t *, void *, const Layout &,
                         hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_kmeans(const void *, void *, const int32_t *, uint32_t *, const Layout &, int,
                         void *, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_attention(const AttnLayout &, hipStream_t) { return hipErrorNotSupported; }
hipError_t attention_static_scratch(void **ptr) {
  *ptr = nullptr;
  return hipErrorNotSupported;
}
}  // namespace vqk
