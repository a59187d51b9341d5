// Host-side argument checks of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (the library's host code is built with both;
// no device is touched: every call below is refused before any HIP call).
// Exit status 0 and no sanitizer report mean every check ran clean.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>

#include "av.h"
#include "av_test.h"

static int fails = 0;
#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    const int got_ = (call);                                                            \
    if (got_ != (want)) {                                                               \
      std::printf("FAIL line %d: %s returned %d, want %d\n", __LINE__, #call, got_, want); \
      ++fails;                                                                          \
    }                                                                                   \
  } while (0)

int main() {
  // fake, 16-byte aligned device addresses: never dereferenced
  void* P = reinterpret_cast<void*>(0x10000);
  int32_t* I = reinterpret_cast<int32_t*>(0x10000);
  float* F = reinterpret_cast<float*>(0x10000);
  const float nan = std::nanf(""), inf = INFINITY;

  // sizes at and beyond their limits
  for (int B : {INT_MIN, -1, 0, 1, 4095, 4096, INT_MAX})
    for (int k : {INT_MIN, 0, 1, 64, 65, INT_MAX})
      for (int R : {INT_MIN, -1, 0, 1, 2048, INT_MAX}) {
        (void)av_workspace_bytes(B, k, R);
        (void)av_spec_workspace_bytes(B, R);
      }
  (void)av_head_update_workspace_bytes(INT_MAX);
  (void)av_head_update_workspace_bytes(INT_MIN);
  EXPECT(av_workspace_bytes(0, 16, 10) == 0, 1);
  (void)av_noalloc_max_bytes();
  for (int R : {INT_MIN, -1, 0, 1, 2048, INT_MAX})
    for (int V : {INT_MIN, 0, 1, 151936, INT_MAX})
      for (int H : {INT_MIN, 0, 1, 4096, INT_MAX}) (void)av_lm_head_workspace_bytes(R, V, H);
  EXPECT(av_lm_head_workspace_bytes(0, 64, 16) == 0, 1);
  for (int s : {-4, -3, -2, -1, 0, 1, INT_MAX, INT_MIN}) (void)av_status_str(s);
  (void)av_last_hip_error();

  // forward: every refusal the header lists
  auto fwd = [&](int dtype, int B, int k, int V, int R, const int32_t* off, void* zp, float lam, float tau,
                 float gs, float T, float* stats, void* ws, size_t wsb, int gdt) {
    return av_verify_opd_fwd(dtype, B, k, V, R, off, zp, P, I, I, lam, tau, gs, T, I, I, F, nullptr, nullptr,
                             stats, nullptr, P, gdt, nullptr, ws, wsb, nullptr);
  };
  const size_t big = size_t(1) << 40;
  EXPECT(fwd(1, 2, 4, 64, 8, nullptr, nullptr, 0.5f, 0.1f, 1.f, 1.f, F, P, big, 0), AV_EINVAL);
  EXPECT(fwd(1, 0, 4, 64, 0, nullptr, P, 0.5f, 0.1f, 1.f, 1.f, F, P, big, 0), AV_EINVAL);
  EXPECT(fwd(1, INT_MAX, 64, 64, INT_MAX, nullptr, P, 0.5f, 0.1f, 1.f, 1.f, F, P, big, 0), AV_EINVAL);
  EXPECT(fwd(1, 2, 65, 64, 130, nullptr, P, 0.5f, 0.1f, 1.f, 1.f, F, P, big, 0), AV_EINVAL);
  EXPECT(fwd(1, 2, 4, INT_MIN, 8, nullptr, P, 0.5f, 0.1f, 1.f, 1.f, F, P, big, 0), AV_EINVAL);
  EXPECT(fwd(1, 2, 4, 64, 8, nullptr, P, nan, 0.1f, 1.f, 1.f, F, P, big, 0), AV_EINVAL);
  EXPECT(fwd(1, 2, 4, 64, 8, nullptr, P, 0.5f, nan, 1.f, 1.f, F, P, big, 0), AV_EINVAL);
  EXPECT(fwd(1, 2, 4, 64, 8, nullptr, P, 0.5f, 0.1f, inf, 1.f, F, P, big, 0), AV_EINVAL);
  EXPECT(fwd(1, 2, 4, 64, 8, nullptr, P, 0.5f, 0.1f, 1.f, nan, F, P, big, 0), AV_EINVAL);
  EXPECT(fwd(1, 2, 4, 64, 8, nullptr, P, 0.5f, 0.1f, 1.f, 1.f, F + 1, P, big, 0), AV_EINVAL);
  EXPECT(fwd(1, 2, 4, 64, 8, nullptr, P, 0.5f, 0.1f, 1.f, 1.f, F, P, 16, 0), AV_EINVAL);
  EXPECT(fwd(7, 2, 4, 64, 8, nullptr, P, 0.5f, 0.1f, 1.f, 1.f, F, P, big, 0), AV_EUNSUPPORTED);
  EXPECT(fwd(1, 2, 4, 64, 8, nullptr, P, 0.5f, 0.1f, 1.f, 1.f, F, P, big, 9), AV_EUNSUPPORTED);
  EXPECT(fwd(1, 1 << 16, 64, 1 << 24, 1 << 22, nullptr, P, 0.5f, 0.1f, 1.f, 1.f, F, P, big, 0),
         AV_EUNSUPPORTED);
  EXPECT(fwd(1, 5000, 4, 64, 5000, I, P, 0.5f, 0.1f, 1.f, 1.f, F, P, big, 0), AV_EUNSUPPORTED);
  EXPECT(av_test_verify_opd_fwd(1, 2, 4, 64, 8, nullptr, P, P, I, I, 0.5f, 0.1f, 1.f, 1.f, I, I, F, nullptr,
                                nullptr, F, nullptr, P, 0, nullptr, P, big, -1, 0, nullptr),
         AV_EINVAL);
  EXPECT(av_test_verify_opd_fwd(1, 2, 4, 64, 8, nullptr, P, P, I, I, 0.5f, 0.1f, 1.f, 1.f, I, I, F, nullptr,
                                nullptr, F, nullptr, P, 0, nullptr, P, big, 0, 5, nullptr),
         AV_EINVAL);
  EXPECT(av_verify_opd_fwd_noalloc(1, 2048, 16, 64, 2048 * 16, nullptr, P, P, I, I, 0.5f, 0.1f, 1.f, 1.f, I, I,
                                   F, nullptr, nullptr, nullptr, nullptr, P, 0, nullptr, nullptr),
         AV_EUNSUPPORTED);
  EXPECT(av_verify_opd_fwd_noalloc(1, 0, 16, 64, 0, nullptr, P, P, I, I, 0.5f, 0.1f, 1.f, 1.f, I, I, F,
                                   nullptr, nullptr, nullptr, nullptr, P, 0, nullptr, nullptr),
         AV_EINVAL);

  // backward
  EXPECT(av_verify_opd_bwd(1, 2, 4, 64, 8, nullptr, P, P, I, I, F, nullptr, 0.5f, 0.1f, 1.f, 2.f, P, 0, 0,
                           nullptr),
         AV_EINVAL);  // tempered without lse_q1
  EXPECT(av_verify_opd_bwd(1, 2, 4, 64 * 256 * 64 + 8, 8, nullptr, P, P, I, I, F, nullptr, 0.5f, 0.1f, 1.f,
                           1.f, P, 0, 0, nullptr),
         AV_EUNSUPPORTED);
  EXPECT(av_verify_opd_bwd(1, 2, 4, 64, 8, nullptr, P, P, I, I, F, nullptr, 0.5f, 0.1f, 1.f, 1.f, P, 0, INT_MIN,
                           nullptr),
         AV_EINVAL);

  // length head, its update, sampling verification, LM head
  EXPECT(av_length_head(F, F, nan, 1.f, 4, 16, 16, 0, F, I, nullptr), AV_EINVAL);
  EXPECT(av_length_head(F, F, 0.f, 1.f, INT_MIN, 16, 16, 0, F, I, nullptr), AV_EINVAL);
  EXPECT(av_length_head_update(F, I, I, 4, 16, 16, F, F, F, F, F, F, 0, 2e-4, 0.9, 0.999, 1e-8, 0.01, nullptr,
                               nullptr, nullptr, P, 1 << 20, nullptr),
         AV_EINVAL);
  EXPECT(av_length_head_update(F, I, I, INT_MAX, 16, 16, F, F, F, F, F, F, 1, 2e-4, 0.9, 0.999, 1e-8, 0.01,
                               nullptr, nullptr, nullptr, P, 8, nullptr),
         AV_EINVAL);
  EXPECT(av_spec_verify(1, INT_MAX, 4, 64, 8, nullptr, P, P, I, I, F, 1, nullptr, 0, I, I, nullptr, nullptr, P,
                        1 << 20, nullptr),
         AV_EINVAL);
  EXPECT(av_spec_verify(1, 2, 4, 64, 8, nullptr, P, P, I, I, F, 1, nullptr, 0, I, I, nullptr, nullptr, P, 7,
                        nullptr),
         AV_EINVAL);
  EXPECT(av_spec_verify(1, 2, 4, 64, 8, nullptr, P, P, I, I, F, 1, F, 1, I, I, nullptr, nullptr, P, 1 << 20,
                        nullptr),
         AV_EINVAL);
  EXPECT(av_workspace_init(nullptr, 1 << 20, nullptr), AV_EINVAL);
  EXPECT(av_workspace_init(reinterpret_cast<char*>(P) + 8, 1 << 20, nullptr), AV_EINVAL);
  EXPECT(av_lm_head_bwd(0, 64, 16, P, P, P, F, F, P, 1 << 20, nullptr), AV_EINVAL);
  EXPECT(av_lm_head_bwd(4, 64, 16, nullptr, P, P, F, F, P, 1 << 20, nullptr), AV_EINVAL);

  std::printf("%s (%d failed)\n", fails ? "FAILED" : "ok", fails);
  return fails ? 1 : 0;
}
