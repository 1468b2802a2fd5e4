// Host sanitizer run of libnf4's C ABI validation layer: every entry point of
// include/nf4.h with null, misaligned, out-of-range and boundary arguments, and
// the host-only size queries over a grid of shapes, built (host code only) with
// AddressSanitizer and UndefinedBehaviorSanitizer.  Without a GPU every call
// that passes validation stops at the device check, so no kernel is launched;
// every argument pointer here is a fake address that is never dereferenced.
#include <cstdint>
#include <cstdio>

#include "nf4.h"

static int bad = 0;
static void expect(const char *what, int64_t got, int64_t want) {
  if (got != want) {
    std::printf("%s: got %lld, want %lld\n", what, (long long)got, (long long)want);
    bad = 1;
  }
}

int main() {
  auto P = reinterpret_cast<void *>(uintptr_t(0x100000));
  auto P2 = reinterpret_cast<void *>(uintptr_t(0x100002));
  auto *c = static_cast<const uint8_t *>(P);
  auto *s = static_cast<const uint16_t *>(P);
  auto *x = static_cast<const uint16_t *>(P);
  auto *y = static_cast<float *>(P);
  const int64_t Ns[] = {-1, 0, 1, 17, 4096, 28672, (int64_t(1) << 26), (int64_t(1) << 31),
                        INT64_MAX / 4};
  const int64_t Ks[] = {-64, 0, 63, 64, 100, 4096, 14336, 32768, 32832, INT64_MAX / 4};
  const int64_t Ms[] = {-5, 0, 1, 2, 4, 8, 31, 32, 33, 512, (int64_t(1) << 40)};
  for (int64_t N : Ns)
    for (int64_t K : Ks) {
      for (int64_t M : Ms) {
        (void)nf4_gemm_smallm_workspace_bytes(N, K, M);
        (void)nf4_gemm_prefill_workspace_bytes(N, K, M);
        const int a = nf4_gemm_smallm(c, s, N, K, x, M, y, nullptr);
        const int b = nf4_gemm_prefill(c, s, N, K, x, M, y, nullptr);
        const int w = nf4_gemm_smallm_ws(c, s, N, K, x, M, y, P, 1 << 20, nullptr);
        const int p = nf4_gemm_prefill_ws(c, s, N, K, x, M, y, P, 1 << 20, nullptr);
        if (a == NF4_OK || b == NF4_OK || w == NF4_OK || p == NF4_OK) {
          std::printf("a call passed the device check without a device\n");
          bad = 1;
        }
      }
      (void)nf4_gemv(c, s, N, K, x, y, nullptr);
      (void)nf4_pack(static_cast<const float *>(P), N, K, static_cast<uint8_t *>(P),
                     static_cast<uint16_t *>(P), nullptr, nullptr);
      (void)nf4_unpack(c, s, N, K, y, nullptr);
      (void)nf4_ring_slot_bytes(N, K);
      for (int64_t T : {int64_t(-1), int64_t(0), int64_t(1), int64_t(1) << 27, int64_t(1) << 40})
        (void)nf4_embed(c, s, N, K, static_cast<const int64_t *>(P), T,
                        static_cast<uint16_t *>(P), nullptr, nullptr);
    }
  expect("gemv null codes", nf4_gemv(nullptr, s, 4, 64, x, y, nullptr), NF4_EINVAL);
  expect("gemv misaligned x", nf4_gemv(c, s, 4, 64, static_cast<const uint16_t *>(P2), y, nullptr),
         NF4_EALIGN);
  expect("smallm M=33", nf4_gemm_smallm(c, s, 4, 64, x, 33, y, nullptr), NF4_ERANGE);
  expect("embed T<0", nf4_embed(c, s, 4, 64, static_cast<const int64_t *>(P), -1,
                                static_cast<uint16_t *>(P), nullptr, nullptr), NF4_EINVAL);
  expect("ring null", nf4_ring_gemm(nullptr, c, s, 4, 64, x, 1, y), NF4_EINVAL);
  expect("ring destroy null", nf4_ring_destroy(nullptr), NF4_EINVAL);
  nf4_ring *r = nullptr;
  expect("ring create misaligned", nf4_ring_create(&r, P2, P, 1024, nullptr, nullptr), NF4_EALIGN);
  float lv[16];
  nf4_codebook(lv);
  nf4_codebook(nullptr);
  for (int st = -8; st <= 2; ++st) (void)nf4_strerror(st);
  std::printf("abi sanitizer run: %s\n", bad ? "FAILED" : "ok");
  return bad;
}
