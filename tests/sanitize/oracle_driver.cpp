// Host sanitizer run of the CPU oracle: every entry point of oracle/nf4_oracle.h
// on small inputs and edge cases (zero, tiny, huge, non-finite groups; every
// code; ragged row subsets; bad embedding ids), built with AddressSanitizer
// and UndefinedBehaviorSanitizer.  It checks memory safety and defined
// behaviour only; the values are pinned by the Python tests.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>
#include <vector>

#include "nf4_oracle.h"

static int run_case(int64_t N, int64_t K, int64_t M, uint32_t seed, float scale, int special) {
  std::mt19937 rng(seed);
  std::normal_distribution<float> nd(0.0f, 1.0f);
  std::vector<float> W(N * K);
  for (auto &w : W) w = nd(rng) * scale;
  if (special == 1) W[0] = NAN;
  if (special == 2) W[K - 1] = std::numeric_limits<float>::infinity();
  if (special == 3) W[1] = 70000.0f;
  if (special == 4)
    for (int64_t k = 0; k < 64 && k < K; ++k) W[k] = 0.0f;
  if (special == 5)
    for (int64_t k = 0; k < 64 && k < K; ++k) W[k] = 3e-8f * (float)(k % 5);
  std::vector<uint8_t> codes(N * K), packed(N * K / 2), back(N * K);
  std::vector<uint16_t> scales(N * (K / 64));
  (void)orc_quantize(W.data(), N, K, codes.data(), scales.data());
  orc_pack(codes.data(), N, K, packed.data());
  orc_unpack_codes(packed.data(), N, K, back.data());
  if (std::memcmp(codes.data(), back.data(), codes.size()) != 0) return 1;
  std::vector<double> Wd(N * K);
  std::vector<float> Wf(N * K);
  orc_dequant_f64(packed.data(), scales.data(), N, K, Wd.data());
  orc_dequant_f32(packed.data(), scales.data(), N, K, Wf.data());
  std::vector<uint16_t> X(M * K);
  for (auto &x : X) {
    const float v = nd(rng);
    uint32_t b;
    std::memcpy(&b, &v, 4);
    x = (uint16_t)(b >> 16);
  }
  std::vector<int64_t> rows;
  for (int64_t r = N - 1; r >= 0; r -= 2) rows.push_back(r);
  std::vector<double> Y(M * N), A(M * N), Yr(M * rows.size()), Ar(M * rows.size());
  orc_gemm_rows(packed.data(), scales.data(), N, K, X.data(), M, nullptr, N, Y.data(), A.data());
  orc_gemm_rows(packed.data(), scales.data(), N, K, X.data(), M, rows.data(),
                (int64_t)rows.size(), Yr.data(), nullptr);
  orc_gemm_rows(packed.data(), scales.data(), N, K, X.data(), M, rows.data(),
                (int64_t)rows.size(), Yr.data(), Ar.data());
  std::vector<int64_t> ids = {0, N - 1, N, -1, (N > 1 ? 1 : 0), 0};
  std::vector<uint16_t> out(ids.size() * K);
  (void)orc_embed(packed.data(), scales.data(), N, K, ids.data(), (int64_t)ids.size(),
                  out.data());
  (void)orc_embed(packed.data(), scales.data(), N, K, ids.data(), 0, out.data());
  return 0;
}

int main() {
  double lv64[16];
  float lv32[16];
  orc_codebook(lv64, lv32);
  for (double p : {1e-300, 1e-12, 0.01, 0.5, 0.9677083, 1.0 - 1e-12}) (void)orc_normal_quantile(p);
  for (float f : {0.0f, -0.0f, 1.0f, 0.1f, 65519.0f, 65520.0f, 6e-8f, 1e-30f, NAN, INFINITY})
    (void)orc_f32_to_f16_bits(f);
  for (uint32_t h = 0; h < 65536; ++h) {
    (void)orc_f16_bits_to_f64((uint16_t)h);
    (void)orc_bf16_bits_to_f64((uint16_t)h);
  }
  for (double v : {0.0, -0.0, 1.0, 3.0e38, 4.0e38, 1e-45, -1e-40, (double)NAN, (double)INFINITY,
                   1.00390625})
    (void)orc_f64_to_bf16_bits(v);
  int bad = 0;
  const int64_t shapes[][3] = {{1, 64, 1}, {2, 64, 3}, {3, 128, 2}, {5, 192, 1}, {7, 4096, 2}};
  uint32_t seed = 1;
  for (const auto &s : shapes)
    for (int special = 0; special <= 5; ++special)
      for (float scale : {0.02f, 1.0f, 3e4f, 1e-6f}) bad |= run_case(s[0], s[1], s[2], seed++, scale, special);
  std::printf("oracle sanitizer run: %s\n", bad ? "round trip FAILED" : "ok");
  return bad;
}
