// nf4_split.h -- the NF4 levels split into bf16 hi + lo (compile time), for the
// matrix-core kernels whose operands are bf16.
//
// hi = bf16(L) and lo = bf16(L - hi), both rounded to nearest even, so that
// |L - hi - lo| < 2^-17 |L|: a level in bf16 alone would be off by up to 2^-9 of
// itself, beyond the product's tolerance.
#pragma once

#include "nf4_device.h"

namespace nf4 {

constexpr uint32_t bf16_rne_bits(uint32_t f) { return (f + 0x7fffu + ((f >> 16) & 1u)) >> 16; }

struct LevelSplit {
  uint32_t hi[16];
  uint32_t lo[16];
};
constexpr LevelSplit make_level_split() {
  LevelSplit r{};
  for (int i = 0; i < 16; ++i) {
    const uint32_t h = bf16_rne_bits(kLevelBits[i]);
    const float rest =
        __builtin_bit_cast(float, kLevelBits[i]) - __builtin_bit_cast(float, h << 16);
    r.hi[i] = h;
    r.lo[i] = bf16_rne_bits(__builtin_bit_cast(uint32_t, rest));
  }
  return r;
}
constexpr LevelSplit kSplit = make_level_split();

}  // namespace nf4
