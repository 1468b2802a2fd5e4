// nf4_device.h -- device-side pieces shared by the libnf4 kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4 {

// The 16 NF4 levels as fp32 bit patterns.  Values: QLoRA's 4-bit NormalFloat
// (quantiles of N(0,1): 8 positive levels from an evenly spaced 9-point
// probability grid between 1 - (1/30 + 1/32)/2 and 1/2, 7 negative ones from an
// 8-point grid, plus an exact 0, normalised to [-1, 1]), each rounded to fp32.
// The deep-fold README's "Method" section names QLoRA's NF4 as the code.
constexpr uint32_t kLevelBits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu, 0xbe91a24bu, 0xbe3d353du,
    0xbdba7869u, 0x00000000u, 0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u,
    0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u, 0x3f800000u};

// Level c as fp32, through a chain of selects (no memory access).
__device__ __forceinline__ float level_f32(uint32_t c) {
  uint32_t r = kLevelBits[0];
#pragma unroll
  for (uint32_t i = 1; i < 16; ++i) r = (c == i) ? kLevelBits[i] : r;
  return __uint_as_float(r);
}

// f16 bit patterns of the levels, rounded to nearest even at compile time.
struct LevelF16 {
  uint32_t v[16];
};
constexpr LevelF16 make_level_f16() {
  LevelF16 r{};
  for (int i = 0; i < 16; ++i)
    r.v[i] = (uint32_t)__builtin_bit_cast(uint16_t,
                                          (_Float16)__builtin_bit_cast(float, kLevelBits[i]));
  return r;
}
constexpr LevelF16 kLevelF16 = make_level_f16();

// ---------------------------------------------------------------------------
// Byte decode table in LDS.
// Entry for a packed byte b holds the two f16 levels of its nibbles:
//   low half  = L[b & 15]  (even k),  high half = L[b >> 4]  (odd k),
// i.e. exactly the operand pair of one v_dot2_f32_f16 against (x[2j], x[2j+1]).
// Each entry is replicated 32 times, 4 bytes apart, at a 256-byte stride: lane l
// reads copy l % 32 at byte address b * 256 + 4 * (l % 32).  LDS serves a 32-bit
// read in two halves of 32 lanes, and within a half every lane hits its own bank
// whatever the codes are (measured: no slower than 64 copies, and half the
// table writes).  The address is one v_perm_b32 from the code word.  The upper
// 128 bytes of each 256-byte row are not written.
// ---------------------------------------------------------------------------
constexpr int kLutWords = 256 * 64;  // 64 KiB of addresses, 32 KiB written

// Wave w writes the entries whose high nibble h satisfies h % nwaves == w: for
// one h that is 16 entries x 32 copies = 128 uint4 stores, 2 per lane.  Store
// (h, j, lane) covers copies 4 (lane % 8) .. + 3 of entry 16h + 8j + lane/8, so
// the high level is a constant of the unrolled loop and the low level an
// 8-way choice fixed per lane.
__device__ __forceinline__ void build_byte_lut(uint32_t *lut, int tid, int nthreads) {
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwaves = nthreads >> 6;
  const uint32_t sub = (uint32_t)lane >> 3;
  uint32_t lo[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint32_t v = kLevelF16.v[8 * j];
#pragma unroll
    for (int q = 1; q < 8; ++q) v = sub == (uint32_t)q ? kLevelF16.v[8 * j + q] : v;
    lo[j] = v;
  }
  uint4 *L4 = reinterpret_cast<uint4 *>(lut);
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    if (h % nwaves == wave) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t e = lo[j] | (kLevelF16.v[h] << 16);
        L4[(16 * h + 8 * j + sub) * 16 + (lane & 7)] = make_uint4(e, e, e, e);
      }
    }
  }
}

// lane offset into an entry: copy lane % 32
__device__ __forceinline__ uint32_t lut_lane_offset(int lane) { return (uint32_t)(lane & 31) * 4u; }

// selector for v_perm_b32: result byte0 = lane offset (low byte of src1),
// byte1 = byte `j` of the code word (src0), bytes 2..3 = 0
//   -> (code_byte_j << 8) | (4 * (lane % 32))
template <int j>
__device__ __forceinline__ uint32_t lut_addr(uint32_t codeword, uint32_t laneoff) {
  constexpr uint32_t sel = 0x0c0c0000u | ((4u + j) << 8) | 0x00u;
  return __builtin_amdgcn_perm(codeword, laneoff, sel);
}

// Buffer resource word 3 for raw (untyped) buffer access on gfx9-family parts,
// and the cache-policy operand of a streamed (read-once) load: non-temporal.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kLoadStream = 2;

// 16-byte load of streamed data (read once): non-temporal hint
typedef uint32_t u32x4_nt_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void *p) {
  const u32x4_nt_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t lds_load_u32(const uint32_t *base, uint32_t byte_addr) {
  return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(base) + byte_addr);
}

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// binary16 bits -> fp32 (exact)
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// ---------------------------------------------------------------------------
// Wave reductions with DPP row operations plus lane reads: no LDS traffic.
// Every lane of a row of 16 ends with the row's sum after four steps (xor 1,
// xor 2, half-row mirror, row mirror -- each pairs lanes symmetrically, so all
// 16 lanes hold identical bits); the four row sums are then added in row order.
// ---------------------------------------------------------------------------
template <int ctrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl,
                                                               0xf, 0xf, false));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace nf4
