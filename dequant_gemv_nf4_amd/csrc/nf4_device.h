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

// Level c as fp32, through a chain of selects (no memory access: the decode
// tables are built from this once per workgroup).
__device__ __forceinline__ float level_f32(uint32_t c) {
  uint32_t r = kLevelBits[0];
#pragma unroll
  for (uint32_t i = 1; i < 16; ++i) r = (c == i) ? kLevelBits[i] : r;
  return __uint_as_float(r);
}

// f16 bit pattern of level c (round to nearest even, the hardware conversion).
__device__ __forceinline__ uint32_t level_f16_bits(uint32_t c) {
  _Float16 h = (_Float16)level_f32(c);
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// ---------------------------------------------------------------------------
// Byte decode table in LDS.
// Entry for a packed byte b holds the two f16 levels of its nibbles:
//   low half  = L[b & 15]  (even k),  high half = L[b >> 4]  (odd k),
// i.e. exactly the operand pair of one v_dot2_f32_f16 against (x[2j], x[2j+1]).
// Each entry is replicated 64 times, 4 bytes apart, so that lane l reads copy l:
// byte address = b * 256 + 4 * lane.  Every lane then hits its own bank whatever
// the codes are, and the address is one v_perm_b32 from the code word.
// ---------------------------------------------------------------------------
constexpr int kLutWords = 256 * 64;  // 64 KiB

__device__ __forceinline__ void build_byte_lut(uint32_t *lut, int tid, int nthreads) {
  // 16384 words written as 4096 uint4 stores of a splatted entry; an entry's
  // 64 copies take 16 consecutive stores, so store index q -> entry q / 16.
  for (int q = tid; q < kLutWords / 4; q += nthreads) {
    uint32_t b = (uint32_t)q >> 4;
    uint32_t e = level_f16_bits(b & 15u) | (level_f16_bits(b >> 4) << 16);
    reinterpret_cast<uint4 *>(lut)[q] = make_uint4(e, e, e, e);
  }
}

// selector for v_perm_b32: result byte0 = lane offset (low byte of src1),
// byte1 = byte `j` of the code word (src0), bytes 2..3 = 0
//   -> (code_byte_j << 8) | (4 * lane)
template <int j>
__device__ __forceinline__ uint32_t lut_addr(uint32_t codeword, uint32_t laneoff) {
  constexpr uint32_t sel = 0x0c0c0000u | ((4u + j) << 8) | 0x00u;
  return __builtin_amdgcn_perm(codeword, laneoff, sel);
}

__device__ __forceinline__ uint32_t lds_load_u32(const uint32_t *base, uint32_t byte_addr) {
  return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(base) + byte_addr);
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }
__device__ __forceinline__ uint32_t as_u32(half2_t v) { return __builtin_bit_cast(uint32_t, v); }

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// binary16 bits -> fp32 (exact)
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Sum over the 64 lanes of a wave, same bits in every lane; fixed order.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace nf4
