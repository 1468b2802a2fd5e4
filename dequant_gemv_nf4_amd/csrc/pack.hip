// pack.hip -- NF4 quantize+pack and unpack kernels (gfx950).
//
// Format: deep-fold README, "Method" -- groups of 64 weights along K, 4-bit NF4
// codes, one FP16 scale per group.  Pack is offline work (the README's
// compressor runs before inference), so these kernels favour plainness.
#include "nf4_device.h"
#include "nf4_launch.h"

namespace nf4 {

// Decision boundaries between neighbouring levels, in fp64: (L[i] + L[i+1]) / 2.
// Exact: neighbouring fp32 levels are within one binade of each other (or one
// is 0), so the sum fits in 53 bits and the halving is exact.
struct Mids {
  double m[15];
};
__host__ __device__ constexpr Mids make_mids() {
  Mids r{};
  for (int i = 0; i < 15; ++i)
    r.m[i] = ((double)__builtin_bit_cast(float, kLevelBits[i]) +
              (double)__builtin_bit_cast(float, kLevelBits[i + 1])) / 2.0;
  return r;
}
__constant__ Mids kMids = make_mids();

__global__ void clear_status_kernel(int32_t *status) { *status = 0; }

// One wave per group of 64 weights, one weight per lane.
__global__ void __launch_bounds__(256) pack_kernel(const float *__restrict__ W, int64_t ngroups,
                                                   uint8_t *__restrict__ codes,
                                                   uint16_t *__restrict__ scales,
                                                   int32_t *__restrict__ status) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (g >= ngroups) return;  // whole wave leaves together
  const float w = W[g * 64 + lane];
  const bool finite = __builtin_isfinite(w);
  const float a = finite ? fabsf(w) : 0.0f;
  const float amax = wave_max(a);
  const bool any_bad = __any(!finite);
  // binary16 scale, round to nearest even (hardware conversion)
  const _Float16 sh = (_Float16)amax;
  const uint32_t sbits = (uint32_t)__builtin_bit_cast(uint16_t, sh);
  const bool overflow = (sbits & 0x7c00u) == 0x7c00u;
  int bad = (any_bad ? 1 : 0) | ((!any_bad && overflow) ? 2 : 0);
  uint32_t code = 7;
  uint32_t sout = 0;
  if (!bad) {
    sout = sbits;
    const double s = (double)(float)sh;
    if (s != 0.0) {
      const double wd = (double)w;
      code = 0;
#pragma unroll
      for (int i = 0; i < 15; ++i) code += (wd > kMids.m[i] * s) ? 1u : 0u;
    }
  }
  // gather 8 nibbles (k = 8t .. 8t+7) into one word in lane 8t
  uint32_t word = code << (4 * (lane & 7));
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) word |= __shfl_xor(word, off, 64);
  if ((lane & 7) == 0) reinterpret_cast<uint32_t *>(codes + g * 32)[lane >> 3] = word;
  if (lane == 0) {
    scales[g] = (uint16_t)sout;
    if (bad && status) atomicOr(status, bad);
  }
}

// One thread per code byte pair-word: 4 bytes -> 8 floats.
__global__ void __launch_bounds__(256) unpack_kernel(const uint8_t *__restrict__ codes,
                                                     const uint16_t *__restrict__ scales,
                                                     int64_t nwords, float *__restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= nwords) return;
  // word t covers weights 8t .. 8t+7, all in group (8t) / 64 (groups are row-local
  // because K % 64 == 0, so the flat index works across rows)
  const uint32_t q = reinterpret_cast<const uint32_t *>(codes)[t];
  const float s = f16_bits_to_f32(scales[t >> 3]);
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = level_f32((q >> (4 * i)) & 15u) * s;
  float4 *o = reinterpret_cast<float4 *>(out + t * 8);
  o[0] = make_float4(v[0], v[1], v[2], v[3]);
  o[1] = make_float4(v[4], v[5], v[6], v[7]);
}

hipError_t launch_pack(const float *W, int64_t N, int64_t K, uint8_t *codes, uint16_t *scales,
                       int32_t *status, hipStream_t stream) {
  if (status) {
    hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(1), 0, stream, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t ngroups = N * (K / 64);
  const int64_t blocks = (ngroups + 3) / 4;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, W, ngroups, codes,
                     scales, status);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                         float *out, hipStream_t stream) {
  const int64_t nwords = N * K / 8;
  const int64_t blocks = (nwords + 255) / 256;
  hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, codes, scales,
                     nwords, out);
  return hipGetLastError();
}

}  // namespace nf4
