// gemm_prefill.hip -- fused NF4 dequant product for prefill batches of any
// size on the matrix cores (gfx950, v_mfma_f32_32x32x16_f16).
//
// Computes Y[m][n] = sum_k L[code(n,k)] * s(n,k/64) * X[m][k].  Sources:
// deep-fold README, "Method" (prefill runs the NF4 product on chunks of
// positions, the weights rebuilt into matrix-core register fragments and never
// written out); Trapetum home page, "The fine print" (prefill saves memory
// traffic, not time: once M is large the product is bound by the matrix cores,
// not by the weight stream).
//
// Tiling.  A workgroup of 4 waves (2 x 2) owns a (64 RM) x (64 CN) tile of Y
// and walks all of K in steps of one scale group (64 k); each wave owns
// RM x CN tiles of 32 x 32.  Per step:
//   - the workgroup stages the activation tile [64 RM][64] in LDS, converted to
//     f16: each row's 64 values are scaled by the power of two that puts their
//     largest |x| just under 2^15 (exact from bf16 down to 2^-32 of that
//     maximum; below, rounded to the f16 grid), with the row's 2^-shift kept
//     beside it;
//   - each wave loads the 32 code bytes of the group for each of its columns
//     (lane (n, h) the 16 bytes of k = 32h .. 32h+31) and decodes them through
//     the LDS byte table (nf4_device.h) straight into B fragments: f16 level
//     pairs, one table read per code byte;
//   - MFMA 32 x 32 x 16: A = activations (lane l: row l % 32, 8 k), B = weights
//     (lane l: column l % 32, the same 8 k).  Slice s of the group gives lane
//     half h the k = 32h + 8s .. +7, so a lane's code word s and its 16 bytes of
//     staged activations line up without any shuffling;
//   - the group's 32 x 32 tile (fp32) is multiplied by s(n, g) * 2^-shift(m, g)
//     and added to the fp32 accumulator.  No weight is rounded together with
//     its scale.
// A register ring keeps the loads of the next four (two, for 128 x 128) groups (activations, codes,
// scales) in flight; the activation stage is double-buffered in LDS, one
// barrier a step.
// Rows past M and columns past N re-read the last valid row or column and are
// never stored.  No atomics, no cross-workgroup traffic: bitwise reproducible.
#include <utility>

#include "nf4_device.h"
#include "nf4_launch.h"

namespace nf4 {

namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPThreads = 256;  // 4 waves: 2 (rows) x 2 (columns)
constexpr int kXRow = 144;      // bytes per staged activation row: 64 f16 + 16 B pad

__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// largest value over each aligned group of 8 lanes (quad swaps, then the
// half-row mirror, which pairs lane i with lane 7 - i of its 8)
__device__ __forceinline__ uint32_t max8(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));
  return v;
}

template <typename F, int... d>
__device__ __forceinline__ void for_slots(F &&f, std::integer_sequence<int, d...>) {
  (f(std::integral_constant<int, d>{}), ...);
}

template <int RM, int CN, int P>
__global__ void __launch_bounds__(kPThreads)
    gemm_prefill_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                        const uint16_t *__restrict__ X, float *__restrict__ Y, int N, int K,
                        int M) {
  constexpr int BM = 64 * RM;
  constexpr int kXChunks = BM * 8 / kPThreads;  // 16-byte activation chunks per thread
  constexpr int kStage = BM * kXRow;            // bytes of one activation buffer
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLutWords + (2 * kStage + 2 * BM * 4) / 4];
  uint32_t *const lut = lds;
  uint8_t *const xs = reinterpret_cast<uint8_t *>(lds + kLutWords);  // [2][BM][kXRow]
  float *const fm = reinterpret_cast<float *>(xs + 2 * kStage);       // [2][BM]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int col = lane & 31, h = lane >> 5;
  const int NG = K >> 6;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * (64 * CN);

  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(codes), 0, (int)((int64_t)N * (K >> 1)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(scales), 0, (int)((int64_t)N * NG * 2), kBufferWord3);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(X), 0, (int)((int64_t)M * K * 2), kBufferWord3);

  // activation chunk j of this thread: row (tid / 8) + 32 j of the tile, k 8 (tid % 8)
  const int part = tid & 7;
  int xvo[kXChunks];
#pragma unroll
  for (int j = 0; j < kXChunks; ++j)
    xvo[j] = (min(m0 + (tid >> 3) + 32 * j, M - 1) * K + 8 * part) * 2;
  int cvo[CN], svo[CN];
#pragma unroll
  for (int c = 0; c < CN; ++c) {
    const int n = min(n0 + 32 * CN * wc + 32 * c + col, N - 1);
    cvo[c] = n * (K >> 1) + 16 * h;
    svo[c] = n * NG * 2;
  }

  // a ring of P groups in flight: slot d holds the loads of groups g = d (mod P)
  u32x4_t xr[P][kXChunks];
  u32x4_t cr[P][CN];
  uint32_t sr[P][CN];
  auto load_x = [&](auto slot, int g) __attribute__((always_inline)) {
    constexpr int d = decltype(slot)::value;
    const int gs = __builtin_amdgcn_readfirstlane(min(g, NG - 1));
#pragma unroll
    for (int j = 0; j < kXChunks; ++j)
      xr[d][j] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xvo[j], 128 * gs, 0);
  };
  auto load_w = [&](auto slot, int g) __attribute__((always_inline)) {
    constexpr int d = decltype(slot)::value;
    const int gs = __builtin_amdgcn_readfirstlane(min(g, NG - 1));
#pragma unroll
    for (int c = 0; c < CN; ++c) {
      cr[d][c] = __builtin_amdgcn_raw_buffer_load_b128(crs, cvo[c], 32 * gs, kLoadStream);
      sr[d][c] = __builtin_amdgcn_raw_buffer_load_b16(srs, svo[c], 2 * gs, 0);
    }
  };

  f32x16_t acc[RM][CN];
#pragma unroll
  for (int r = 0; r < RM; ++r)
#pragma unroll
    for (int c = 0; c < CN; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.f;

  const uint32_t laneoff = 4u * lane;
  // one step: stage group g's activations, refill the slot's activations with
  // group g + P, multiply, refill the slot's codes and scales
  auto step = [&](auto slot, int g) __attribute__((always_inline)) {
    constexpr int d = decltype(slot)::value;
    uint8_t *const xb = xs + (d & 1) * kStage;
    float *const fb = fm + (d & 1) * BM;
#pragma unroll
    for (int j = 0; j < kXChunks; ++j) {
      const u32x4_t v = xr[d][j];
      uint32_t mx = max(max(bf16x2_absmax_bits(v[0]), bf16x2_absmax_bits(v[1])),
                        max(bf16x2_absmax_bits(v[2]), bf16x2_absmax_bits(v[3])));
      mx = max8(mx);
      const int sh = f16_range_shift(mx);
      const int row = (tid >> 3) + 32 * j;
      *reinterpret_cast<uint4 *>(xb + row * kXRow + 16 * part) =
          make_uint4(bf16x2_to_f16x2(v[0], sh), bf16x2_to_f16x2(v[1], sh),
                     bf16x2_to_f16x2(v[2], sh), bf16x2_to_f16x2(v[3], sh));
      if (part == 0) fb[row] = ldexpf(1.0f, -sh);
    }
    __syncthreads();
    load_x(slot, g + P);

    f32x16_t t[RM][CN];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t a[RM], b[CN];
#pragma unroll
      for (int r = 0; r < RM; ++r)
        a[r] = *reinterpret_cast<const u32x4_t *>(xb + (32 * RM * wr + 32 * r + col) * kXRow +
                                                   64 * h + 16 * s);
#pragma unroll
      for (int c = 0; c < CN; ++c) {
        const uint32_t w = cr[d][c][s];
        b[c][0] = lds_load_u32(lut, lut_addr<0>(w, laneoff));
        b[c][1] = lds_load_u32(lut, lut_addr<1>(w, laneoff));
        b[c][2] = lds_load_u32(lut, lut_addr<2>(w, laneoff));
        b[c][3] = lds_load_u32(lut, lut_addr<3>(w, laneoff));
      }
#pragma unroll
      for (int r = 0; r < RM; ++r)
#pragma unroll
        for (int c = 0; c < CN; ++c) {
          f32x16_t z;
          if (s == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) z[i] = 0.f;
          } else {
            z = t[r][c];
          }
          t[r][c] = mfma32(a[r], b[c], z);
        }
    }
    // tile element i of lane (col, h) is row 8 (i / 4) + 4 h + i % 4
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      float f[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v =
            *reinterpret_cast<const float4 *>(fb + 32 * RM * wr + 32 * r + 8 * q + 4 * h);
        f[4 * q + 0] = v.x;
        f[4 * q + 1] = v.y;
        f[4 * q + 2] = v.z;
        f[4 * q + 3] = v.w;
      }
#pragma unroll
      for (int c = 0; c < CN; ++c) {
        const float sc = f16_bits_to_f32(sr[d][c]);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[r][c][i] = fmaf(t[r][c][i], f[i] * sc, acc[r][c][i]);
      }
    }
    load_w(slot, g + P);
    __builtin_amdgcn_sched_barrier(0);  // refills stay after the step that frees the slot
  };

  // (issued in the loop's order: activations, then codes and scales, per group)
  for_slots(
      [&](auto slot) __attribute__((always_inline)) {
        load_x(slot, decltype(slot)::value);
        load_w(slot, decltype(slot)::value);
        __builtin_amdgcn_sched_barrier(0);
      },
      std::make_integer_sequence<int, P>{});
  build_byte_lut(lut, tid, kPThreads);

  int g = 0;
  for (; g + P <= NG; g += P)
    for_slots([&](auto slot) __attribute__((always_inline)) { step(slot, g + decltype(slot)::value); },
              std::make_integer_sequence<int, P>{});
  for_slots(
      [&](auto slot) __attribute__((always_inline)) {
        if (g + decltype(slot)::value < NG) step(slot, g + decltype(slot)::value);
      },
      std::make_integer_sequence<int, P>{});

#pragma unroll
  for (int r = 0; r < RM; ++r)
#pragma unroll
    for (int c = 0; c < CN; ++c) {
      const int n = n0 + 32 * CN * wc + 32 * c + col;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + 32 * RM * wr + 32 * r + 8 * (i >> 2) + 4 * h + (i & 3);
        if (m < M && n < N) Y[(int64_t)m * N + n] = acc[r][c][i];
      }
    }
}

int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

constexpr int kCUs = 256;

template <int RM, int CN>
hipError_t go_prefill(const uint8_t *codes, const uint16_t *scales, int N, int K,
                      const uint16_t *X, int M, float *Y, hipStream_t stream) {
  const dim3 grid(cdiv(N, 64 * CN), cdiv(M, 64 * RM));
  // groups in flight (even: the LDS stage alternates); the 128 x 128 tile has
  // room in registers for two only
  constexpr int P = RM * CN == 4 ? 2 : 4;
  hipLaunchKernelGGL((gemm_prefill_kernel<RM, CN, P>), grid, dim3(kPThreads), 0, stream, codes,
                     scales, X, Y, N, K, M);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_prefill(const uint8_t *codes, const uint16_t *scales, int64_t N,
                               int64_t K, const uint16_t *X, int64_t M, float *Y,
                               hipStream_t stream) {
  const int n = (int)N, k = (int)K, m = (int)M;
  // the largest tile that still gives every CU a workgroup, else the smallest
  // (128 x 64 is never needed: 64 x 128 gives at least as many workgroups)
  auto blocks = [&](int bm, int bn) { return (int64_t)cdiv(n, bn) * cdiv(m, bm); };
  if (blocks(128, 128) >= kCUs) return go_prefill<2, 2>(codes, scales, n, k, X, m, Y, stream);
  if (blocks(64, 128) >= kCUs) return go_prefill<1, 2>(codes, scales, n, k, X, m, Y, stream);
  return go_prefill<1, 1>(codes, scales, n, k, X, m, Y, stream);
}

}  // namespace nf4
