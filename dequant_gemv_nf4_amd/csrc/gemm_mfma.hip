// gemm_mfma.hip -- fused NF4 dequant product for activation batches of up to 32
// rows on the matrix cores (gfx950, v_mfma_f32_16x16x32_bf16).
//
// Computes Y[m][n] = sum_k L[code(n,k)] * s(n,k/64) * X[m][k].  Source:
// deep-fold README, "Method": prefill runs the NF4 product on prompt chunks of up
// to 32 positions, rebuilding weights into matrix-core register fragments.
//
// MFMA mapping (D = A.B + C, 16 x 16 x 32, bf16 operands, fp32 accumulate):
//   A = activations, 16 rows m x 32 k: the bf16 inputs as they are, loaded from
//       memory straight into the fragment (no conversion, no staging);
//   B = decoded weights, 32 k x 16 columns n (one weight row per column);
//   D = Y tile: lane l holds Y[4*(l/16) + r][n0 + l%16], r = 0..3.
// Lane l supplies k-slots 8*(l/16) .. +7 of both A and B.  In scale group q,
// step h (0, 1), the slots of lane-group g are k = 64q + 16g + 8h + e, so a
// lane's 16 weights of a group are one 8-byte load and its 16 activations are
// 32 contiguous bytes.
//
// A level in bf16 alone would be off by up to 2^-9 of itself, so each level is
// split into hi = bf16(L) and lo = bf16(L - hi) (|L - hi - lo| < 2^-17 |L|) and
// each step runs two MFMAs, A.B_hi and A.B_lo, into one group tile.  With exact
// activations every product is exact in fp32.  The group tile is scaled by the
// lane's own column scale in fp32 and added to the accumulator: no weight is
// ever rounded together with its scale.
//
// Decode: a byte table in LDS; entry b holds the (hi pair, lo pair) of b's two
// nibbles, 8 bytes, in 32 copies 8 bytes apart so that lane l reads copy l % 32
// and no two lanes of a half-wave share a bank; the address is one v_perm_b32 of
// the code word.  64 KiB.
//
// Work: a workgroup of 8 waves (one per CU) owns TB consecutive 16-column tiles.
// Wave w takes scale groups w, w+8, w+16, ... of all TB tiles, so one activation
// fragment serves TB tiles and the eight waves read neighbouring 32-byte pieces
// of each weight row together.  A register ring holds the loads of the next D
// groups; every load is unconditional (past-the-end groups and tiles re-read a
// valid address), so waits are exact.  The 8 partial tiles are summed in LDS in
// wave order: deterministic, no atomics.
//
// Every model shape runs one of two step kernels: at M <= 8 the quad-step
// kernel (four groups per step, whole cache lines per load instruction,
// gemm_mfma_quad_kernel), above that the pair-step kernel (two groups per step,
// gemm_mfma_pair_kernel), which with a caller workspace can also split K over
// S workgroups per tile group (blockIdx.y), whose partial tiles meet in the
// workspace and are added in split order by the last to finish (see
// plan_pair for where that pays).
#include <utility>

#include "nf4_device.h"
#include "nf4_launch.h"
#include "nf4_split.h"

namespace nf4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;  // 8 waves
constexpr int kWaves = kThreads / 64;

// Entry b (b = 16 h + j, j = low nibble = even k) at byte 256 b + 8 c, copy c:
//   word 0 = hi[j] | hi[h] << 16,  word 1 = lo[j] | lo[h] << 16.
// Wave w writes the 16 entries of each high nibble h with h % 8 == w: 4096
// contiguous bytes = 256 uint4 (two copies each), 4 per lane; store (i, lane)
// covers entry 16h + 4i + lane/16, so the high level is a constant of the
// unrolled loop and the low level a 4-way choice fixed per lane.
__device__ __forceinline__ void build_split_lut(uint32_t *lut, int lane, int wave) {
  // the 4-way choice as a shift of four packed 16-bit constants (a select chain
  // would be turned into a table in memory)
  const uint32_t sh = 16u * ((uint32_t)lane >> 4);
  uint32_t lhi[4], llo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    constexpr auto pack4 = [](const uint32_t *v) {
      return (uint64_t)v[0] | (uint64_t)v[1] << 16 | (uint64_t)v[2] << 32 | (uint64_t)v[3] << 48;
    };
    lhi[i] = (uint32_t)(pack4(&kSplit.hi[4 * i]) >> sh) & 0xffffu;
    llo[i] = (uint32_t)(pack4(&kSplit.lo[4 * i]) >> sh) & 0xffffu;
  }
  uint4 *L4 = reinterpret_cast<uint4 *>(lut);
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    if (h % kWaves == wave) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t eh = lhi[i] | (kSplit.hi[h] << 16);
        const uint32_t el = llo[i] | (kSplit.lo[h] << 16);
        L4[h * 256 + i * 64 + lane] = make_uint4(eh, el, eh, el);
      }
    }
  }
}

// v_perm_b32 selector: (byte j of the code word) << 8 | (low byte of laneoff)
template <int j>
__device__ __forceinline__ uint32_t split_addr(uint32_t codeword, uint32_t laneoff) {
  constexpr uint32_t sel = 0x0c0c0000u | ((4u + j) << 8);
  return __builtin_amdgcn_perm(codeword, laneoff, sel);
}

__device__ __forceinline__ u32x2_t lds_load_u64(const uint32_t *base, uint32_t byte_addr) {
  return *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const char *>(base) + byte_addr);
}

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_f16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// the wave's largest (Max) or smallest of a 32-bit value, as a scalar
template <bool Max>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
  auto f = [](uint32_t a, uint32_t b) { return Max ? max(a, b) : min(a, b); };
  // (the DPP source of a lane outside the row pattern is never read: every
  // control below pairs lanes within a row of 16)
  v = f(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xf, 0xf, false));
  v = f(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xf, 0xf, false));
  v = f(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xf, 0xf, false));
  v = f(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xf, 0xf, false));
  const uint32_t a = f((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                       (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = f((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                       (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return f(a, b);
}

template <int d>
using Slot = std::integral_constant<int, d>;

// f(Slot<0>{}), f(Slot<1>{}), ... f(Slot<D-1>{}): ring slots as compile-time
// indices, so the ring stays in registers
template <typename F, int... d>
__device__ __forceinline__ void for_slots(F &&f, std::integer_sequence<int, d...>) {
  (f(Slot<d>{}), ...);
}

// MT = 16-row activation tiles (1 for M <= 16, else 2); TB = column tiles per
// workgroup; D = groups in flight per wave.
template <int MT, int TB, int D>
__global__ void __launch_bounds__(kThreads)
    gemm_mfma_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                     const uint16_t *__restrict__ X, float *__restrict__ Y, int N, int K, int M) {
  // one LDS block: the decode table while the groups run, then the partial tiles
  constexpr int kRedWords = kWaves * TB * MT * 4 * 64;
  constexpr int kLdsWords = kRedWords > kLutWords ? kRedWords : kLutWords;
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsWords];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, lg = lane >> 4;
  const int NG = K >> 6;
  const int NT = (N + 15) >> 4;
  const int t0 = blockIdx.x * TB;
  const int nsteps = wave < NG ? (NG - 1 - wave) / kWaves + 1 : 0;

  // per-lane offsets: weight row of column n in each tile (tiles past the end
  // re-read the first tile, columns past N re-read row N-1) and activation row
  uint32_t coff[TB], soff[TB];
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    const int t = (t0 + j < NT) ? t0 + j : t0;
    const uint32_t n = (uint32_t)min(16 * t + col, N - 1);
    coff[j] = n * (uint32_t)(K >> 1) + 8u * lg;
    soff[j] = n * (uint32_t)NG;
  }
  uint32_t xoff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xoff[mt] = (uint32_t)min(16 * mt + col, M - 1) * K + 16u * lg;

  u32x2_t rc[D][TB];
  uint32_t rs[D][TB];
  u32x4_t ra[D][MT][2];

  auto load = [&](auto slot, int i) __attribute__((always_inline)) {
    constexpr int d = decltype(slot)::value;
    const uint32_t q = (uint32_t)min(wave + kWaves * i, NG - 1);
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      rc[d][j] = *reinterpret_cast<const u32x2_t *>(codes + coff[j] + 32u * q);
      rs[d][j] = scales[soff[j] + q];
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4_t *p = reinterpret_cast<const u32x4_t *>(X + xoff[mt] + 64u * q);
      ra[d][mt][0] = p[0];
      ra[d][mt][1] = p[1];
    }
  };

  f32x4_t acc[TB][MT];
#pragma unroll
  for (int j = 0; j < TB; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[j][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint32_t laneoff = 8u * (lane & 31);
  auto compute = [&](auto slot) __attribute__((always_inline)) {
    constexpr int d = decltype(slot)::value;
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      f32x4_t g[MT];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w = rc[d][j][h];
        u32x4_t bh, bl;
        u32x2_t e;
        e = lds_load_u64(lds, split_addr<0>(w, laneoff)); bh[0] = e[0]; bl[0] = e[1];
        e = lds_load_u64(lds, split_addr<1>(w, laneoff)); bh[1] = e[0]; bl[1] = e[1];
        e = lds_load_u64(lds, split_addr<2>(w, laneoff)); bh[2] = e[0]; bl[2] = e[1];
        e = lds_load_u64(lds, split_addr<3>(w, laneoff)); bh[3] = e[0]; bl[3] = e[1];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          g[mt] = mfma_bf16(ra[d][mt][h], bh, h == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : g[mt]);
          g[mt] = mfma_bf16(ra[d][mt][h], bl, g[mt]);
        }
      }
      const float s = f16_bits_to_f32(rs[d][j]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][mt][r] = fmaf(g[mt][r], s, acc[j][mt][r]);
    }
  };

  // prologue: the first D groups in flight while the table is built
  for_slots([&](auto slot) __attribute__((always_inline)) { load(slot, decltype(slot)::value); },
            std::make_integer_sequence<int, D>{});
  build_split_lut(lds, lane, wave);
  __syncthreads();

  for (int base = 0; base < nsteps; base += D) {
    for_slots(
        [&](auto slot) __attribute__((always_inline)) {
          constexpr int d = decltype(slot)::value;
          if (base + d < nsteps) compute(slot);
          load(slot, base + d + D);
        },
        std::make_integer_sequence<int, D>{});
  }

  // partial tiles of the 8 waves, summed in wave order
  __syncthreads();  // the table is no longer read
  float *red = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int j = 0; j < TB; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[(((wave * TB + j) * MT + mt) * 4 + r) * 64 + lane] = acc[j][mt][r];
  __syncthreads();
  constexpr int kOut = TB * MT * 256;  // outputs per workgroup
  for (int o = tid; o < kOut; o += kThreads) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += red[w * kOut + o];
    const int ln = o & 63, r = (o >> 6) & 3, tm = o >> 8;
    const int mt = tm % MT, j = tm / MT;
    const int m = 16 * mt + 4 * (ln >> 4) + r;
    const int n = 16 * (t0 + j) + (ln & 15);
    if (t0 + j < NT && m < M && n < N) Y[(int64_t)m * N + n] = s;
  }
}

// ---------------------------------------------------------------------------
// Pair-step variant (an even number of groups per row and 4-byte aligned
// scales, which covers every model shape): a step is a pair of groups (128 k,
// 64 code bytes per row).  A lane loads 16 contiguous code bytes of its row --
// lane-group g takes bytes 16g .. 16g+15 of the pair, so one wave instruction
// reads 64 contiguous bytes of each of 16 rows -- and one 32-bit word holding
// both scales of the pair.  Lane-groups 0/1 then hold bytes of the first group
// and 2/3 of the second; one v_permlane32_swap per half (lanes l <-> l + 32)
// leaves every lane with 8 bytes of each group: byte offset pi(g) = 0, 16, 8,
// 24 for g = 0..3 within the group, the same in both groups, so each MFMA still
// covers one group and its tile is scaled by that group's scale.  Every load is
// a buffer load whose per-lane offset is fixed and whose step offset is a
// scalar: no vector address arithmetic per step.
// ---------------------------------------------------------------------------
template <int MT, int TB, int D>
__global__ void __launch_bounds__(kThreads)
    gemm_mfma_pair_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                          const uint16_t *__restrict__ X, float *__restrict__ Y, int N, int K,
                          int M, int S, uint32_t *__restrict__ cnt) {
  constexpr int kRedWords = kWaves * TB * MT * 4 * 64;
  constexpr int kLdsWords = kRedWords > kLutWords ? kRedWords : kLutWords;
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsWords];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, lg = lane >> 4;
  const int NG = K >> 6;
  const int NP = NG >> 1;  // pairs per row
  const int NT = (N + 15) >> 4;
  const int t0 = blockIdx.x * TB;
  // the workspace: the counter area, then the partial tiles (the address is
  // derived here, so that every argument fits the preloaded argument registers)
  float *const part =
      S > 1 ? reinterpret_cast<float *>(reinterpret_cast<char *>(cnt) + kSplitCounterBytes)
            : nullptr;
  // K-split blockIdx.y of S takes the pair steps [p0, p0 + np)
  const int split = blockIdx.y;
  const int p0 = (int)((int64_t)split * NP / S);
  const int np = (int)((int64_t)(split + 1) * NP / S) - p0;
  const int nsteps = wave < np ? (np - 1 - wave) / kWaves + 1 : 0;

  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(codes), 0, (int)((int64_t)N * (K >> 1)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(scales), 0, (int)((int64_t)N * NG * 2), kBufferWord3);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(X), 0, M * K * 2, kBufferWord3);

  // fixed per-lane byte offsets; tiles past the end re-read the first tile,
  // columns past N re-read row N-1
  int cvo[TB], svo[TB];
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    const int t = (t0 + j < NT) ? t0 + j : t0;
    const int n = min(16 * t + col, N - 1);
    cvo[j] = n * (K >> 1) + 16 * lg;
    svo[j] = n * NG * 2;
  }
  // activations of lane-group g after the swap: k = 128 p + 64 q + 2 pi(g) + 8 h + e
  const int pi2 = 2 * ((lg & 1) * 16 + (lg >> 1) * 8);  // 2 pi(g): 0, 32, 16, 48
  int xvo[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xvo[mt] = (min(16 * mt + col, M - 1) * K + pi2) * 2;

  u32x4_t rc[D][TB];
  uint32_t rs[D][TB];
  u32x4_t ra[D][MT][4];  // [group q][half h] -> index 2q + h

  auto load = [&](auto slot, int i) __attribute__((always_inline)) {
    constexpr int d = decltype(slot)::value;
    const int p = __builtin_amdgcn_readfirstlane(p0 + min(wave + kWaves * i, np - 1));
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      rc[d][j] = __builtin_amdgcn_raw_buffer_load_b128(crs, cvo[j], 64 * p, kLoadStream);
      rs[d][j] = __builtin_amdgcn_raw_buffer_load_b32(srs, svo[j], 4 * p, 0);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          ra[d][mt][2 * q + h] =
              __builtin_amdgcn_raw_buffer_load_b128(xrs, xvo[mt] + 128 * q + 16 * h, 256 * p, 0);
  };

  f32x4_t acc[TB][MT];
#pragma unroll
  for (int j = 0; j < TB; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[j][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint32_t laneoff = 8u * (lane & 31);
  auto compute = [&](auto slot) __attribute__((always_inline)) {
    constexpr int d = decltype(slot)::value;
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      // lanes l and l + 32 trade halves: afterwards words 0, 1 hold the first
      // group's bytes and words 2, 3 the second's
      const u32x4_t c = rc[d][j];
      const auto s02 = __builtin_amdgcn_permlane32_swap(c[0], c[2], false, false);
      const auto s13 = __builtin_amdgcn_permlane32_swap(c[1], c[3], false, false);
      const uint32_t wq[2][2] = {{s02[0], s13[0]}, {s02[1], s13[1]}};
      const uint32_t sw = rs[d][j];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        f32x4_t g[MT];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t w = wq[q][h];
          u32x4_t bh, bl;
          u32x2_t e;
          e = lds_load_u64(lds, split_addr<0>(w, laneoff)); bh[0] = e[0]; bl[0] = e[1];
          e = lds_load_u64(lds, split_addr<1>(w, laneoff)); bh[1] = e[0]; bl[1] = e[1];
          e = lds_load_u64(lds, split_addr<2>(w, laneoff)); bh[2] = e[0]; bl[2] = e[1];
          e = lds_load_u64(lds, split_addr<3>(w, laneoff)); bh[3] = e[0]; bl[3] = e[1];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const u32x4_t a = ra[d][mt][2 * q + h];
            g[mt] = mfma_bf16(a, bh, h == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : g[mt]);
            g[mt] = mfma_bf16(a, bl, g[mt]);
          }
        }
        const float sc = f16_bits_to_f32(q == 0 ? (sw & 0xffffu) : (sw >> 16));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[j][mt][r] = fmaf(g[mt][r], sc, acc[j][mt][r]);
      }
    }
  };

  // (slots issued in the loop's order, so the waits agree on both paths into it)
  for_slots(
      [&](auto slot) __attribute__((always_inline)) {
        load(slot, decltype(slot)::value);
        __builtin_amdgcn_sched_barrier(0);
      },
      std::make_integer_sequence<int, D>{});
  build_split_lut(lds, lane, wave);
  __syncthreads();

  // whole rounds without branches, then the last partial round
  int base = 0;
  for (; base + D <= nsteps; base += D) {
    for_slots(
        [&](auto slot) __attribute__((always_inline)) {
          constexpr int d = decltype(slot)::value;
          compute(slot);
          // with one pair in flight and up to two tiles, no refill after the
          // wave's last pair: the spare load would hold the wave at its end for
          // one more memory round trip, and the wait before each pair is for
          // every load in flight anyway (with more tiles the branch costs
          // registers: spills at 7 tiles of two row tiles)
          if (D > 1 || TB > 2 || base + d + D < nsteps) load(slot, base + d + D);
          // keep each slot's refill right after its use (the scheduler would
          // otherwise sink all refills to the end of the round)
          __builtin_amdgcn_sched_barrier(0);
        },
        std::make_integer_sequence<int, D>{});
  }
  for_slots(
      [&](auto slot) __attribute__((always_inline)) {
        constexpr int d = decltype(slot)::value;
        if (base + d < nsteps) compute(slot);
      },
      std::make_integer_sequence<int, D>{});

  __syncthreads();  // the table is no longer read
  float *red = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int j = 0; j < TB; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[(((wave * TB + j) * MT + mt) * 4 + r) * 64 + lane] = acc[j][mt][r];
  __syncthreads();
  constexpr int kOut = TB * MT * 256;
  auto store = [&](int o, float v) __attribute__((always_inline)) {
    const int ln = o & 63, r = (o >> 6) & 3, tm = o >> 8;
    const int mt = tm % MT, j = tm / MT;
    const int m = 16 * mt + 4 * (ln >> 4) + r;
    const int n = 16 * (t0 + j) + (ln & 15);
    if (t0 + j < NT && m < M && n < N) Y[(int64_t)m * N + n] = v;
  };
  float *const mine = S > 1 ? part + ((int64_t)blockIdx.x * S + split) * kOut : nullptr;
  for (int o = tid; o < kOut; o += kThreads) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += red[w * kOut + o];
    if (S == 1)
      store(o, sum);
    else  // agent-coherent store: straight to the point all XCDs see
      __hip_atomic_store(mine + o, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (S == 1) return;
  // K-splits: the last split of this tile group to finish adds all S partial
  // tiles in split order (the same bits whichever finishes last) and re-arms the
  // group's counter for the next call.  Ordering (the AMDGPU memory model's
  // release/acquire sequences, restricted to the locations involved): partials
  // are written with agent-scope atomic stores, performed at the agent's
  // coherence point and not held in one XCD's L2, so publishing them needs no L2
  // write-back; vmcnt(0) waits until each thread's stores are performed, and
  // the barrier orders those waits before the counter increment.  Only the
  // workgroup that saw the final count reads them, with agent-scope atomic
  // loads that also go to the coherence point (no stale L2 line can answer, so
  // no invalidate is needed), issued after the increment returned.
  __shared__ int last;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's partial stores are done
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(cnt + blockIdx.x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == (uint32_t)(S - 1);
    if (last) __hip_atomic_store(cnt + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last) return;
  const float *const all = part + (int64_t)blockIdx.x * S * kOut;
  for (int o = tid; o < kOut; o += kThreads) {
    float sum = __hip_atomic_load(all + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int q = 1; q < S; ++q)
      sum += __hip_atomic_load(all + (int64_t)q * kOut + o, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    store(o, sum);
  }
}

// ---------------------------------------------------------------------------
// Quad-step variant for M <= 8 (a multiple of four groups per row and 8-byte
// aligned scales): a step is four groups (256 k, 128 code bytes = one cache
// line per row).  The memory pipeline's cost grows with the cache lines one
// load instruction touches, so every code load covers whole lines: instruction
// 0 reads rows 0..7 of a tile and instruction 1 rows 8..15, eight lanes per
// row, 16 bytes each.  Lane (n, g) -- column n = lane % 16, lane-group
// g = lane / 16, half a = n / 8 -- reads chunk g + 4a of row n % 8 and chunk
// g + 4(1 - a) of row 8 + n % 8: one 16-byte chunk of its own row (chunk g) and
// one of its partner's, lane n +- 8 of the same 16-lane row.  One DPP row
// rotation by 8 trades the partner chunks (each lane then holds chunks g and
// g + 4 of its own row), and one v_permlane32_swap per word pair (lane-groups g
// and g + 2) leaves every lane with 8 bytes of each of the four groups, at byte
// offset 16 (g & 1) + 8 (g >> 1) within the group (the pair step's offsets).
// The four scales of a row's step are one 8-byte load.
//
// Activations: rows 8..15 of the 16-row tile are padding at M <= 8, so lanes of
// half a = 1 load the second half (h = 1) of the same line of row n % 8 and one
// DPP row rotation hands it to lane n - 8: one instruction per group covers 8
// rows x 128 bytes.  (The padding rows' fragments are whatever arrives; their
// outputs are never stored.)
//
// Work: wave w of the workgroup takes a contiguous range of the steps; no
// K-splits.  Kernel trace of the Llama-3.1-8B shapes at M = 8 (graph replay),
// pair step -> quad step: q|k|v 6144 x 4096 10.5 -> 9.8 us, o 4096 x 4096
// 7.6 -> 7.4, gate|up 28672 x 4096 29.6 -> 27.2, down 4096 x 14336 16.8 -> 15.2.
// ---------------------------------------------------------------------------
template <int TB>
__global__ void __launch_bounds__(kThreads)
    gemm_mfma_quad_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                          const uint16_t *__restrict__ X, float *__restrict__ Y, int N, int K,
                          int M) {
  constexpr int kRedWords = kWaves * TB * 4 * 64;
  constexpr int kLdsWords = kRedWords > kLutWords ? kRedWords : kLutWords;
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsWords];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, lg = lane >> 4;
  const bool upper = col >= 8;  // half a = 1 of the 16-lane row
  const int m8 = col & 7;
  const int NG = K >> 6;
  const int NQ = NG >> 2;  // steps per row
  const int NT = (N + 15) >> 4;
  const int t0 = blockIdx.x * TB;
  // wave w takes the steps [wq0, wq0 + wn)
  const int wq0 = wave * NQ / kWaves;
  const int wn = (wave + 1) * NQ / kWaves - wq0;

  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(codes), 0, (int)((int64_t)N * (K >> 1)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(scales), 0, (int)((int64_t)N * NG * 2), kBufferWord3);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(X), 0, M * K * 2, kBufferWord3);

  // fixed per-lane byte offsets; tiles past the end re-read the first tile,
  // rows past N re-read row N-1 (both lanes of a chunk pair clamp alike)
  int cv0[TB], cv1[TB], svo[TB];
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    const int t = (t0 + j < NT) ? t0 + j : t0;
    const int r0 = min(16 * t + m8, N - 1), r1 = min(16 * t + 8 + m8, N - 1);
    cv0[j] = r0 * (K >> 1) + 16 * (lg + (upper ? 4 : 0));
    cv1[j] = r1 * (K >> 1) + 16 * (lg + (upper ? 0 : 4));
    svo[j] = min(16 * t + col, N - 1) * NG * 2;
  }
  // activations: row n % 8, the lane-group's 32 bytes of each group
  // (2 * (16 (g & 1) + 8 (g >> 1)) bytes in), half a of them
  const int xvo = (min(m8, M - 1) * K) * 2 + 64 * (lg & 1) + 32 * (lg >> 1) + (upper ? 16 : 0);

  u32x4_t rc0[TB], rc1[TB], ra[4];
  u32x2_t rs[TB];

  auto load = [&](int i) __attribute__((always_inline)) {
    const int q = __builtin_amdgcn_readfirstlane(max(min(wq0 + min(i, wn - 1), NQ - 1), 0));
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      rc0[j] = __builtin_amdgcn_raw_buffer_load_b128(crs, cv0[j], 128 * q, kLoadStream);
      rc1[j] = __builtin_amdgcn_raw_buffer_load_b128(crs, cv1[j], 128 * q, kLoadStream);
      rs[j] = __builtin_amdgcn_raw_buffer_load_b64(srs, svo[j], 8 * q, 0);
    }
#pragma unroll
    for (int gq = 0; gq < 4; ++gq)
      ra[gq] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xvo + 128 * gq, 512 * q, 0);
  };

  f32x4_t acc[TB];
#pragma unroll
  for (int j = 0; j < TB; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint32_t laneoff = 8u * (lane & 31);
  auto compute = [&]() __attribute__((always_inline)) {
    // activation fragments [group][half]: own load, then the partner's
    u32x4_t A[4][2];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      A[gq][0] = ra[gq];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        A[gq][1][e] = (uint32_t)__builtin_amdgcn_mov_dpp((int)ra[gq][e], 0x128, 0xf, 0xf, false);
    }
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      // own chunk g and, from lane n +- 8, chunk g + 4 of this lane's row
      uint32_t r[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t own = upper ? rc1[j][e] : rc0[j][e];
        const uint32_t out = upper ? rc0[j][e] : rc1[j][e];
        r[e] = own;
        r[4 + e] = (uint32_t)__builtin_amdgcn_mov_dpp((int)out, 0x128, 0xf, 0xf, false);
      }
      // lane-groups g and g + 2 trade words 2, 3 of each chunk for words 0, 1:
      // afterwards words 2q, 2q + 1 hold group q
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const auto lo = __builtin_amdgcn_permlane32_swap(r[e], r[2 + e], false, false);
        r[e] = lo[0];
        r[2 + e] = lo[1];
        const auto hi = __builtin_amdgcn_permlane32_swap(r[4 + e], r[6 + e], false, false);
        r[4 + e] = hi[0];
        r[6 + e] = hi[1];
      }
      const u32x2_t sw = rs[j];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        f32x4_t g;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t w = r[2 * gq + h];
          u32x4_t bh, bl;
          u32x2_t e;
          e = lds_load_u64(lds, split_addr<0>(w, laneoff)); bh[0] = e[0]; bl[0] = e[1];
          e = lds_load_u64(lds, split_addr<1>(w, laneoff)); bh[1] = e[0]; bl[1] = e[1];
          e = lds_load_u64(lds, split_addr<2>(w, laneoff)); bh[2] = e[0]; bl[2] = e[1];
          e = lds_load_u64(lds, split_addr<3>(w, laneoff)); bh[3] = e[0]; bl[3] = e[1];
          g = mfma_bf16(A[gq][h], bh, h == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : g);
          g = mfma_bf16(A[gq][h], bl, g);
        }
        const uint32_t sword = sw[gq >> 1];
        const float sc = f16_bits_to_f32((gq & 1) ? (sword >> 16) : (sword & 0xffffu));
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) acc[j][rr] = fmaf(g[rr], sc, acc[j][rr]);
      }
      // one tile at a time: interleaving tiles only raises register pressure
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  load(0);
  __builtin_amdgcn_sched_barrier(0);
  build_split_lut(lds, lane, wave);
  __syncthreads();
  // one step in flight per wave: the refill follows the step's use.  Up to two
  // tiles, no load goes out after the wave's last step: a spare load would still
  // be waited for before the reduction (one more memory round trip; o 4096 x
  // 4096 at M = 8: 7.2 -> 6.2 us without it).  The wait before each step is for
  // every load in flight either way, so the branch costs no overlap.  (At 3 and
  // 4 tiles the branch raises the register count past two workgroups per CU;
  // those shapes, K above 8192 with more than 512 tiles, keep the spare load.)
  for (int i = 0; i < wn; ++i) {
    compute();
    if (TB > 2 || i + 1 < wn) load(i + 1);
    __builtin_amdgcn_sched_barrier(0);
  }

  __syncthreads();  // the table is no longer read
  float *red = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int j = 0; j < TB; ++j)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) red[((wave * TB + j) * 4 + rr) * 64 + lane] = acc[j][rr];
  __syncthreads();
  constexpr int kOut = TB * 256;
  for (int o = tid; o < kOut; o += kThreads) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += red[w * kOut + o];
    const int ln = o & 63, rr = (o >> 6) & 3, j = o >> 8;
    const int m = 4 * (ln >> 4) + rr;
    const int n = 16 * (t0 + j) + (ln & 15);
    if (t0 + j < NT && m < M && n < N) Y[(int64_t)m * N + n] = sum;
  }
}

// ---------------------------------------------------------------------------
// Streaming form of the quad step for more column tiles than CUs, M <= 32
// (gemm_mfma_stream_kernel).  MR = 8 (M <= 8) keeps the quad step's activation
// loads (rows 8..15 of the tile are padding); MR = 16 and 32 load one or two
// full 16-row activation tiles, both halves of each fragment.  One workgroup of 8 waves per CU walks IT tiles,
// tile t*nblocks + b, so the whole grid streams one band of rows at a time.  A
// wave owns the same steps of K, [q0, q0 + ns), in every tile: its activation
// fragments (both halves) are loaded once and stay in registers, instead of
// being read again from L2 for every tile, and the code and scale loads of two
// tiles are in flight per wave.  Each tile has its own accumulator; after the
// last tile the eight partials of a tile are added in LDS in slice order
// (deterministic, and the same sums in the same order as the quad-step
// kernel, so both give identical bits).  The slices are rotated by the
// workgroup index so that the CUs do not all read the same activation lines at
// the same moment (q|k|v 6144 x 4096 at M = 8: 10.2 -> 9.4 us).  Llama-3.1-8B
// gate|up (28672 x 4096) at M = 8: 26.0 -> 19 us against the quad step.
// ---------------------------------------------------------------------------
template <int MR, int NS, int IT, bool SW, bool F16>
__global__ void __launch_bounds__(kThreads)
    gemm_mfma_stream_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                            const uint16_t *__restrict__ X, float *__restrict__ Y, int N, int K,
                            int M, int nblocks, int S, uint32_t *__restrict__ cnt) {
  // MR = 8: rows 8..15 of the 16-row tile are padding (the quad step's
  // activation loads); MR = 16 or 32: one or two full 16-row tiles
  constexpr int MT = MR == 32 ? 2 : 1;
  constexpr int kRedWords = kWaves * IT * MT * 256;
  constexpr int kLdsWords = kRedWords > kLutWords ? kRedWords : kLutWords;
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsWords];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, lg = lane >> 4;
  const bool upper = col >= 8;
  const int m8 = col & 7;
  const int NG = K >> 6;
  const int NQ = NG >> 2;
  const int NT = (N + 15) >> 4;
  // K-split blockIdx.y of S takes the steps [p0, p0 + np); its waves share them
  const int split = blockIdx.y;
  const int p0 = split * NQ / S;
  const int np = (split + 1) * NQ / S - p0;
  const int slice = (wave + (int)blockIdx.x) & (kWaves - 1);
  const int q0 = p0 + slice * np / kWaves;
  const int ns = p0 + (slice + 1) * np / kWaves - q0;  // 0 <= ns <= NS
  float *const part =
      S > 1 ? reinterpret_cast<float *>(reinterpret_cast<char *>(cnt) + kSplitCounterBytes)
            : nullptr;

  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(codes), 0, (int)((int64_t)N * (K >> 1)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(scales), 0, (int)((int64_t)N * NG * 2), kBufferWord3);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(X), 0, M * K * 2, kBufferWord3);

  // per-lane offsets within a tile starting at row 0 (the quad step's chunk
  // assignment); the tile's row offset and the step's offset are scalars
  const int cv0 = m8 * (K >> 1) + 16 * (lg + (upper ? 4 : 0));
  const int cv1 = (8 + m8) * (K >> 1) + 16 * (lg + (upper ? 0 : 4));
  const int svo = col * NG * 2;
  // activations of lane-group g in group q of a step: k = 64 q + 32 (g & 1) +
  // 16 (g >> 1) + 8 h + e, the offsets the exchange leaves the weights at
  int xvo[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    xvo[mt] = MR == 8 ? (min(m8, M - 1) * K) * 2 + 64 * (lg & 1) + 32 * (lg >> 1) + (upper ? 16 : 0)
                      : (min(16 * mt + col, M - 1) * K) * 2 + 64 * (lg & 1) + 32 * (lg >> 1);

  // step of register slot s (slots past the slice re-read its last step)
  auto step_of = [&](int s) {
    return __builtin_amdgcn_readfirstlane(max(min(q0 + min(s, ns - 1), NQ - 1), 0));
  };
  // first row of tile t of this workgroup: a last, partial tile is moved back to
  // end at row N - 1 (its rows below 16 * tile belong to the tile before and are
  // not stored), and tiles past the end re-read the last one
  auto tile_row = [&](int t) {
    const int tile = min(t * nblocks + (int)blockIdx.x, NT - 1);
    return __builtin_amdgcn_readfirstlane(min(16 * tile, N - 16));
  };

  u32x4_t A[NS][MT][4][2];  // [step][row tile][group][half]
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int q = step_of(s);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
#pragma unroll
        for (int h = 0; h < (MR == 8 ? 1 : 2); ++h)
          A[s][mt][gq][h] =
              __builtin_amdgcn_raw_buffer_load_b128(xrs, xvo[mt] + 128 * gq + 16 * h, 512 * q, 0);
  }

  uint32_t wide = 0;  // bit 4 s + gq: group gq of slot s is added exactly (below)
  float gfac[NS][4];  // 2^(Emax - 141): undoes the group's f16 shift

  constexpr int kRing = IT < 2 ? IT : 2;  // tiles in flight
  u32x4_t rc[kRing][NS][2];
  // scales: one 8-byte load per step, or (SW: every wave of the launch owns
  // exactly NS steps, NS even) one 16-byte load per two steps.  A load touches
  // the 16 rows' lines either way, and the memory pipeline's cost follows the
  // lines an instruction touches, so SW halves the cost of the scales.
  constexpr int kScaleLoads = SW ? NS / 2 : NS;
  u32x2_t rs[kRing][NS];
  u32x4_t rsw[kRing][SW ? NS / 2 : 1];
  auto load_tile = [&](auto slot, int t) __attribute__((always_inline)) {
    constexpr int d = decltype(slot)::value;
    const int tb = tile_row(t);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int q = step_of(s);
      const int coff = tb * (K >> 1) + 128 * q;
      rc[d][s][0] = __builtin_amdgcn_raw_buffer_load_b128(crs, cv0, coff, kLoadStream);
      rc[d][s][1] = __builtin_amdgcn_raw_buffer_load_b128(crs, cv1, coff, kLoadStream);
      if constexpr (!SW) rs[d][s] = __builtin_amdgcn_raw_buffer_load_b64(srs, svo, tb * NG * 2 + 8 * q, 0);
    }
    if constexpr (SW) {
#pragma unroll
      for (int j = 0; j < kScaleLoads; ++j)
        rsw[d][j] = __builtin_amdgcn_raw_buffer_load_b128(srs, svo, tb * NG * 2 + 8 * (q0 + 2 * j), 0);
    }
  };

  f32x4_t acc[IT][MT];
#pragma unroll
  for (int t = 0; t < IT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // table lane offsets: copy lane % 32 of 4-byte f16-pair entries (F16) or of
  // 8-byte (hi pair, lo pair) entries
  const uint32_t laneoff = F16 ? lut_lane_offset(lane) : 8u * (lane & 31);
  auto compute = [&](auto slot, f32x4_t (&ac)[MT]) __attribute__((always_inline)) {
    constexpr int d = decltype(slot)::value;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s >= ns) break;
      // the quad step's exchange: own chunk and the partner's, then lane-groups
      // g and g + 2 trade words so that words 2q, 2q + 1 hold group q
      uint32_t r[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t own = upper ? rc[d][s][1][e] : rc[d][s][0][e];
        const uint32_t out = upper ? rc[d][s][0][e] : rc[d][s][1][e];
        r[e] = own;
        r[4 + e] = (uint32_t)__builtin_amdgcn_mov_dpp((int)out, 0x128, 0xf, 0xf, false);
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const auto lo = __builtin_amdgcn_permlane32_swap(r[e], r[2 + e], false, false);
        r[e] = lo[0];
        r[2 + e] = lo[1];
        const auto hi = __builtin_amdgcn_permlane32_swap(r[4 + e], r[6 + e], false, false);
        r[4 + e] = hi[0];
        r[6 + e] = hi[1];
      }
      u32x2_t sw;
      if constexpr (SW) {
        sw[0] = rsw[d][s >> 1][2 * (s & 1)];
        sw[1] = rsw[d][s >> 1][2 * (s & 1) + 1];
      } else {
        sw = rs[d][s];
      }
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        f32x4_t g[MT];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t w = r[2 * gq + h];
          if constexpr (F16) {
            const u32x4_t b = {lds_load_u32(lds, lut_addr<0>(w, laneoff)),
                               lds_load_u32(lds, lut_addr<1>(w, laneoff)),
                               lds_load_u32(lds, lut_addr<2>(w, laneoff)),
                               lds_load_u32(lds, lut_addr<3>(w, laneoff))};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              g[mt] = mfma_f16(A[s][mt][gq][h], b, h == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : g[mt]);
          } else {
            u32x4_t bh, bl;
            u32x2_t e;
            e = lds_load_u64(lds, split_addr<0>(w, laneoff)); bh[0] = e[0]; bl[0] = e[1];
            e = lds_load_u64(lds, split_addr<1>(w, laneoff)); bh[1] = e[0]; bl[1] = e[1];
            e = lds_load_u64(lds, split_addr<2>(w, laneoff)); bh[2] = e[0]; bl[2] = e[1];
            e = lds_load_u64(lds, split_addr<3>(w, laneoff)); bh[3] = e[0]; bl[3] = e[1];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              g[mt] = mfma_bf16(A[s][mt][gq][h], bh, h == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : g[mt]);
              g[mt] = mfma_bf16(A[s][mt][gq][h], bl, g[mt]);
            }
          }
        }
        const uint32_t sword = sw[gq >> 1];
        float sc = f16_bits_to_f32((gq & 1) ? (sword >> 16) : (sword & 0xffffu));
        if constexpr (F16) sc *= gfac[s][gq];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) ac[mt][rr] = fmaf(g[mt][rr], sc, ac[mt][rr]);
      }
    }
  };

  load_tile(Slot<0>{}, 0);
  if constexpr (IT > 1) load_tile(Slot<1>{}, 1);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (F16)
    build_byte_lut(lds, tid, kThreads);
  else
    build_split_lut(lds, lane, wave);
  // F16: activations to f16, one power-of-two shift per group of 64 k shared by all
  // rows: the group's largest |x| (a max over the whole wave, which holds every
  // row of the group) goes to [2^14, 2^15), on the bit patterns (subtract
  // (Emax - 29) << 7 from each bf16 magnitude, saturating, and shift left by 3
  // into the f16 fields).  Exact unless a non-zero value lands below the f16
  // normals (more than 2^28 under the largest) or the largest is under 2^-98:
  // such a group is flagged, its tiles are multiplied by 0 instead of undoing
  // the shift (the staged values are finite: the largest f16 exponent field is
  // 29), and its terms are added exactly after the tiles.  Otherwise the shift
  // is undone, with the column's scale, on the group's fp32 tile.
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      if constexpr (!F16) continue;
      // the group's largest magnitude and its smallest non-zero one, less 1
      // (zero wraps to 0xffff), as bf16 bit patterns
      u16x2 pm = {0, 0}, pn = {0xffff, 0xffff};
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int h = 0; h < (MR == 8 ? 1 : 2); ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const u16x2 mag = __builtin_bit_cast(u16x2, A[s][mt][gq][h][e] & 0x7fff7fffu);
            pm = __builtin_elementwise_max(pm, mag);
            pn = __builtin_elementwise_min(pn, mag - (u16x2){1, 1});
          }
      const uint32_t mx = wave_reduce_u32<true>(max((uint32_t)pm[0], (uint32_t)pm[1]));
      const uint32_t mnm1 = wave_reduce_u32<false>(min((uint32_t)pn[0], (uint32_t)pn[1]));
      const uint32_t emax = mx >> 7;
      const uint32_t bias = ((emax - 29u) << 7) & 0xffffu;
      const u16x2 bias2 = __builtin_bit_cast(u16x2, bias * 0x10001u);
      // lost: a non-zero magnitude at or below bias + 0x7f (an exponent field of
      // 0 or less after the subtraction)
      const bool gw = mx != 0 && (emax < 29u || mnm1 < bias + 0x7fu);
      wide |= gw ? 1u << (4 * s + gq) : 0u;
      gfac[s][gq] = gw || mx == 0 ? 0.0f : __uint_as_float((emax - 14u) << 23);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int h = 0; h < (MR == 8 ? 1 : 2); ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w = A[s][mt][gq][h][e];
            const u16x2 mag = __builtin_bit_cast(u16x2, w & 0x7fff7fffu);
            const uint32_t f = __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(mag, bias2)
                                                                << (u16x2){3, 3}) |
                               (w & 0x80008000u);
            A[s][mt][gq][h][e] = f;
          }
      __builtin_amdgcn_sched_barrier(0);  // one group at a time (registers)
    }
  // MR = 8: the second half of each activation fragment comes from lane n +- 8
  // of the row, which loaded it (a DPP row rotation by 8)
  if constexpr (MR == 8) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          A[s][0][gq][1][e] =
              (uint32_t)__builtin_amdgcn_mov_dpp((int)A[s][0][gq][0][e], 0x128, 0xf, 0xf, false);
  }
  __syncthreads();
  // tiles unrolled, so the ring slots are compile-time registers and no load
  // goes out past the last tile
  [&]<int... t>(std::integer_sequence<int, t...>) {
    (
        [&] {
          compute(Slot<t % kRing>{}, acc[t]);
          if constexpr (t + kRing < IT) load_tile(Slot<t % kRing>{}, t + kRing);
          __builtin_amdgcn_sched_barrier(0);
        }(),
        ...);
  }(std::make_integer_sequence<int, IT>{});

  __syncthreads();  // the table is no longer read
  float *red = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int t = 0; t < IT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        red[(((slice * IT + t) * MT + mt) * 4 + rr) * 64 + lane] = acc[t][mt][rr];
  // ---- exact pass for the groups f16 could not hold (only in waves that have
  // one; about 1e-8 of the groups of N(0, 1) data).  The row loop added nothing
  // for such a group.  Lane (n, g) adds to its own partials in LDS, for column n
  // of each tile and its rows 4 g + rr of each row tile, every term of the group
  // as (fp32 level x fp32 scale) x bf16 activation with one fp32 fma: each term
  // rounded once, no partial sum formed before the scale is applied.
  if (F16 && wide != 0) {
#pragma unroll 1
    for (int sg = 0; sg < 4 * NS; ++sg) {
      if ((wide >> sg & 1u) == 0 || (sg >> 2) >= ns) continue;
      const int G = 4 * step_of(sg >> 2) + (sg & 3);  // the group's index along K
#pragma unroll 1
      for (int t = 0; t < IT; ++t) {
        const int n = tile_row(t) + col;
        const uint8_t *cp = codes + (int64_t)n * (K >> 1) + 32 * G;
        const float sc = f16_bits_to_f32(scales[(int64_t)n * NG + G]);
#pragma unroll 1
        for (int mr = 0; mr < 4 * MT; ++mr) {
          const int m = 16 * (mr >> 2) + 4 * lg + (mr & 3);
          if (m >= M || (MR == 8 && m >= 8)) continue;
          const uint16_t *xr = X + (int64_t)m * K + 64 * G;
          float *slot = red + ((((slice * IT + t) * MT + (mr >> 2)) * 4 + (mr & 3)) * 64 + lane);
          float v = *slot;
#pragma unroll 1
          for (int j = 0; j < 32; ++j) {
            const uint32_t byte = cp[j];
            const uint32_t xw = *reinterpret_cast<const uint32_t *>(xr + 2 * j);
            v = fmaf(level_f32(byte & 15u) * sc, bf16_lo(xw), v);
            v = fmaf(level_f32(byte >> 4) * sc, bf16_hi(xw), v);
          }
          *slot = v;
        }
      }
    }
  }
  __syncthreads();
  constexpr int kOut = IT * MT * 256;
  auto store = [&](int o, float v) __attribute__((always_inline)) {
    const int ln = o & 63, rr = (o >> 6) & 3, tm = o >> 8;
    const int t = tm / MT, mt = tm % MT;
    const int tile = t * nblocks + (int)blockIdx.x;
    const int m = 16 * mt + 4 * (ln >> 4) + rr;
    const int n = min(16 * tile, N - 16) + (ln & 15);
    if (tile < NT && m < M && n >= 16 * tile && n < N) Y[(int64_t)m * N + n] = v;
  };
  float *const mine = S > 1 ? part + ((int64_t)blockIdx.x * S + split) * kOut : nullptr;
  for (int o = tid; o < kOut; o += kThreads) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += red[w * kOut + o];
    if (S == 1)
      store(o, sum);
    else  // agent-coherent store: straight to the point all XCDs see
      __hip_atomic_store(mine + o, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (S == 1) return;
  // K-splits: the last split of this workgroup's tiles to finish adds the S
  // partials in split order and re-arms the counter (the ordering argument of
  // the pair-step kernel's splits: agent-scope atomic stores and loads at the
  // coherence point, vmcnt(0) and the barrier before the increment, loads only
  // after it returned the final count)
  __shared__ int last;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's partial stores are done
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(cnt + blockIdx.x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == (uint32_t)(S - 1);
    if (last) __hip_atomic_store(cnt + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last) return;
  const float *const all = part + (int64_t)blockIdx.x * S * kOut;
  for (int o = tid; o < kOut; o += kThreads) {
    float sum = __hip_atomic_load(all + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int q = 1; q < S; ++q)
      sum += __hip_atomic_load(all + (int64_t)q * kOut + o, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    store(o, sum);
  }
}

namespace {

constexpr int kCUs = 256;

template <int MT, int TB>
hipError_t go(const uint8_t *codes, const uint16_t *scales, int N, int K, const uint16_t *X, int M,
              float *Y, hipStream_t stream) {
  // groups in flight per wave: about 8 to 16 weight pieces, within the register file
  constexpr int D = TB == 1 ? 8 : TB == 2 ? 6 : TB <= 4 ? 4 : 2;
  const int tiles = (N + 15) / 16;
  const int blocks = (tiles + TB - 1) / TB;
  hipLaunchKernelGGL((gemm_mfma_kernel<MT, TB, D>), dim3(blocks), dim3(kThreads), 0, stream, codes,
                     scales, X, Y, N, K, M);
  return hipGetLastError();
}

template <int MT, int TB>
hipError_t go_pair(const uint8_t *codes, const uint16_t *scales, int N, int K, const uint16_t *X,
                   int M, float *Y, int S, uint32_t *cnt, float *part, hipStream_t stream) {
  constexpr int D = 1;  // pairs in flight per wave (measured: deeper rings run slower)
  const int tiles = (N + 15) / 16;
  const int blocks = (tiles + TB - 1) / TB;
  hipLaunchKernelGGL((gemm_mfma_pair_kernel<MT, TB, D>), dim3(blocks, S), dim3(kThreads), 0,
                     stream, codes, scales, X, Y, N, K, M, S, cnt);
  (void)part;  // the kernel derives the same address from cnt
  return hipGetLastError();
}

template <int MT>
hipError_t go_pair_tb(int TB, const uint8_t *codes, const uint16_t *scales, int N, int K,
                      const uint16_t *X, int M, float *Y, int S, uint32_t *cnt, float *part,
                      hipStream_t s) {
  switch (TB) {
    case 1: return go_pair<MT, 1>(codes, scales, N, K, X, M, Y, S, cnt, part, s);
    case 2: return go_pair<MT, 2>(codes, scales, N, K, X, M, Y, S, cnt, part, s);
    case 3: return go_pair<MT, 3>(codes, scales, N, K, X, M, Y, S, cnt, part, s);
    case 4: return go_pair<MT, 4>(codes, scales, N, K, X, M, Y, S, cnt, part, s);
    case 5: return go_pair<MT, 5>(codes, scales, N, K, X, M, Y, S, cnt, part, s);
    // (never chosen for MT = 2, whose 6-tile form spills registers)
    case 6: return go_pair<MT, MT == 2 ? 7 : 6>(codes, scales, N, K, X, M, Y, S, cnt, part, s);
    case 7: return go_pair<MT, 7>(codes, scales, N, K, X, M, Y, S, cnt, part, s);
    default: return go_pair<MT, 8>(codes, scales, N, K, X, M, Y, S, cnt, part, s);
  }
}

template <int TB>
hipError_t go_quad(const uint8_t *codes, const uint16_t *scales, int N, int K, const uint16_t *X,
                   int M, float *Y, hipStream_t stream) {
  const int tiles = (N + 15) / 16;
  const int blocks = (tiles + TB - 1) / TB;
  hipLaunchKernelGGL((gemm_mfma_quad_kernel<TB>), dim3(blocks), dim3(kThreads), 0, stream, codes,
                     scales, X, Y, N, K, M);
  return hipGetLastError();
}

// Quad-step plan: enough column tiles per workgroup for one workgroup per CU,
// at most 4 (at 4 tiles two workgroups share a CU; a sweep over the 8B shapes
// at M = 8 put 4 ahead of 7 on gate|up, 25.7 vs 26.6 us, and K-splits behind
// no split everywhere).
hipError_t go_quad_plan(const uint8_t *codes, const uint16_t *scales, int N, int K,
                        const uint16_t *X, int M, float *Y, hipStream_t s) {
  const int tiles = (N + 15) / 16;
  switch (std::min((tiles + kCUs - 1) / kCUs, 4)) {
    case 1: return go_quad<1>(codes, scales, N, K, X, M, Y, s);
    case 2: return go_quad<2>(codes, scales, N, K, X, M, Y, s);
    case 3: return go_quad<3>(codes, scales, N, K, X, M, Y, s);
    default: return go_quad<4>(codes, scales, N, K, X, M, Y, s);
  }
}

struct StreamPlan {
  int ns, it, nb, S;  // steps per wave, tiles per workgroup, workgroups per split, K-splits
};

template <int MR, int NS, int IT>
hipError_t go_stream(const uint8_t *codes, const uint16_t *scales, int N, int K, const uint16_t *X,
                     int M, float *Y, const StreamPlan &p, uint32_t *cnt, hipStream_t stream) {
  // wide scale loads when every wave's slice is exactly NS steps, NS even
  const int NQ = (K >> 6) >> 2;
  const bool wide = NS % 2 == 0 && NQ % (p.S * kWaves) == 0 && NQ / (p.S * kWaves) == NS;
  // f16 products from 5 tiles per workgroup: the per-group shift costs set-up
  // that shorter walks do not win back
  constexpr bool F16 = IT >= 5;
  if (wide)
    hipLaunchKernelGGL((gemm_mfma_stream_kernel<MR, NS, IT, NS % 2 == 0, F16>), dim3(p.nb, p.S),
                       dim3(kThreads), 0, stream, codes, scales, X, Y, N, K, M, p.nb, p.S, cnt);
  else
    hipLaunchKernelGGL((gemm_mfma_stream_kernel<MR, NS, IT, false, F16>), dim3(p.nb, p.S),
                       dim3(kThreads), 0, stream, codes, scales, X, Y, N, K, M, p.nb, p.S, cnt);
  return hipGetLastError();
}

template <int MR, int NS>
hipError_t go_stream_it(const uint8_t *codes, const uint16_t *scales, int N, int K,
                        const uint16_t *X, int M, float *Y, const StreamPlan &p, uint32_t *cnt,
                        hipStream_t s) {
  switch (p.it) {
    case 1: return go_stream<MR, NS, 1>(codes, scales, N, K, X, M, Y, p, cnt, s);
    case 2: return go_stream<MR, NS, 2>(codes, scales, N, K, X, M, Y, p, cnt, s);
    case 3: return go_stream<MR, NS, 3>(codes, scales, N, K, X, M, Y, p, cnt, s);
    case 4: return go_stream<MR, NS, 4>(codes, scales, N, K, X, M, Y, p, cnt, s);
    case 5: return go_stream<MR, NS, 5>(codes, scales, N, K, X, M, Y, p, cnt, s);
    case 6: return go_stream<MR, NS, 6>(codes, scales, N, K, X, M, Y, p, cnt, s);
    case 7: return go_stream<MR, NS, 7>(codes, scales, N, K, X, M, Y, p, cnt, s);
    default: return go_stream<MR, NS, 8>(codes, scales, N, K, X, M, Y, p, cnt, s);
  }
}

// Streaming plan: one workgroup per CU, 2 to 8 tiles each (3 to 8 above M = 8),
// at most 4 steps per wave at M <= 8 (the activation fragments of 4 steps are
// 128 registers), 2 at M = 9..32.  Measured on the Llama-3.1-8B shapes: ahead
// of the quad step wherever a workgroup gets two or more tiles; at one tile per
// CU (4096 columns) the quad step is as fast or faster, and with 7 steps per
// wave (down, 14336 of K) all steps in flight ran slower (17.9 vs 14.1 us).
// Against the pair step (M = 9..32): gate|up 28672 x 4096 at M = 12, 16, 32
// 29.6, 30.3, 35.6 -> 19.5, 20.0, 26.0 us; at two tiles per CU (q|k|v, 6144
// rows) even or behind (M = 32: 14.8 vs 14.5), so from three.
//
// With a workspace, up to 512 tiles and at least 4096 of K, K is split over
// workgroups of several tiles instead, so that a CU reads only its share of
// the activations and every CU streams the same share of the codes:
//  - M <= 8, 257 to 512 tiles (which leave half the CUs with two tiles and half
//    with one): two splits (q|k|v 6144 x 4096 at M = 8: 9.3 -> 8.8 us).  At one
//    tile per CU the split's exchange of partial tiles, three more memory round
//    trips in a row, costs more than it saves (o 4096 x 4096 and down 4096 x
//    14336 at M = 8 in two and four splits: 6.1 -> 7.4 and 13.3 -> 15.8 us);
//  - M = 9..32, where the activations a one-tile CU reads are 2 to 8 times its
//    codes: two splits up to 4096 of K, four above, each workgroup taking as
//    many tiles as splits (against the pair step's own splits at M = 32: q|k|v
//    15.7 -> 12.2 us, o 11.0 -> 10.5, down 4096 x 14336 26.7 -> 23.5; at M = 16
//    10.5 -> 9.3, 8.2 -> 7.9, 17.8 -> 16.9; twice as many splits ran 30-60 %
//    slower).
bool stream_plan(int N, int K, int M, bool split, StreamPlan &p) {
  const int NQ = (K >> 6) >> 2;
  const int tiles = (N + 15) / 16;
  if (M < 1 || M > 32 || (K >> 6) % 4 != 0 || N < 16) return false;
  const int nsmax = M <= 8 ? 4 : 2;
  if (split && tiles <= 2 * kCUs && NQ >= 16 && (M > 8 || tiles > kCUs)) {
    p.S = M <= 8 || NQ <= 16 ? 2 : 4;
    p.it = tiles <= kCUs ? p.S : (tiles * p.S + kCUs - 1) / kCUs;
    p.nb = (tiles + p.it - 1) / p.it;
    p.ns = ((NQ + p.S - 1) / p.S + kWaves - 1) / kWaves;
    if (p.ns <= nsmax && p.it <= 8 && (p.ns < 4 || p.it <= 5) && p.nb <= kSplitCounters)
      return true;
  }
  p.S = 1;
  p.ns = (NQ + kWaves - 1) / kWaves;
  p.nb = std::min(tiles, kCUs);
  p.it = (tiles + p.nb - 1) / p.nb;
  return tiles > kCUs && p.ns >= 1 && p.ns <= nsmax && p.it >= (M <= 8 ? 2 : 3) && p.it <= 8 &&
         (p.ns < 4 || p.it <= 5);  // (4 steps and 6 tiles spill registers)
}

int64_t stream_workspace_bytes(int M, const StreamPlan &p) {
  if (p.S == 1) return 0;
  const int MT = M <= 16 ? 1 : 2;
  return kSplitCounterBytes + (int64_t)p.nb * p.S * p.it * MT * 256 * 4;
}

template <int MR>
hipError_t go_stream_ns(const uint8_t *codes, const uint16_t *scales, int N, int K,
                        const uint16_t *X, int M, float *Y, const StreamPlan &p, uint32_t *cnt,
                        hipStream_t s) {
  switch (p.ns) {
    case 1: return go_stream_it<MR, 1>(codes, scales, N, K, X, M, Y, p, cnt, s);
    case 2: return go_stream_it<MR, 2>(codes, scales, N, K, X, M, Y, p, cnt, s);
    case 3: return go_stream_it<MR, MR == 8 ? 3 : 2>(codes, scales, N, K, X, M, Y, p, cnt, s);
    default: return go_stream_it<MR, MR == 8 ? 4 : 2>(codes, scales, N, K, X, M, Y, p, cnt, s);
  }
}

hipError_t go_stream_plan(const uint8_t *codes, const uint16_t *scales, int N, int K,
                          const uint16_t *X, int M, float *Y, const StreamPlan &p, uint32_t *cnt,
                          hipStream_t s) {
  if (M <= 8) return go_stream_ns<8>(codes, scales, N, K, X, M, Y, p, cnt, s);
  if (M <= 16) return go_stream_ns<16>(codes, scales, N, K, X, M, Y, p, cnt, s);
  return go_stream_ns<32>(codes, scales, N, K, X, M, Y, p, cnt, s);
}

// Pair-step plan: TB column tiles per workgroup and S K-splits.  Without a
// workspace, S = 1 and TB just gives every CU a workgroup.  With one, K is split
// where a sweep of (TB, S) over the Llama-3.1-8B shapes measured it faster:
//  - one column tile per CU, two 16-row tiles (M > 16): four tiles in four
//    K-splits from 8192 of K (down: 38.0 -> 27.6 us at M = 32), else two in two
//    (4096 x 4096: 14.2 -> 13.5 us);
//  - one column tile per CU, M of 5 to 16, 8192 of K or more: two tiles in two
//    K-splits (down 4096 x 14336: M = 16 22.9 -> 19.8 us, M = 8 18.2 -> 17.4);
//  - two column tiles per workgroup (fewer workgroups than CUs), M > 16: three
//    tiles in two K-splits, which fills every CU (q|k|v 6144 x 4096 at M = 32:
//    17.8 -> 16.2 us).
// Elsewhere (M <= 4, K = 4096 at M <= 16, the wide gate|up tiles) the shorter
// K-ranges lose more to set-up and to the partial-tile traffic than they save.
struct PairPlan {
  int TB, S;
};

PairPlan plan_pair(int N, int K, int M, bool split) {
  const int NT = (N + 15) / 16;
  const int NP = (K >> 6) >> 1;
  PairPlan p{std::min((NT + kCUs - 1) / kCUs, 8), 1};
  if (M > 16 && p.TB == 6) p.TB = 7;  // the 6-tile form spills registers at MT = 2
  if (!split || NP < 16 || NT > kSplitCounters) return p;
  if (p.TB == 1 && M > 16) p = NP >= 64 ? PairPlan{4, 4} : PairPlan{2, 2};
  else if (p.TB == 1 && M > 4 && NP >= 64) p = PairPlan{2, 2};
  else if (p.TB == 2 && M > 16) p = PairPlan{3, 2};
  return p;
}

int64_t pair_workspace_bytes(int N, int M, const PairPlan &p) {
  if (p.S == 1) return 0;
  const int MT = M <= 16 ? 1 : 2;
  const int64_t groups = ((N + 15) / 16 + p.TB - 1) / p.TB;
  return kSplitCounterBytes + groups * p.S * p.TB * MT * 256 * 4;
}

template <int MT>
hipError_t go_tb(int TB, const uint8_t *codes, const uint16_t *scales, int N, int K,
                 const uint16_t *X, int M, float *Y, hipStream_t s) {
  switch (TB) {
    case 1: return go<MT, 1>(codes, scales, N, K, X, M, Y, s);
    case 2: return go<MT, 2>(codes, scales, N, K, X, M, Y, s);
    case 3: return go<MT, 3>(codes, scales, N, K, X, M, Y, s);
    case 4: return go<MT, 4>(codes, scales, N, K, X, M, Y, s);
    case 5: return go<MT, 5>(codes, scales, N, K, X, M, Y, s);
    case 6: return go<MT, 6>(codes, scales, N, K, X, M, Y, s);
    case 7: return go<MT, 7>(codes, scales, N, K, X, M, Y, s);
    default: return go<MT, 8>(codes, scales, N, K, X, M, Y, s);
  }
}

// M <= 8 with a multiple of four groups per row runs in quad steps (given
// 8-byte aligned scales) and never splits K; neither does the pair-step kernel
// that stands in for it when the scales are only 4-byte aligned
bool quad_shape(int K, int M) { return M <= 8 && (K >> 6) % 4 == 0; }

}  // namespace

bool gemm_mfma_streams(int64_t N, int64_t K, int M) {
  StreamPlan p;
  return stream_plan((int)N, (int)K, M, false, p);
}

int64_t gemm_mfma_workspace_bytes(int64_t N, int64_t K, int M) {
  if (M < 1 || M > 32 || (K >> 6) % 2 != 0) return 0;
  StreamPlan sp;
  const int64_t stream_need =
      stream_plan((int)N, (int)K, M, true, sp) ? stream_workspace_bytes(M, sp) : 0;
  if (quad_shape((int)K, M)) return stream_need;
  return std::max(stream_need,
                  pair_workspace_bytes((int)N, M, plan_pair((int)N, (int)K, M, true)));
}

hipError_t launch_gemm_mfma(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                            const uint16_t *X, int M, float *Y, void *workspace,
                            int64_t workspace_bytes, hipStream_t stream) {
  if (M < 1 || M > 32) return hipErrorInvalidValue;
  const int n = (int)N, k = (int)K;
  // pair steps need an even group count and 4-byte aligned scales (every model
  // shape); otherwise one group per step
  const bool aligned8 = (reinterpret_cast<uintptr_t>(scales) & 7) == 0;
  StreamPlan sp;
  if (aligned8 && stream_plan(n, k, M, workspace != nullptr, sp)) {
    if (sp.S > 1 && workspace_bytes < stream_workspace_bytes(M, sp)) return hipErrorInvalidValue;
    return go_stream_plan(codes, scales, n, k, X, M, Y, sp, static_cast<uint32_t *>(workspace),
                          stream);
  }
  if (quad_shape(k, M) && aligned8) return go_quad_plan(codes, scales, n, k, X, M, Y, stream);
  const bool pair = ((k >> 6) % 2 == 0) && ((reinterpret_cast<uintptr_t>(scales) & 3) == 0);
  if (pair) {
    PairPlan p = plan_pair(n, k, M, workspace != nullptr && !quad_shape(k, M));
    uint32_t *cnt = nullptr;
    float *part = nullptr;
    if (p.S > 1) {
      const int64_t need = pair_workspace_bytes(n, M, p);
      if (workspace_bytes < need) return hipErrorInvalidValue;
      cnt = static_cast<uint32_t *>(workspace);
      part = reinterpret_cast<float *>(static_cast<char *>(workspace) + kSplitCounterBytes);
    }
    if (M <= 16) return go_pair_tb<1>(p.TB, codes, scales, n, k, X, M, Y, p.S, cnt, part, stream);
    return go_pair_tb<2>(p.TB, codes, scales, n, k, X, M, Y, p.S, cnt, part, stream);
  }
  // column tiles per workgroup: enough for one workgroup per CU, at most 8
  // (past that, workgroups run in rounds)
  const int tiles = (n + 15) / 16;
  const int TB = std::min((tiles + kCUs - 1) / kCUs, 8);
  if (M <= 16) return go_tb<1>(TB, codes, scales, n, k, X, M, Y, stream);
  return go_tb<2>(TB, codes, scales, n, k, X, M, Y, stream);
}

}  // namespace nf4
