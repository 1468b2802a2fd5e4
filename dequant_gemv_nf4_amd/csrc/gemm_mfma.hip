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
#include <utility>

#include "nf4_device.h"
#include "nf4_launch.h"

namespace nf4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;  // 8 waves
constexpr int kWaves = kThreads / 64;

// ---------------------------------------------------------------------------
// bf16 hi / lo split of the levels, at compile time (round to nearest even).
// ---------------------------------------------------------------------------
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

}  // namespace

hipError_t launch_gemm_mfma(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                            const uint16_t *X, int M, float *Y, hipStream_t stream) {
  if (M < 1 || M > 32) return hipErrorInvalidValue;
  const int n = (int)N, k = (int)K;
  // column tiles per workgroup: enough for one workgroup per CU, at most 8
  // (past that, workgroups run in rounds)
  const int tiles = (n + 15) / 16;
  const int TB = std::min((tiles + kCUs - 1) / kCUs, 8);
  if (M <= 16) return go_tb<1>(TB, codes, scales, n, k, X, M, Y, stream);
  return go_tb<2>(TB, codes, scales, n, k, X, M, Y, stream);
}

}  // namespace nf4
