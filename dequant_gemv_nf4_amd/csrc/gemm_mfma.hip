// gemm_mfma.hip -- fused NF4 dequant product for activation batches of 8..32 rows
// on the matrix cores (gfx950, v_mfma_f32_16x16x32_f16).
//
// Computes Y[m][n] = sum_k L[code(n,k)] * s(n,k/64) * X[m][k].  Source:
// deep-fold README, "Method": prefill runs the NF4 product on prompt chunks of
// up to 32 positions, rebuilding weights into matrix-core register fragments.
//
// MFMA mapping (D = A.B + C, 16 x 16 x 32):
//   A = activations, 16 rows m x 32 k, in f16;
//   B = decoded weights, 32 k x 16 columns n (one weight row per column);
//   D = Y tile: lane l holds Y[4*(l/16) + r][n0 + l%16], r = 0..3.
// Lane l supplies k-slots 8*(l/16) .. +7 of both A and B.  Within one scale
// group (64 k) the slots of lane-group g in step h are k = 16g + 8h + e, so a
// lane's 16 weights of a group are one 8-byte load and its 16 activations are 32
// contiguous bytes.  Both steps of a group land in a scratch tile D_g, which is
// scaled by that weight row's group scale in fp32 (lane-local: the scale belongs
// to the lane's own column) and added to a chunk accumulator.  No weight is
// rounded together with its scale.
//
// Activations: the block stages X[:, chunk] (KC = 512 k) in LDS as f16, each row
// m multiplied by a power of two so that its largest |x| in the chunk sits just
// under 2^15 (exact conversion from bf16 down to 2^-29 of that maximum); the
// chunk accumulator is multiplied back by that power of two when the chunk ends.
// Staging of chunk c+1 overlaps the products of chunk c (double buffer).
//
// Work split: 8 waves per block = T row tiles (16 rows each) x KS K-slices; the
// slices of a tile take interleaved groups of each chunk.  Their partial tiles
// are summed in LDS in slice order at the end: deterministic, no atomics.
// Decode: same bank-replicated byte table and v_perm addressing as the GEMV.
#include "nf4_device.h"
#include "nf4_launch.h"

namespace nf4 {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kKC = 512;                  // k per staged chunk (8 groups)
constexpr int kXStride = kKC + 8;         // f16 elements per staged row (16 B pad)
constexpr int kThreads = 512;             // 8 waves

__device__ __forceinline__ f16x8_t as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8_t, v); }

template <int MT, int T>
__global__ void __launch_bounds__(kThreads)
    gemm_mfma_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                     const uint16_t *__restrict__ X, float *__restrict__ Y, int N, int K, int M) {
  constexpr int KS = 8 / T;        // K-slices per row tile
  constexpr int MP = 16 * MT;      // staged activation rows
  constexpr int GPW = 8 / KS;      // groups per chunk handled by one wave
  // one LDS block carved by hand: the decode table first, at offset 0, so that its
  // byte addresses need no base added before each read
  constexpr int kXsWords = 2 * MP * kXStride / 2;
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLutWords + kXsWords + 2 * MP];
  uint32_t *const lut = lds;
  typedef uint16_t XRow[kXStride];
  XRow *const xs0 = reinterpret_cast<XRow *>(lds + kLutWords);  // [2][MP] rows
  float *const fx0 = reinterpret_cast<float *>(lds + kLutWords + kXsWords);  // [2][MP]
  auto xs = [&](int buf, int row) -> uint16_t * { return xs0[buf * MP + row]; };
  auto fx = [&](int buf, int row) -> float & { return fx0[buf * MP + row]; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tile = wave / KS;
  const int ks = wave % KS;
  const int lg = lane >> 4;        // lane group: k-slot block
  const int col = lane & 15;       // weight row within the tile / activation row within A
  const int n = (blockIdx.x * T + tile) * 16 + col;
  const bool nvalid = n < N;
  const int64_t row_bytes = K >> 1;
  const int64_t row_groups = K >> 6;
  const int nchunks = (K + kKC - 1) / kKC;

  // ---- weights: this wave's groups of a chunk, one 8-byte load per lane per group
  auto load_w = [&](int c, uint2 *w, uint32_t *s) {
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
      const int q = ks + j * KS;                 // group within the chunk
      const int gk = c * (kKC / 64) + q;         // group index along K
      if (nvalid && gk < row_groups) {
        w[j] = *reinterpret_cast<const uint2 *>(codes + (int64_t)n * row_bytes + gk * 32 + lg * 8);
        s[j] = scales[(int64_t)n * row_groups + gk];
      } else {
        w[j] = make_uint2(0, 0);
        s[j] = 0;
      }
    }
  };

  // ---- activations: 16 threads per staged row; 32 bf16 per thread
  constexpr int TPR = kThreads / MP;             // threads per row (16 or 32)
  constexpr int EPT = kKC / TPR;                 // elements per thread (32 or 16)
  const int srow = tid / TPR;
  const int spart = tid % TPR;
  auto load_x = [&](int c, uint4 *raw) {
    const int k0 = c * kKC + spart * EPT;
#pragma unroll
    for (int v = 0; v < EPT / 8; ++v) {
      if (srow < M && k0 + 8 * v < K)
        raw[v] = *reinterpret_cast<const uint4 *>(X + (int64_t)srow * K + k0 + 8 * v);
      else
        raw[v] = make_uint4(0, 0, 0, 0);
    }
  };
  auto stage_x = [&](int buf, const uint4 *raw) {
    uint32_t mx = 0;
#pragma unroll
    for (int v = 0; v < EPT / 8; ++v) {
      const uint32_t w4[4] = {raw[v].x, raw[v].y, raw[v].z, raw[v].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t a = w4[i] & 0x7fff7fffu;
        mx = max(mx, max(a & 0xffffu, a >> 16));
      }
    }
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    int e = 0;
    (void)frexpf(__uint_as_float(mx << 16), &e);
    const int sh = 15 - e;
#pragma unroll
    for (int v = 0; v < EPT / 8; ++v) {
      const uint32_t w4[4] = {raw[v].x, raw[v].y, raw[v].z, raw[v].w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        _Float16 lo = (_Float16)ldexpf(bf16_lo(w4[i]), sh);
        _Float16 hi = (_Float16)ldexpf(bf16_hi(w4[i]), sh);
        o[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
               ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      *reinterpret_cast<uint4 *>(&xs(buf, srow)[spart * EPT + 8 * v]) =
          make_uint4(o[0], o[1], o[2], o[3]);
    }
    if (spart == 0) fx(buf, srow) = ldexpf(1.0f, -sh);
  };

  uint2 wcur[GPW];
  uint32_t scur[GPW];
  load_w(0, wcur, scur);
  uint4 xraw[EPT / 8];
  load_x(0, xraw);
  build_byte_lut(lut, tid, kThreads);
  stage_x(0, xraw);
  __syncthreads();

  const uint32_t laneoff = (uint32_t)lane * 4u;
  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nchunks;
    uint2 wnxt[GPW];
    uint32_t snxt[GPW];
    if (more) {
      load_w(c + 1, wnxt, snxt);
      load_x(c + 1, xraw);
    }
    f32x4_t cacc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) cacc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
      const int q = ks + j * KS;
      if (c * (kKC / 64) + q < row_groups) {     // uniform across the wave
        // decode the lane's 16 weights into two B fragments (steps h = 0, 1)
        uint4 b[2];
        const uint32_t wd[2] = {wcur[j].x, wcur[j].y};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          b[h].x = lds_load_u32(lut, lut_addr<0>(wd[h], laneoff));
          b[h].y = lds_load_u32(lut, lut_addr<1>(wd[h], laneoff));
          b[h].z = lds_load_u32(lut, lut_addr<2>(wd[h], laneoff));
          b[h].w = lds_load_u32(lut, lut_addr<3>(wd[h], laneoff));
        }
        const float sc = f16_bits_to_f32(scur[j]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const uint16_t *xrow = &xs(buf, mt * 16 + col)[q * 64 + lg * 16];
          const uint4 a0 = *reinterpret_cast<const uint4 *>(xrow);
          const uint4 a1 = *reinterpret_cast<const uint4 *>(xrow + 8);
          f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a0), as_f16x8(b[0]),
                                                            f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a1), as_f16x8(b[1]), d, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) cacc[mt][r] = fmaf(d[r], sc, cacc[mt][r]);
        }
      }
    }
    // undo the chunk's activation scaling: rows m = 16 mt + 4 lg + r
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[mt][r] = fmaf(cacc[mt][r], fx(buf, mt * 16 + lg * 4 + r), acc[mt][r]);
    if (more) {
      stage_x(buf ^ 1, xraw);
#pragma unroll
      for (int j = 0; j < GPW; ++j) {
        wcur[j] = wnxt[j];
        scur[j] = snxt[j];
      }
    }
    __syncthreads();
  }

  // ---- sum the KS slice partials of each tile in slice order; reuse xs as scratch
  float *red = reinterpret_cast<float *>(xs0);  // needs 8 * 64 * 4 * MT floats
  if (KS > 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[((wave * MT + mt) * 4 + r) * 64 + lane] = acc[mt][r];
    __syncthreads();
    if (ks == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float s = 0.0f;
          for (int j = 0; j < KS; ++j) s += red[(((wave + j) * MT + mt) * 4 + r) * 64 + lane];
          acc[mt][r] = s;
        }
    }
  }
  if (ks == 0 && nvalid) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mt * 16 + lg * 4 + r;
        if (m < M) Y[(int64_t)m * N + n] = acc[mt][r];
      }
  }
}

namespace {
template <int MT, int T>
hipError_t go(const uint8_t *codes, const uint16_t *scales, int N, int K, const uint16_t *X,
              int M, float *Y, hipStream_t stream) {
  const int tiles = (N + 15) / 16;
  const int blocks = (tiles + T - 1) / T;
  hipLaunchKernelGGL((gemm_mfma_kernel<MT, T>), dim3(blocks), dim3(kThreads), 0, stream, codes,
                     scales, X, Y, N, K, M);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_mfma(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                            const uint16_t *X, int M, float *Y, hipStream_t stream) {
  if (M < 1 || M > 32) return hipErrorInvalidValue;
  const int n = (int)N, k = (int)K;
  // row tiles per block: as many as keep >= 256 blocks (one per CU)
  const int tiles = (n + 15) / 16;
  int T = 1;
  while (T < 8 && tiles / (2 * T) >= 256) T *= 2;
  if (M <= 16) {
    switch (T) {
      case 1: return go<1, 1>(codes, scales, n, k, X, M, Y, stream);
      case 2: return go<1, 2>(codes, scales, n, k, X, M, Y, stream);
      case 4: return go<1, 4>(codes, scales, n, k, X, M, Y, stream);
      default: return go<1, 8>(codes, scales, n, k, X, M, Y, stream);
    }
  }
  switch (T) {
    case 1: return go<2, 1>(codes, scales, n, k, X, M, Y, stream);
    case 2: return go<2, 2>(codes, scales, n, k, X, M, Y, stream);
    case 4: return go<2, 4>(codes, scales, n, k, X, M, Y, stream);
    default: return go<2, 8>(codes, scales, n, k, X, M, Y, stream);
  }
}

}  // namespace nf4
