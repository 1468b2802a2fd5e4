// gemv.hip -- fused NF4 dequant matrix-vector product on the vector ALUs (gfx950).
//
// Computes Y[m][n] = sum_k L[code(n,k)] * s(n,k/64) * X[m][k] for M = 1 (decode,
// deep-fold README "Method": the N=1 GEMV) and for small M up to 7, where the
// weight decode is shared by M dot products.  The dense matrix is never formed
// (Trapetum home page: the 4-bit weights are decoded inside the matmul).
//
// Work mapping.  A row's K is cut into 32-weight "units" (16 code bytes, half a
// scale group).  Inside a workgroup the waves form G row groups x S K-slices; a
// lane owns up to UPL units of its slice -- the same units for every row it
// visits -- so its activations are loaded once, kept in registers as f16 pairs,
// and reused across all rows.  Per row a lane streams UPL x 16 bytes of codes
// (one 128-bit load each, consecutive lanes on consecutive 16-byte chunks) plus
// one fp16 scale per unit.
//
// Decode: one v_perm_b32 turns a code byte into the LDS address of its entry in
// the bank-replicated byte table (nf4_device.h); the entry is the f16 pair
// (L[lo], L[hi]) and feeds one v_dot2_f32_f16 against (x[2j], x[2j+1]).  So two
// weights cost one perm, one LDS read and one dot per activation row; the group
// scale is applied once per unit with an fp32 FMA.
//
// Activation range: each lane scales its activations by a power of two so that
// its largest |x| sits just under 2^15 before rounding to f16 (bf16 -> f16 is
// then exact down to 2^-29 of that maximum), and undoes it on the fp32 partial.
//
// Reduction: partial sums are reduced over the wave's lanes in a fixed butterfly
// order, then over the S slices in LDS in slice order: no atomics, so results
// are bitwise reproducible.
#include "nf4_device.h"
#include "nf4_launch.h"

namespace nf4 {

typedef __fp16 fp16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(fp16x2_t, a), __builtin_bit_cast(fp16x2_t, b),
                                c, false);
}

constexpr int kMaxRedFloats = 4096;  // 16 KiB for cross-slice partials
constexpr int kMaxWaves = 8;         // waves per workgroup

template <int M, int UPL>
__global__ void __launch_bounds__(64 * kMaxWaves)
    gemv_valu_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                     const uint16_t *__restrict__ X, float *__restrict__ Y, int N, int K, int S,
                     int G, int Us, int iters) {
  __shared__ uint32_t lut[kLutWords];
  __shared__ float red[kMaxRedFloats];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int slice = wave % S;
  const int grp = wave / S;
  const int U = K >> 5;
  const int ub = slice * Us;
  const int ue = min(U, ub + Us);
  const int rows_per_block = G * iters;
  const int row0 = blockIdx.x * rows_per_block;
  const int64_t row_bytes = K >> 1;
  const int64_t row_groups = K >> 6;

  int unit[UPL];
  bool valid[UPL];
#pragma unroll
  for (int i = 0; i < UPL; ++i) {
    unit[i] = ub + lane + 64 * i;
    valid[i] = unit[i] < ue;
  }

  auto load_row = [&](int r, uint4 *c, uint32_t *s) {
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
      if (valid[i] && r < N) {
        c[i] = *reinterpret_cast<const uint4 *>(codes + (int64_t)r * row_bytes + unit[i] * 16);
        s[i] = scales[(int64_t)r * row_groups + (unit[i] >> 1)];
      } else {
        c[i] = make_uint4(0, 0, 0, 0);
        s[i] = 0;
      }
    }
  };

  // first row's codes in flight before the table build
  uint4 cw[UPL];
  uint32_t sw[UPL];
  load_row(row0 + grp, cw, sw);

  // activations of this lane's units: bf16 pairs, later rewritten as f16 pairs
  uint32_t xh[M][UPL][16];
  int xshift[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
      if (valid[i]) {
        const uint4 *src = reinterpret_cast<const uint4 *>(X + (int64_t)m * K + unit[i] * 32);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          uint4 t = src[v];
          xh[m][i][4 * v + 0] = t.x;
          xh[m][i][4 * v + 1] = t.y;
          xh[m][i][4 * v + 2] = t.z;
          xh[m][i][4 * v + 3] = t.w;
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) xh[m][i][v] = 0;
      }
    }
  }

  build_byte_lut(lut, tid, blockDim.x);

#pragma unroll
  for (int m = 0; m < M; ++m) {
    // largest magnitude among this lane's activations of row m (bf16 bits order
    // like the values once the sign is dropped)
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < UPL; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        uint32_t w = xh[m][i][v] & 0x7fff7fffu;
        mx = max(mx, max(w & 0xffffu, w >> 16));
      }
    int e = 0;
    (void)frexpf(__uint_as_float(mx << 16), &e);  // max < 2^e
    const int sh = 15 - e;
    xshift[m] = sh;
#pragma unroll
    for (int i = 0; i < UPL; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        uint32_t w = xh[m][i][v];
        _Float16 lo = (_Float16)ldexpf(bf16_lo(w), sh);
        _Float16 hi = (_Float16)ldexpf(bf16_hi(w), sh);
        xh[m][i][v] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
  }

  __syncthreads();

  const uint32_t laneoff = (uint32_t)lane * 4u;
  for (int it = 0; it < iters; ++it) {
    const int r = row0 + grp + it * G;
    const bool more = it + 1 < iters;
    uint4 cn[UPL];
    uint32_t sn[UPL];
    if (more) load_row(r + G, cn, sn);
    if (r < N) {
      float acc[M];
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = 0.0f;
#pragma unroll
      for (int i = 0; i < UPL; ++i) {
        if (valid[i]) {
          const uint32_t q[4] = {cw[i].x, cw[i].y, cw[i].z, cw[i].w};
          float p[M];
#pragma unroll
          for (int m = 0; m < M; ++m) p[m] = 0.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t l0 = lds_load_u32(lut, lut_addr<0>(q[j], laneoff));
            const uint32_t l1 = lds_load_u32(lut, lut_addr<1>(q[j], laneoff));
            const uint32_t l2 = lds_load_u32(lut, lut_addr<2>(q[j], laneoff));
            const uint32_t l3 = lds_load_u32(lut, lut_addr<3>(q[j], laneoff));
#pragma unroll
            for (int m = 0; m < M; ++m) {
              p[m] = dot2(l0, xh[m][i][4 * j + 0], p[m]);
              p[m] = dot2(l1, xh[m][i][4 * j + 1], p[m]);
              p[m] = dot2(l2, xh[m][i][4 * j + 2], p[m]);
              p[m] = dot2(l3, xh[m][i][4 * j + 3], p[m]);
            }
          }
          const float sc = f16_bits_to_f32(sw[i]);
#pragma unroll
          for (int m = 0; m < M; ++m) acc[m] = fmaf(p[m], sc, acc[m]);
        }
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float t = wave_sum(ldexpf(acc[m], -xshift[m]));
        if (lane == 0) red[(m * rows_per_block + (r - row0)) * S + slice] = t;
      }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < UPL; ++i) {
        cw[i] = cn[i];
        sw[i] = sn[i];
      }
    }
  }
  __syncthreads();
  for (int t = tid; t < M * rows_per_block; t += blockDim.x) {
    const int m = t / rows_per_block;
    const int rl = t - m * rows_per_block;
    const int r = row0 + rl;
    if (r < N) {
      float s = 0.0f;
      for (int sl = 0; sl < S; ++sl) s += red[t * S + sl];
      Y[(int64_t)m * N + r] = s;
    }
  }
}

namespace {

struct Plan {
  int S, G, Us, upl, iters, blocks, threads;
};

int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Choose slices / row groups / rows per block for an (N, K, M) product.
bool plan_valu(int64_t N, int64_t K, int M, Plan &p) {
  const int U = (int)(K / 32);
  const int upl_cap = M == 1 ? 4 : (M <= 3 ? 2 : 1);
  int S = cdiv(U, 64 * upl_cap);
  if (S > kMaxWaves) return false;
  // widen the K split while too few row groups exist to give every CU work
  for (;;) {
    const int G = std::max(1, kMaxWaves / S);
    if (cdiv(N, G) >= 512 || 2 * S > kMaxWaves) break;
    S *= 2;
  }
  const int G = std::max(1, kMaxWaves / S);
  const int Us = cdiv(U, S);
  const int upl = cdiv(Us, 64);
  int iters = (int)std::max<int64_t>(1, N / ((int64_t)G * 512));
  while (iters > 1 && M * G * iters * S > kMaxRedFloats) --iters;
  if (M * G * iters * S > kMaxRedFloats) return false;
  p.S = S;
  p.G = G;
  p.Us = Us;
  p.upl = upl;
  p.iters = iters;
  p.blocks = cdiv(N, (int64_t)G * iters);
  p.threads = 64 * S * G;
  return upl <= upl_cap && p.threads <= 64 * kMaxWaves;
}

template <int M, int UPL>
hipError_t go(const Plan &p, const uint8_t *codes, const uint16_t *scales, int N, int K,
              const uint16_t *X, float *Y, hipStream_t stream) {
  hipLaunchKernelGGL((gemv_valu_kernel<M, UPL>), dim3(p.blocks), dim3(p.threads), 0, stream,
                     codes, scales, X, Y, N, K, p.S, p.G, p.Us, p.iters);
  return hipGetLastError();
}

}  // namespace

bool valu_supported(int64_t N, int64_t K, int M) {
  Plan p;
  return plan_valu(N, K, M, p);
}

hipError_t launch_gemv_valu(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                            const uint16_t *X, int M, float *Y, hipStream_t stream) {
  Plan p;
  if (!plan_valu(N, K, M, p)) return hipErrorInvalidConfiguration;
  const int n = (int)N, k = (int)K;
  switch (M * 8 + p.upl) {
    case 1 * 8 + 1: return go<1, 1>(p, codes, scales, n, k, X, Y, stream);
    case 1 * 8 + 2: return go<1, 2>(p, codes, scales, n, k, X, Y, stream);
    case 1 * 8 + 3: return go<1, 3>(p, codes, scales, n, k, X, Y, stream);
    case 1 * 8 + 4: return go<1, 4>(p, codes, scales, n, k, X, Y, stream);
    case 2 * 8 + 1: return go<2, 1>(p, codes, scales, n, k, X, Y, stream);
    case 2 * 8 + 2: return go<2, 2>(p, codes, scales, n, k, X, Y, stream);
    case 3 * 8 + 1: return go<3, 1>(p, codes, scales, n, k, X, Y, stream);
    case 3 * 8 + 2: return go<3, 2>(p, codes, scales, n, k, X, Y, stream);
    case 4 * 8 + 1: return go<4, 1>(p, codes, scales, n, k, X, Y, stream);
    case 5 * 8 + 1: return go<5, 1>(p, codes, scales, n, k, X, Y, stream);
    case 6 * 8 + 1: return go<6, 1>(p, codes, scales, n, k, X, Y, stream);
    case 7 * 8 + 1: return go<7, 1>(p, codes, scales, n, k, X, Y, stream);
    default: return hipErrorInvalidConfiguration;
  }
}

}  // namespace nf4
