// gemv.hip -- fused NF4 dequant matrix-vector product on the vector ALUs (gfx950).
//
// Computes Y[m][n] = sum_k L[code(n,k)] * s(n,k/64) * X[m][k] for M = 1 (decode,
// deep-fold README "Method": the N=1 GEMV) and for small M up to 7, where the
// weight decode is shared by M dot products.  The dense matrix is never formed
// (Trapetum home page: the 4-bit weights are decoded inside the matmul).
//
// Work mapping.  A row's K is cut into 32-weight "units" (16 code bytes, half a
// scale group).  One workgroup of 8 waves per CU; the waves form G row groups x
// S K-slices, and a lane owns up to UPL units of its slice (units ub + lane +
// 64 i) -- the same units for every row it visits -- so its activations sit in
// registers as f16 pairs for the whole kernel.  Rows are dealt round-robin over
// the grid, so at any moment all CUs stream one contiguous band of rows.  Per row
// a lane issues UPL 128-bit code loads (consecutive lanes on consecutive 16-byte
// chunks) and one or two 2-byte scale loads that cover the wave's groups; each
// unit's scale is then fetched from the loading lane with ds_bpermute.  A ring of
// kDepth rows per wave keeps the loads in flight; loads carry no branches (a
// branch around a load makes the compiler wait for every load in flight before
// the register can be reused).
//
// Decode: one v_perm_b32 turns a code byte into the LDS address of its entry in
// the bank-replicated byte table (nf4_device.h); the entry is the f16 pair
// (L[lo], L[hi]) and feeds one v_dot2_f32_f16 against (x[2j], x[2j+1]).  Two
// weights cost one perm, one LDS read and one dot per activation row; the group
// scale is applied once per unit in fp32.
//
// Activations are converted once per workgroup: thread t turns unit t of each
// activation row into f16 after scaling it by a power of two that puts its
// largest |x| just under 2^15 (exact from bf16 down to 2^-29 of that maximum),
// and stages it in LDS with the shift; lanes then copy their units into
// registers.  The shift is undone on the unit's fp32 partial.  Activation loads
// are issued before the first code loads so that the set-up does not wait
// behind them (loads return in order).
//
// Reduction: per row, lanes are summed with DPP row operations in a fixed order;
// the S slices of a row are added in LDS in slice order.  No atomics: results
// are bitwise reproducible.
#include "nf4_device.h"
#include "nf4_launch.h"

namespace nf4 {

typedef __fp16 fp16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(fp16x2_t, a), __builtin_bit_cast(fp16x2_t, b),
                                c, false);
}

constexpr int kThreads = 512;                           // 8 waves, one workgroup per CU
constexpr int kWaves = kThreads / 64;
constexpr int kRedFloats = 4096;                        // cross-slice partials (16 KiB)
constexpr int kStageBytes = 163840 - 4 * kLutWords - 4 * kRedFloats;  // 80 KiB for activations
constexpr int kUnitStageBytes = 64 + 4;                 // 32 f16 + a shift, per (row, unit)
constexpr int kMaxUnits = 1024;                         // K <= 32768

template <int M, int UPL>
__global__ void __launch_bounds__(kThreads)
    gemv_valu_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                     const uint16_t *__restrict__ X, float *__restrict__ Y, int N, int K, int S,
                     int G, int Us, int iters) {
  constexpr int kDepth = 4;  // rows of codes in flight per wave (registers)
  // one LDS block carved by hand so that the decode table starts at offset 0: its
  // byte addresses (< 64 KiB) then need no base added before each read
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLutWords + kRedFloats + kStageBytes / 4];
  uint32_t *const lut = lds;
  float *const red = reinterpret_cast<float *>(lds + kLutWords);
  uint8_t *const stage = reinterpret_cast<uint8_t *>(lds + kLutWords + kRedFloats);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slice = wave % S;
  const int grp = wave / S;  // S * G == 8: every wave streams rows
  const int U = K >> 5;
  const int ub = slice * Us;
  const int ue = min(U, ub + Us);
  const int rows_per_block = G * iters;
  // rows are dealt round-robin over the grid: step t of group g of workgroup b
  // handles row (t * blocks + b) * G + g
  const int row0 = blockIdx.x * G;
  const int rstride = gridDim.x * G;
  const int64_t row_bytes = K >> 1;
  const int64_t row_groups = K >> 6;

  int unit[UPL];
  bool valid[UPL];
  int uload[UPL];  // a lane past its slice loads a real unit of the row; unused
#pragma unroll
  for (int i = 0; i < UPL; ++i) {
    unit[i] = ub + lane + 64 * i;
    valid[i] = unit[i] < ue;
    uload[i] = valid[i] ? unit[i] : 0;
  }
  // scales: lane l loads the scales of groups ub/2 + l (+ 64); Us is a multiple
  // of 4, so a slice owns whole groups, at most 128 of them.  Unit ub + l + 64 i
  // reads its scale from lane (l/2 + 32 i) mod 64 of load i / 2.
  constexpr int kScaleLoads = (UPL + 1) / 2;
  const int gb = ub >> 1;
  int gload[kScaleLoads];
#pragma unroll
  for (int j = 0; j < kScaleLoads; ++j) gload[j] = min(gb + lane + 64 * j, (int)row_groups - 1);
  int sperm[UPL];
#pragma unroll
  for (int i = 0; i < UPL; ++i) sperm[i] = ((lane >> 1) + 32 * (i & 1)) * 4;

  // ---- activations, pass 0: loads first (they must not queue behind codes)
  const int per_pass = kStageBytes / (M * kUnitStageBytes);
  const int npass = (U + per_pass - 1) / per_pass;
  // (row, unit) items per thread and pass: a pass holds at most kStageBytes
  constexpr int kPassItems = kStageBytes / kUnitStageBytes;
  constexpr int kItems = ((M * kMaxUnits < kPassItems ? M * kMaxUnits : kPassItems) + kThreads - 1) /
                         kThreads;
  uint4 xraw[kItems][4];
  auto load_x = [&](int u0, int nu) {
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      // no branch around the loads (see above): threads past the end load the
      // pass's last item again
      const int it = min(tid + j * kThreads, M * nu - 1);
      const int m = it / nu;
      const int uu = it - m * nu;
      const uint4 *src = reinterpret_cast<const uint4 *>(X + (int64_t)m * K + (u0 + uu) * 32);
#pragma unroll
      for (int q = 0; q < 4; ++q) xraw[j][q] = src[q];
    }
  };
  load_x(0, min(per_pass, U));

  // ---- rows: the first kDepth rows of codes go out before any set-up work
  const int row_first = min(row0 + grp, N - 1);
  // the row is the same for the whole wave: its base address lives in scalar
  // registers and each load takes a 32-bit per-lane offset (no vector address math)
  auto load_row = [&](int r, uint4 *c, uint32_t *s) {
    const int rr = __builtin_amdgcn_readfirstlane(r < N ? r : row_first);  // past the end:
    const uint8_t *crow = codes + (int64_t)rr * row_bytes;     // the wave's own first row
    const uint16_t *srow = scales + (int64_t)rr * row_groups;
#pragma unroll
    for (int i = 0; i < UPL; ++i)
      c[i] = *reinterpret_cast<const uint4 *>(crow + (uint32_t)(uload[i] * 16));
#pragma unroll
    for (int j = 0; j < kScaleLoads; ++j) s[j] = srow[(uint32_t)gload[j]];
  };
  uint4 cb[kDepth][UPL];
  uint32_t sb[kDepth][kScaleLoads];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) load_row(row0 + grp + d * rstride, cb[d], sb[d]);

  build_byte_lut(lut, tid, kThreads);

  // ---- activations: convert, stage, copy into registers (pass by pass)
  uint32_t xh[M][UPL][16];
  float xf[M][UPL];  // 2^-shift of each unit
  uint4 *stage_x = reinterpret_cast<uint4 *>(stage);                      // [4][M][per_pass]
  int *stage_sh = reinterpret_cast<int *>(stage + M * per_pass * 64);     // [M][per_pass]
  for (int pass = 0; pass < npass; ++pass) {
    const int u0 = pass * per_pass;
    const int nu = min(per_pass, U - u0);
    if (pass > 0) load_x(u0, nu);
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const int it = tid + j * kThreads;
      if (it < M * nu) {
        const int m = it / nu;
        const int uu = it - m * nu;
        uint32_t mx = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          mx = max(mx, max(max(bf16x2_absmax_bits(xraw[j][q].x), bf16x2_absmax_bits(xraw[j][q].y)),
                           max(bf16x2_absmax_bits(xraw[j][q].z), bf16x2_absmax_bits(xraw[j][q].w))));
        const int sh = f16_range_shift(mx);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          stage_x[(q * M + m) * per_pass + uu] = make_uint4(
              bf16x2_to_f16x2(xraw[j][q].x, sh), bf16x2_to_f16x2(xraw[j][q].y, sh),
              bf16x2_to_f16x2(xraw[j][q].z, sh), bf16x2_to_f16x2(xraw[j][q].w, sh));
        stage_sh[m * per_pass + uu] = sh;
      }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int i = 0; i < UPL; ++i) {
        const int uu = unit[i] - u0;
        if (valid[i] && uu >= 0 && uu < nu) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 t = stage_x[(q * M + m) * per_pass + uu];
            xh[m][i][4 * q + 0] = t.x;
            xh[m][i][4 * q + 1] = t.y;
            xh[m][i][4 * q + 2] = t.z;
            xh[m][i][4 * q + 3] = t.w;
          }
          xf[m][i] = ldexpf(1.0f, -stage_sh[m * per_pass + uu]);
        } else if (pass == 0) {
#pragma unroll
          for (int q = 0; q < 16; ++q) xh[m][i][q] = 0;
          xf[m][i] = 0.0f;
        }
      }
    if (pass + 1 < npass) __syncthreads();  // the next pass overwrites the stage
  }

  // ---- rows
  const uint32_t laneoff = (uint32_t)lane * 4u;
  auto compute_row = [&](int r, int step, const uint4 *c, const uint32_t *s) {
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.0f;
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
      const uint32_t q[4] = {c[i].x, c[i].y, c[i].z, c[i].w};
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
      // units outside the lane's slice: activations are 0, scale forced to 0
      const uint32_t sbits = (uint32_t)__builtin_amdgcn_ds_bpermute(sperm[i], (int)s[i >> 1]);
      const float sc = valid[i] ? f16_bits_to_f32(sbits) : 0.0f;
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = fmaf(p[m], sc * xf[m][i], acc[m]);
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float t = wave_sum(acc[m]);
      if (lane == 0) {
        if (S == 1)
          Y[(int64_t)m * N + r] = t;
        else
          red[(m * rows_per_block + step * G + grp) * S + slice] = t;
      }
    }
  };

  for (int it = 0; it < iters; it += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int r = row0 + grp + (it + d) * rstride;
      if (it + d < iters && r < N) compute_row(r, it + d, cb[d], sb[d]);
      load_row(r + kDepth * rstride, cb[d], sb[d]);
    }
  }
  if (S > 1) {
    __syncthreads();
    for (int t = tid; t < M * rows_per_block; t += kThreads) {
      const int m = t / rows_per_block;
      const int rl = t - m * rows_per_block;  // = step * G + group
      const int r = row0 + (rl / G) * rstride + rl % G;
      if (r < N) {
        float s = 0.0f;
        for (int sl = 0; sl < S; ++sl) s += red[t * S + sl];
        Y[(int64_t)m * N + r] = s;
      }
    }
  }
}

namespace {

struct Plan {
  int S, G, Us, upl, iters, blocks;
};

int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

constexpr int kCUs = 256;

// registers: activations take M * UPL * 16 VGPRs of the 256 an 8-wave group allows
int upl_cap(int M) { return M == 1 ? 4 : (M == 2 ? 3 : (M <= 4 ? 2 : 1)); }

// Choose slices / row groups / rows per workgroup for an (N, K, M) product.
bool plan_valu(int64_t N, int64_t K, int M, Plan &p) {
  const int U = (int)(K / 32);
  if (U > kMaxUnits) return false;
  int S = 1;  // a power of two, so that S * G covers the 8 waves exactly
  while (S < cdiv(U, 64 * upl_cap(M))) S *= 2;
  if (S > kWaves) return false;
  // widen the K split while there are too few rows to give every CU a row group
  while (2 * S <= kWaves && cdiv(N, std::max(1, kWaves / S)) < kCUs) S *= 2;
  const int G = std::max(1, kWaves / S);
  const int Us = 4 * cdiv(U, 4 * S);  // whole pairs of groups per slice
  const int upl = cdiv(Us, 64);
  // rows per workgroup: G * iters, about N / (number of CUs)
  int iters = std::max(1, cdiv(N, (int64_t)G * kCUs));
  while (iters > 1 && S > 1 && M * G * iters * S > kRedFloats) --iters;
  if (S > 1 && M * G * iters * S > kRedFloats) return false;
  p.S = S;
  p.G = G;
  p.Us = Us;
  p.upl = upl;
  p.iters = iters;
  p.blocks = cdiv(N, (int64_t)G * iters);
  return upl <= upl_cap(M) && S * G == kWaves;
}

template <int M, int UPL>
hipError_t go(const Plan &p, const uint8_t *codes, const uint16_t *scales, int N, int K,
              const uint16_t *X, float *Y, hipStream_t stream) {
  hipLaunchKernelGGL((gemv_valu_kernel<M, UPL>), dim3(p.blocks), dim3(kThreads), 0, stream, codes,
                     scales, X, Y, N, K, p.S, p.G, p.Us, p.iters);
  return hipGetLastError();
}

}  // namespace

bool valu_supported(int64_t N, int64_t K, int M) {
  Plan p;
  return M >= 1 && M <= 7 && plan_valu(N, K, M, p);
}

hipError_t launch_gemv_valu(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                            const uint16_t *X, int M, float *Y, hipStream_t stream) {
  Plan p;
  if (M < 1 || M > 7 || !plan_valu(N, K, M, p)) return hipErrorInvalidConfiguration;
  const int n = (int)N, k = (int)K;
  switch (M * 8 + p.upl) {
    case 1 * 8 + 1: return go<1, 1>(p, codes, scales, n, k, X, Y, stream);
    case 1 * 8 + 2: return go<1, 2>(p, codes, scales, n, k, X, Y, stream);
    case 1 * 8 + 3: return go<1, 3>(p, codes, scales, n, k, X, Y, stream);
    case 1 * 8 + 4: return go<1, 4>(p, codes, scales, n, k, X, Y, stream);
    case 2 * 8 + 1: return go<2, 1>(p, codes, scales, n, k, X, Y, stream);
    case 2 * 8 + 2: return go<2, 2>(p, codes, scales, n, k, X, Y, stream);
    case 2 * 8 + 3: return go<2, 3>(p, codes, scales, n, k, X, Y, stream);

    case 3 * 8 + 1: return go<3, 1>(p, codes, scales, n, k, X, Y, stream);
    case 3 * 8 + 2: return go<3, 2>(p, codes, scales, n, k, X, Y, stream);
    case 4 * 8 + 1: return go<4, 1>(p, codes, scales, n, k, X, Y, stream);
    case 4 * 8 + 2: return go<4, 2>(p, codes, scales, n, k, X, Y, stream);
    case 5 * 8 + 1: return go<5, 1>(p, codes, scales, n, k, X, Y, stream);
    case 6 * 8 + 1: return go<6, 1>(p, codes, scales, n, k, X, Y, stream);
    case 7 * 8 + 1: return go<7, 1>(p, codes, scales, n, k, X, Y, stream);
    default: return hipErrorInvalidConfiguration;
  }
}

}  // namespace nf4
