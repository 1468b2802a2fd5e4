// gemm_prefill.hip -- fused NF4 dequant product for prefill batches of any
// size on the matrix cores (gfx950, v_mfma_f32_32x32x16_bf16).
//
// Computes Y[m][n] = sum_k L[code(n,k)] * s(n,k/64) * X[m][k].  Sources:
// deep-fold README, "Method" (prefill runs the NF4 product on chunks of
// positions, the weights rebuilt into matrix-core register fragments and never
// written out); Trapetum overview, "The fine print" (prefill saves memory
// traffic, not time: once M is large the product is bound by the matrix cores,
// not by the weight stream).
//
// Tiling.  A workgroup owns a (64 RM) x (64 CN) tile of Y.  Its waves form KS
// K-splits of 4 waves (2 x 2); split q walks the scale groups of its share of K,
// one group (64 k) per step, and each of its waves owns RM x CN tiles of 32 x 32.
// Where the group count allows (SB: a multiple of 8 KS groups per workgroup), the
// share is the q-th KS-th of the workgroup's range, and a lane reads the scales
// of 8 steps in one 16-byte load (a scale load touches one line per column
// whatever its width, so per-step 2-byte loads cost 8 times the lines; 5-7 %
// faster on the Llama-3.1-8B shapes at M = 128..512); otherwise split q takes
// the groups q, q + KS, ... and one 2-byte scale per step.  Per step:
//   - the split stages the activation tile [64 RM][64] in LDS as it is (bf16,
//     rows padded to 144 bytes so that fragment reads do not collide in banks);
//   - each wave loads the 32 code bytes of the group for each of its columns
//     (lane (n, h) the 16 bytes of k = 32h .. 32h+31) and decodes them through
//     an LDS table straight into B fragments: each level split into bf16 hi +
//     lo (nf4_split.h), one table read per code byte and half;
//   - MFMA 32 x 32 x 16: A = activations (lane l: row l % 32, 8 k), B = weights
//     (lane l: column l % 32, the same 8 k), two MFMAs (hi, lo) per slice into
//     the group's tile.  Slice s of the group gives lane half h the
//     k = 32h + 8s .. +7, so a lane's code word s and its 16 bytes of staged
//     activations line up without any shuffling;
//   - the group's 32 x 32 tile (fp32) is multiplied by the column's scale (one
//     per lane) and added to the fp32 accumulator.  No weight is rounded
//     together with its scale and the activations are exact, so every product
//     is exact in fp32.
// A register ring keeps the loads of the next P steps (activations, codes,
// scales) in flight; the activation stage is double-buffered in LDS, one
// barrier a step.  At the end the splits' tiles are added in split order.
// Rows past M and columns past N re-read the last valid row or column and are
// never stored.  Without a workspace there is no cross-workgroup traffic; with
// one (nf4_gemm_prefill_ws) K is also split over workgroups whose partial tiles
// meet in the workspace and are added in split order by the last to finish (the
// end of the kernel).  Either way the results are bitwise reproducible.
#include <utility>

#include "nf4_device.h"
#include "nf4_launch.h"
#include "nf4_split.h"

namespace nf4 {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPThreads = 256;  // 4 waves: 2 (rows) x 2 (columns)
constexpr int kXRow = 144;      // bytes per staged activation row: 64 bf16 + 16 B pad

__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Decode table: entry b (b = 16 h + j, j = low nibble = even k) is 256 bytes at
// 256 b: 32 copies of hi[j] | hi[h] << 16, then 32 copies of lo[j] | lo[h] << 16,
// 4 bytes apart, so lane l reads copy l % 32 of either half (no two lanes of a
// half-wave share a bank) at (b << 8) | 4 (l % 32), the lo pair 128 bytes on.
// Wave w writes the entries of each high nibble h with h % nwaves == w: 16
// entries = 256 uint4, 4 per lane; store (i, lane) covers entry 16 h + 4 i +
// lane / 16, uint4 lane % 16 (hi below 8), so the high level is a constant of
// the unrolled loop and the low level a 4-way choice fixed per lane.  64 KiB.
__device__ __forceinline__ void build_hilo_lut(uint32_t *lut, int tid, int nthreads) {
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwaves = nthreads >> 6;
  // the 4-way choice as a shift of four packed 16-bit constants (a select chain
  // would be turned into a table in memory)
  const uint32_t sh = 16u * ((uint32_t)lane >> 4);
  const bool hi = (lane & 15) < 8;
  uint32_t low[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    constexpr auto pack4 = [](const uint32_t *v) {
      return (uint64_t)v[0] | (uint64_t)v[1] << 16 | (uint64_t)v[2] << 32 | (uint64_t)v[3] << 48;
    };
    const uint32_t lh = (uint32_t)(pack4(&kSplit.hi[4 * i]) >> sh) & 0xffffu;
    const uint32_t ll = (uint32_t)(pack4(&kSplit.lo[4 * i]) >> sh) & 0xffffu;
    low[i] = hi ? lh : ll;
  }
  uint4 *L4 = reinterpret_cast<uint4 *>(lut);
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    if (h % nwaves == wave) {
      const uint32_t top = (hi ? kSplit.hi[h] : kSplit.lo[h]) << 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t e = low[i] | top;
        L4[h * 256 + i * 64 + lane] = make_uint4(e, e, e, e);
      }
    }
  }
}

// v_perm_b32 selector: (byte j of the code word) << 8 | (low byte of laneoff)
template <int j>
__device__ __forceinline__ uint32_t hilo_addr(uint32_t codeword, uint32_t laneoff) {
  constexpr uint32_t sel = 0x0c0c0000u | ((4u + j) << 8);
  return __builtin_amdgcn_perm(codeword, laneoff, sel);
}

template <typename F, int... d>
__device__ __forceinline__ void for_slots(F &&f, std::integer_sequence<int, d...>) {
  (f(std::integral_constant<int, d>{}), ...);
}

}  // namespace

// KS K-splits of 4 waves each over the same output tile: split q takes groups q,
// q + KS, q + 2 KS, ... or (SB) the q-th KS-th of the workgroup's groups, and the
// splits' tiles are added in split order at the end.
template <int RM, int CN, int P, int KS, bool SB>
__global__ void __launch_bounds__(kPThreads * KS)
    gemm_prefill_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                        const uint16_t *__restrict__ X, float *__restrict__ Y, int N, int K,
                        int M, int S, uint32_t *__restrict__ cnt) {
  constexpr int BM = 64 * RM;
  constexpr int kXChunks = BM * 8 / kPThreads;  // 16-byte activation chunks per thread
  constexpr int kStage = BM * kXRow;            // bytes of one activation buffer
  constexpr int kStageWords = KS * 2 * kStage / 4;
  constexpr int kRedWords = KS > 1 ? 4 * RM * CN * 16 * 64 : 0;
  static_assert(kRedWords <= kStageWords, "the split reduction reuses the activation stage");
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLutWords + kStageWords];
  uint32_t *const lut = lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = wave >> 2;        // K-split of this wave
  const int tq = tid & (kPThreads - 1);  // thread index within the split
  const int wr = (wave >> 1) & 1, wc = wave & 1;
  const int col = lane & 31, h = lane >> 5;
  const int NG = K >> 6;
  // workgroup K-split blockIdx.z of S takes the groups [g0, g0 + ng)
  const int zs = blockIdx.z;
  // SB: ranges in whole blocks of 8 KS groups, and split q takes the q-th KS-th of
  // its workgroup's range (8 consecutive groups per 16-byte scale load)
  const int GU = SB ? 8 * KS : 1;
  const int g0 = GU * (int)((int64_t)zs * (NG / GU) / S);
  const int ng = GU * (int)((int64_t)(zs + 1) * (NG / GU) / S) - g0;
  const int nsteps = (ng + KS - 1) / KS;  // the same for every split (barriers match)
  const int gq0 = SB ? g0 + split * nsteps : 0;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * (64 * CN);
  // this split's activation stages [2][BM][kXRow]
  uint8_t *const xs = reinterpret_cast<uint8_t *>(lds + kLutWords) + split * 2 * kStage;

  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(codes), 0, (int)((int64_t)N * (K >> 1)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(scales), 0, (int)((int64_t)N * NG * 2), kBufferWord3);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(X), 0, (int)((int64_t)M * K * 2), kBufferWord3);

  // activation chunk j of this thread: row (tq / 8) + 32 j of the tile, k 8 (tq % 8)
  const int part = tq & 7;
  int xvo[kXChunks];
#pragma unroll
  for (int j = 0; j < kXChunks; ++j)
    xvo[j] = (min(m0 + (tq >> 3) + 32 * j, M - 1) * K + 8 * part) * 2;
  int cvo[CN], svo[CN];
#pragma unroll
  for (int c = 0; c < CN; ++c) {
    const int n = min(n0 + 32 * CN * wc + 32 * c + col, N - 1);
    cvo[c] = n * (K >> 1) + 16 * h;
    svo[c] = n * NG * 2;
  }

  // a ring of P steps in flight: slot d holds the loads of steps j = d (mod P);
  // step j of split q is group KS j + q (SB: group j of the split's range; past
  // the end: the last group again)
  u32x4_t xr[P][kXChunks];
  u32x4_t cr[P][CN];
  uint32_t sr[P][CN];
  auto group_of = [&](int j) __attribute__((always_inline)) {
    if constexpr (SB) return __builtin_amdgcn_readfirstlane(gq0 + min(j, nsteps - 1));
    return __builtin_amdgcn_readfirstlane(g0 + min(KS * j + split, ng - 1));
  };
  // SB: the scales of 8 steps per 16-byte load; scur serves the steps of block
  // j / 8, snxt holds block j / 8 + 1 (issued 8 steps ahead; lanes n and n + 32
  // load the same column)
  u32x4_t scur[CN], snxt[CN];
  auto load_sblock = [&](int blk) __attribute__((always_inline)) {
    const int gb = __builtin_amdgcn_readfirstlane(gq0 + 8 * min(blk, (nsteps >> 3) - 1));
#pragma unroll
    for (int c = 0; c < CN; ++c)
      snxt[c] = __builtin_amdgcn_raw_buffer_load_b128(srs, svo[c], 2 * gb, 0);
  };
  auto load_x = [&](auto slot, int j) __attribute__((always_inline)) {
    constexpr int d = decltype(slot)::value;
    const int gs = group_of(j);
#pragma unroll
    for (int i = 0; i < kXChunks; ++i)
      xr[d][i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xvo[i], 128 * gs, 0);
  };
  auto load_w = [&](auto slot, int j) __attribute__((always_inline)) {
    constexpr int d = decltype(slot)::value;
    const int gs = group_of(j);
#pragma unroll
    for (int c = 0; c < CN; ++c) {
      cr[d][c] = __builtin_amdgcn_raw_buffer_load_b128(crs, cvo[c], 32 * gs, kLoadStream);
      if constexpr (!SB) sr[d][c] = __builtin_amdgcn_raw_buffer_load_b16(srs, svo[c], 2 * gs, 0);
    }
  };

  f32x16_t acc[RM][CN];
#pragma unroll
  for (int r = 0; r < RM; ++r)
#pragma unroll
    for (int c = 0; c < CN; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.f;

  const uint32_t laneoff = 4u * (lane & 31);
  // one step: stage the activations, refill the slot's activations with step
  // j + P, multiply, refill the slot's codes and scales
  auto step = [&](auto slot, int j) __attribute__((always_inline)) {
    constexpr int d = decltype(slot)::value;
    uint8_t *const xb = xs + (d & 1) * kStage;
#pragma unroll
    for (int i = 0; i < kXChunks; ++i)
      *reinterpret_cast<u32x4_t *>(xb + ((tq >> 3) + 32 * i) * kXRow + 16 * part) = xr[d][i];
    __syncthreads();
    load_x(slot, j + P);
    if constexpr (SB) {
      if ((j & 7) == 0) {
#pragma unroll
        for (int c = 0; c < CN; ++c) scur[c] = snxt[c];
        load_sblock((j >> 3) + 1);
      }
    }
    // the last step of a split with fewer groups only keeps the barriers in step
    if (SB || KS * j + split < ng) {
      f32x16_t t[RM][CN];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4_t a[RM], bh[CN], bl[CN];
#pragma unroll
        for (int r = 0; r < RM; ++r)
          a[r] = *reinterpret_cast<const u32x4_t *>(xb + (32 * RM * wr + 32 * r + col) * kXRow +
                                                     64 * h + 16 * s);
#pragma unroll
        for (int c = 0; c < CN; ++c) {
          const uint32_t w = cr[d][c][s];
          const uint32_t e0 = hilo_addr<0>(w, laneoff), e1 = hilo_addr<1>(w, laneoff);
          const uint32_t e2 = hilo_addr<2>(w, laneoff), e3 = hilo_addr<3>(w, laneoff);
          bh[c] = u32x4_t{lds_load_u32(lut, e0), lds_load_u32(lut, e1), lds_load_u32(lut, e2),
                          lds_load_u32(lut, e3)};
          bl[c] = u32x4_t{lds_load_u32(lut, e0 + 128), lds_load_u32(lut, e1 + 128),
                          lds_load_u32(lut, e2 + 128), lds_load_u32(lut, e3 + 128)};
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
            t[r][c] = mfma32(a[r], bh[c], z);
            t[r][c] = mfma32(a[r], bl[c], t[r][c]);
          }
      }
      // the group's tile times the column's scale (a lane holds one column)
#pragma unroll
      for (int c = 0; c < CN; ++c) {
        float sc;
        if constexpr (SB) {
          const int e = (j >> 1) & 3;
          const uint32_t w = e == 0 ? scur[c][0] : e == 1 ? scur[c][1] : e == 2 ? scur[c][2] : scur[c][3];
          sc = f16_bits_to_f32((j & 1) ? w >> 16 : w & 0xffffu);
        } else {
          sc = f16_bits_to_f32(sr[d][c]);
        }
#pragma unroll
        for (int r = 0; r < RM; ++r)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[r][c][i] = fmaf(t[r][c][i], sc, acc[r][c][i]);
      }
    }
    load_w(slot, j + P);
    __builtin_amdgcn_sched_barrier(0);  // refills stay after the step that frees the slot
  };

  // (issued in the loop's order: activations, then codes and scales, per step)
  for_slots(
      [&](auto slot) __attribute__((always_inline)) {
        load_x(slot, decltype(slot)::value);
        load_w(slot, decltype(slot)::value);
        __builtin_amdgcn_sched_barrier(0);
      },
      std::make_integer_sequence<int, P>{});
  if constexpr (SB) load_sblock(0);
  build_hilo_lut(lut, tid, kPThreads * KS);

  int j = 0;
  for (; j + P <= nsteps; j += P)
    for_slots([&](auto slot) __attribute__((always_inline)) { step(slot, j + decltype(slot)::value); },
              std::make_integer_sequence<int, P>{});
  for_slots(
      [&](auto slot) __attribute__((always_inline)) {
        if (j + decltype(slot)::value < nsteps) step(slot, j + decltype(slot)::value);
      },
      std::make_integer_sequence<int, P>{});

  if constexpr (KS > 1) {
    // splits 1.. park their tiles in the (now idle) stage; split 0 adds them in order
    float *const red = reinterpret_cast<float *>(lds + kLutWords);
    const int wq = wave & 3;
    for (int q = 1; q < KS; ++q) {
      __syncthreads();
      if (split == q) {
#pragma unroll
        for (int r = 0; r < RM; ++r)
#pragma unroll
          for (int c = 0; c < CN; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              red[(((wq * RM + r) * CN + c) * 16 + i) * 64 + lane] = acc[r][c][i];
      }
      __syncthreads();
      if (split == 0) {
#pragma unroll
        for (int r = 0; r < RM; ++r)
#pragma unroll
          for (int c = 0; c < CN; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              acc[r][c][i] += red[(((wq * RM + r) * CN + c) * 16 + i) * 64 + lane];
      }
    }
  }

  constexpr int BN = 64 * CN;
  if (S == 1) {
    if (split != 0) return;
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
    return;
  }
  // Workgroup K-splits: split 0 of each writes its tile to the workspace with
  // agent-coherent stores; the last of the S workgroups of this tile to finish
  // (a counter per tile, re-armed by that workgroup) adds the S tiles in split
  // order, so the bits do not depend on which finishes last.
  // the workspace: the counter area, then the partial tiles (the address and the
  // tile index are derived here, so that every argument fits the preloaded
  // argument registers)
  const int tiles_n = (N + BN - 1) / BN;
  float *const partial = reinterpret_cast<float *>(reinterpret_cast<char *>(cnt) + kSplitCounterBytes);
  const int64_t tile = (int64_t)blockIdx.y * tiles_n + blockIdx.x;
  if (split == 0) {
    float *const mine = partial + (tile * S + zs) * (BM * BN);
#pragma unroll
    for (int r = 0; r < RM; ++r)
#pragma unroll
      for (int c = 0; c < CN; ++c) {
        const int nl = 32 * CN * wc + 32 * c + col;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ml = 32 * RM * wr + 32 * r + 8 * (i >> 2) + 4 * h + (i & 3);
          __hip_atomic_store(mine + ml * BN + nl, acc[r][c][i], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      }
  }
  // Ordering (the AMDGPU memory model's release/acquire sequences, restricted to
  // the locations involved): every partial is written with an agent-scope
  // atomic store, which is performed at the agent's coherence point rather than
  // in one XCD's L2, so no L2 write-back is needed to publish it; vmcnt(0)
  // waits until this thread's stores are performed there, and the barrier
  // orders every thread's wait before the counter increment.  The workgroup that
  // sees the final count reads the partials with agent-scope atomic loads, which
  // also go to the coherence point (no stale L2 line can answer them, so no L2
  // invalidate is needed), and it issues them only after the increment returned.
  __shared__ int last;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's stores are done
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == (uint32_t)(S - 1);
    if (last) __hip_atomic_store(cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last) return;
  const float *const all = partial + tile * S * (BM * BN);
  for (int e = tid; e < BM * BN; e += kPThreads * KS) {
    const int m = m0 + e / BN, n = n0 + e % BN;
    if (m >= M || n >= N) continue;
    float sum = __hip_atomic_load(all + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int q = 1; q < S; ++q)
      sum += __hip_atomic_load(all + (int64_t)q * (BM * BN) + e, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    Y[(int64_t)m * N + n] = sum;
  }
}

namespace {

int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

constexpr int kCUs = 256;

template <int RM, int CN, int P, int KS>
hipError_t go_prefill(const uint8_t *codes, const uint16_t *scales, int N, int K,
                      const uint16_t *X, int M, float *Y, int S, uint32_t *cnt, float *partial,
                      hipStream_t stream) {
  const dim3 grid(cdiv(N, 64 * CN), cdiv(M, 64 * RM), S);
  const int NG = K >> 6;
  // 16-byte scale loads need whole blocks of 8 KS groups per workgroup and 16-byte
  // aligned scales
  if (NG % (8 * KS) == 0 && S <= NG / (8 * KS) && (reinterpret_cast<uintptr_t>(scales) & 15) == 0)
    hipLaunchKernelGGL((gemm_prefill_kernel<RM, CN, P, KS, true>), grid, dim3(kPThreads * KS), 0,
                       stream, codes, scales, X, Y, N, K, M, S, cnt);
  else
    hipLaunchKernelGGL((gemm_prefill_kernel<RM, CN, P, KS, false>), grid, dim3(kPThreads * KS), 0,
                       stream, codes, scales, X, Y, N, K, M, S, cnt);
  (void)partial;  // the kernel derives the same address from cnt
  return hipGetLastError();
}

// Workgroup tile (64 RM x 64 CN), in-workgroup K-splits KS and workgroup
// K-splits S.  Larger tiles read each weight and activation byte for more
// outputs, and pay even with fewer workgroups than CUs: a sweep of the tiles
// and S on the Llama-3.1-8B shapes (M = 64 .. 512) picked 128 x 128 from M = 128
// once the grid reaches about 180 workgroups (gate|up at M = 128: 134 -> 83 us;
// q|k|v at M = 512, 192 workgroups: 101 -> 71 us), and for K >= 8192 at M >= 512
// with workgroup K-splits filling the CUs (down at M = 512: 201 -> 141 us); then
// 64 x 128 from M = 128 at about 180 workgroups (q|k|v at M = 256: 56 -> 47 us);
// else 64 x 64 (at M = 64 it beats 64 x 128 even on 28672 rows).  P (steps in
// flight, even: the LDS stage alternates) and KS are as large as the registers
// allow.  With a workspace, a grid of fewer than 256 workgroups is multiplied by
// the largest S that keeps it within 256 (and at least two steps per wave).
struct PrefillPlan {
  int RM, CN, KS, S;
  int64_t tiles;
};

PrefillPlan plan_prefill(int n, int k, int m, bool split) {
  auto blocks = [&](int bm, int bn) { return (int64_t)cdiv(n, bn) * cdiv(m, bm); };
  constexpr int kEnough = 180;  // workgroups for a large tile to pay
  PrefillPlan p;
  if (m >= 128 && (blocks(128, 128) >= kEnough || (m >= 512 && k >= 8192)))
    p = PrefillPlan{2, 2, 2, 1, blocks(128, 128)};
  else if (m >= 128 && blocks(64, 128) >= kEnough)
    p = PrefillPlan{1, 2, 2, 1, blocks(64, 128)};
  else
    p = PrefillPlan{1, 1, 4, 1, blocks(64, 64)};
  if (split && p.tiles < kCUs) {
    // whole rounds only: a second, partial round of workgroups costs more than
    // the split saves (measured on q|k|v at M = 128)
    const int smax = (k >> 6) / (2 * p.KS);
    p.S = std::max(1, std::min((int)(kCUs / p.tiles), smax));
  }
  return p;
}

int64_t prefill_workspace_bytes(const PrefillPlan &p) {
  if (p.S == 1) return 0;
  return kSplitCounterBytes + (int64_t)p.tiles * p.S * (64 * p.RM) * (64 * p.CN) * 4;
}

}  // namespace

int64_t gemm_prefill_workspace_bytes(int64_t N, int64_t K, int64_t M) {
  return prefill_workspace_bytes(plan_prefill((int)N, (int)K, (int)M, true));
}

hipError_t launch_gemm_prefill(const uint8_t *codes, const uint16_t *scales, int64_t N,
                               int64_t K, const uint16_t *X, int64_t M, float *Y, void *workspace,
                               int64_t workspace_bytes, hipStream_t stream) {
  const int n = (int)N, k = (int)K, m = (int)M;
  const PrefillPlan p = plan_prefill(n, k, m, workspace != nullptr);
  uint32_t *cnt = nullptr;
  float *partial = nullptr;
  if (p.S > 1) {
    if (workspace_bytes < prefill_workspace_bytes(p)) return hipErrorInvalidValue;
    cnt = static_cast<uint32_t *>(workspace);
    partial = reinterpret_cast<float *>(static_cast<char *>(workspace) + kSplitCounterBytes);
  }
  if (p.RM == 2) return go_prefill<2, 2, 2, 2>(codes, scales, n, k, X, m, Y, p.S, cnt, partial, stream);
  if (p.CN == 2) return go_prefill<1, 2, 2, 2>(codes, scales, n, k, X, m, Y, p.S, cnt, partial, stream);
  return go_prefill<1, 1, 2, 4>(codes, scales, n, k, X, m, Y, p.S, cnt, partial, stream);
}

}  // namespace nf4
