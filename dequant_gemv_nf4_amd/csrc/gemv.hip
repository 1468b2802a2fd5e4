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
// chunks) and one 32-bit scale load (two scales) that covers the wave's groups;
// each unit's scale is then fetched from the loading lane with ds_bpermute.
// Loads are buffer loads: the row offset is a scalar and the per-lane offsets are
// fixed registers, so the address unit gets no per-row vector arithmetic.  A
// short ring of rows per wave keeps the next loads in flight; no load sits behind
// a branch and no register a load in flight reads is rewritten early, so the
// compiler's waits cover exactly the row being consumed.  Order of the set-up:
// activation loads, the first code rows, then the decode table (built while the
// rows are in flight), then the activation staging.  All kernel arguments fit
// the preloaded argument registers, so nothing waits on an argument load.
//
// Decode: one v_perm_b32 turns a code byte into the LDS address of its entry in
// the bank-replicated byte table (nf4_device.h); the entry is the f16 pair
// (L[lo], L[hi]) and feeds one v_dot2_f32_f16 against (x[2j], x[2j+1]).  Two
// weights cost one perm, one LDS read and one dot per activation row; the table
// reads run two code words ahead of the dots; the group scale is applied once per
// unit in fp32.
//
// Activations are converted once per workgroup: X is read in coalesced 16-byte
// chunks, each 32-value unit is scaled by the power of two that puts its largest
// |x| in [2^14, 2^15) and converted to f16 with integer operations on the bit
// patterns (a saturating subtract of the exponent difference and a shift, two
// values per instruction), then staged in LDS with its shift; lanes copy their
// units into registers.  The shift is undone on the unit's fp32 partial.  A unit
// whose values do not all land on f16 normals (a non-zero value more than 2^28
// below the largest in binary exponent, or a largest below 2^-98) is staged as
// zeros and handled by the exact pass after the row loop.  Activation loads are
// issued before the first code loads so that the set-up does not wait behind
// them (loads return in order).
//
// Reduction: per row, lanes are summed with DPP row operations in a fixed order;
// row results wait in LDS and the S slices of a row are added in slice order
// when every row is done.  No atomics: results are bitwise reproducible.
#include <type_traits>

#include "nf4_device.h"
#include "nf4_launch.h"

namespace nf4 {

typedef __fp16 fp16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

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
constexpr int kWideUnit = 0x40000000;  // staged shift of a unit that f16 cannot hold exactly
// activation chunks (16 bytes) per thread: all of M * K fits the stage in one go
constexpr int kXChunks = (kStageBytes / kUnitStageBytes * 4 + kThreads - 1) / kThreads;

template <int M, int UPL, bool WS, bool NT>
__global__ void __launch_bounds__(kThreads)
    gemv_valu_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                     const uint16_t *__restrict__ X, float *__restrict__ Y, int N, int K,
                     int sgu, int iters, int nblocks) {
  // (13 argument words in all, so that every one arrives preloaded in scalar
  // registers: no argument load sits between a wave's start and its first loads)
  const int S = sgu & 15, G = (sgu >> 4) & 15, Us = sgu >> 8;
  // rows of codes in flight per wave (registers).  Two: measured deeper rings
  // run slower at every M (three, four and six rows at M = 1; four and six at
  // M = 2..4, e.g. 28672x4096 at M = 4 22.7 us with four, 20.9 with two), since
  // a wave whose next load waits for room at the address unit cannot go on to
  // compute rows whose data has arrived.
  constexpr int kDepth = 2;
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
  __builtin_assume(U > 0 && U <= kMaxUnits);  // lets index math use 24-bit multiplies
  const int ub = slice * Us;
  const int ue = min(U, ub + Us);
  const int rows_per_block = G * iters;
  // rows are dealt round-robin over the grid: step t of group g of workgroup b
  // handles row (t * blocks + b) * G + g
  const int row0 = blockIdx.x * G;
  const int rstride = nblocks * G;
  const int64_t row_bytes = K >> 1;
  const int64_t row_groups = K >> 6;

  int unit[UPL];
  bool valid[UPL];
  // a lane past its slice loads a unit that a lane of the same load instruction
  // reads anyway (that instruction's first unit, else the slice's first): the
  // duplicate stays within lines the instruction fetches; its data is unused
  int uload[UPL];
#pragma unroll
  for (int i = 0; i < UPL; ++i) {
    unit[i] = ub + lane + 64 * i;
    valid[i] = unit[i] < ue;
    uload[i] = valid[i] ? unit[i] : (ub + 64 * i < ue ? ub + 64 * i : ub);
  }
  // scales.  Us is a multiple of 4, so a slice owns whole groups, at most 128 of
  // them, starting at an even group gb.  Unit ub + l + 64 i needs group
  // gb + l/2 + 32 i.
  //  WS (even group count, 4-byte aligned scales): lane l loads the 32-bit word
  //    holding groups gb + 2l and gb + 2l + 1, one load per row for the whole
  //    slice; unit i reads word l/4 + 16 i from its lane and takes half (l/2) & 1.
  //  otherwise: lane l loads the 2-byte scale of group gb + l (+ 64); unit i
  //    reads it from lane (l/2 + 32 i) mod 64 of load i / 2.
  // (32-bit words matter: a 16-bit value kept in a register ring across loop
  // iterations gets repacked at the back edge, which waits for the load.)
  constexpr int kScaleLoads = WS ? 1 : (UPL + 1) / 2;
  using ScaleT = typename std::conditional<WS, uint32_t, uint16_t>::type;
  const int gb = ub >> 1;
  int gload[kScaleLoads];
#pragma unroll
  for (int j = 0; j < kScaleLoads; ++j)
    gload[j] = WS ? min((gb >> 1) + lane, (int)(row_groups >> 1) - 1)
                  : min(gb + lane + 64 * j, (int)row_groups - 1);
  int sperm[UPL];
#pragma unroll
  for (int i = 0; i < UPL; ++i)
    sperm[i] = WS ? ((lane >> 2) + 16 * i) * 4 : ((lane >> 1) + 32 * (i & 1)) * 4;

  // ---- activations, loads first (they must not queue behind codes).  X [M][K]
  // is read as 16-byte chunks of 8 values, consecutive threads on consecutive
  // chunks; chunk c is quarter c % 4 of unit (c / 4) % U of row c / (4 U).
  // Threads past the end load the last chunk again (no branch around loads).
  const int nchunks = M * U * 4;

  // A wave issues only the chunk loads it needs (the branch is uniform per wave).
  uint4 xr[kXChunks];
  const int wave_chunk0 = tid & ~63;
#pragma unroll
  for (int j = 0; j < kXChunks; ++j) {
    if (wave_chunk0 + j * kThreads < nchunks) {
      const int c = min(tid + j * kThreads, nchunks - 1);
      xr[j] = *reinterpret_cast<const uint4 *>(X + (int64_t)c * 8);
    }
  }

  // ---- rows: the first kDepth rows of codes go out before any set-up work
  const int row_first = min(row0 + grp, N - 1);
  // Buffer loads: the row offset is a scalar, the per-lane offsets are fixed
  // registers, so no vector address arithmetic runs per row and no register a
  // load in flight still reads is ever rewritten.  Matrices are below 2 GiB.
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(codes), 0, (int)((int64_t)N * row_bytes), kBufferWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(scales), 0, (int)((int64_t)N * row_groups * 2), kBufferWord3);
  int cvo[UPL], svo[kScaleLoads];
#pragma unroll
  for (int i = 0; i < UPL; ++i) cvo[i] = uload[i] * 16;
#pragma unroll
  for (int j = 0; j < kScaleLoads; ++j) svo[j] = gload[j] * (WS ? 4 : 2);
  // Step t of the wave is row r.  A step past the wave's last (or a row past N)
  // still issues its loads, so that the ring's load counts stay the same on every
  // path, but through descriptors of zero size: a buffer load out of range
  // returns zeros without a memory access.  (Re-reading a row just read instead
  // cost HBM traffic under the non-temporal hint, whose lines leave the cache
  // early: 13B q|k|v read 1.09x its bytes, 1.006x with the empty descriptors.)
  // The offset then is that of row `fallback`, a real row, so it cannot overflow.
  const __amdgpu_buffer_rsrc_t crs0 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(codes), 0, 0, kBufferWord3);
  const __amdgpu_buffer_rsrc_t srs0 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(scales), 0, 0, kBufferWord3);
  auto load_row = [&](int t, int r, int fallback, uint4 *c, ScaleT *s) {
    const bool real = t < iters && r < N;  // uniform
    const int rr = __builtin_amdgcn_readfirstlane(real ? r : fallback);
    const int coff = rr * (int)row_bytes;
    const int soff = rr * (int)row_groups * 2;
    const __amdgpu_buffer_rsrc_t cr = real ? crs : crs0;
    const __amdgpu_buffer_rsrc_t sr = real ? srs : srs0;
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
      const u32x4_nt_t v =
          __builtin_amdgcn_raw_buffer_load_b128(cr, cvo[i], coff, NT ? kLoadStream : 0);
      c[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
#pragma unroll
    for (int j = 0; j < kScaleLoads; ++j) {
      if constexpr (WS)
        s[j] = __builtin_amdgcn_raw_buffer_load_b32(sr, svo[j], soff, 0);
      else
        s[j] = __builtin_amdgcn_raw_buffer_load_b16(sr, svo[j], soff, 0);
    }
  };
  uint4 cb[kDepth][UPL];
  ScaleT sb[kDepth][kScaleLoads];
  // (rows issued in the same order as in the loop, so that the load counts the
  // compiler waits on agree on both paths into the loop)
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    load_row(d, row0 + grp + d * rstride, row_first, cb[d], sb[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // The decode table is built while the first rows are in flight: it needs no
  // memory, and the code rows, with the longest wait, go out first.
  build_byte_lut(lut, tid, kThreads);

  // ---- activations: convert, stage, copy into registers.  Each unit is scaled
  // by its own power of two (the largest |x| of its 32 values, a max over the 4
  // threads of a quad), converted to f16 and staged as stage_x[q][m][u] (uint4)
  // with its shift in stage_sh[m][u].
  uint32_t xh[M][UPL][16];
  float xf[M][UPL];  // 2^-shift of each unit
  uint4 *stage_x = reinterpret_cast<uint4 *>(stage);                 // [4][M][U]
  const int q_elems = M * U;                                         // stage_x stride of q
  int *stage_sh = reinterpret_cast<int *>(stage + M * U * 64);       // [M][U]
  // (only the chunks a wave loaded: the loop is unrolled for the largest M K,
  // and work on unloaded chunks would cost the whole wave its set-up time)
#pragma unroll
  for (int j = 0; j < kXChunks; ++j) {
    if (wave_chunk0 + j * kThreads < nchunks) {  // uniform per wave
      const int c = tid + j * kThreads;
      const uint4 v = xr[j];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      u16x2 mag[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) mag[e] = __builtin_bit_cast(u16x2, w[e] & 0x7fff7fffu);
      const uint32_t pm = __builtin_bit_cast(
          uint32_t, __builtin_elementwise_max(__builtin_elementwise_max(mag[0], mag[1]),
                                              __builtin_elementwise_max(mag[2], mag[3])));
      uint32_t mx = max(pm & 0xffffu, pm >> 16);  // the unit's largest |x|, bf16 bits
      mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0xB1, 0xf, 0xf, false));
      mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x4E, 0xf, 0xf, false));
      // Scaling by 2^(141 - Emax) puts the largest in [2^14, 2^15): on the bit
      // patterns, subtract (Emax - 29) << 7 from each magnitude (saturating, so
      // zero stays zero) and shift left by 3 to the f16 exponent and mantissa
      // fields.  Exact for a value of exponent E >= Emax - 28 (an f16 normal);
      // a non-zero magnitude below that is "lost".
      const uint32_t emax = mx >> 7;
      const uint32_t bias = ((emax - 29u) << 7) & 0xffffu;
      const u16x2 bias2 = __builtin_bit_cast(u16x2, bias * 0x10001u);
      const u16x2 thr = __builtin_bit_cast(u16x2, (bias + 0x7fu) * 0x10001u);
      uint32_t lost = 0;  // non-zero where 0 < |x| < 2^(Emax - 28 - 127)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        lost |= __builtin_bit_cast(
            uint32_t, __builtin_elementwise_sub_sat(thr, mag[e] - (u16x2){1, 1}));
      lost |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lost, 0xB1, 0xf, 0xf, false);
      lost |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lost, 0x4E, 0xf, 0xf, false);
      if (c < nchunks) {  // nchunks is a multiple of 4: a quad is valid or not as a whole
        // wide: some value would be lost, or the largest is below 2^-98 (the
        // shift would leave the subtraction's range); all-zero units are exact
        const bool wide = mx != 0 && (emax < 29u || lost != 0);
        const int q = c & 3;
        const int mu = c >> 2;  // m * U + u
        // a unit f16 cannot hold exactly is staged as zeros: the row loop adds
        // nothing for it, and the exact pass after the loop adds its terms
        uint4 f = make_uint4(0u, 0u, 0u, 0u);
        if (!wide) {
          uint32_t h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            h[e] = __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(mag[e], bias2)
                                                    << (u16x2){3, 3}) |
                   (w[e] & 0x80008000u);
          f = make_uint4(h[0], h[1], h[2], h[3]);
        }
        stage_x[q * q_elems + mu] = f;
        if (q == 0) stage_sh[mu] = wide ? kWideUnit : (int)(141u - emax);
      }
    }
  }
  __syncthreads();
  // (the block strides are scalars: kept out of per-lane 64-bit multiply-adds,
  // which would read the neighbour of an offset register, here a ring register
  // with a load in flight, and wait for it)
  const int rows_stride = __builtin_amdgcn_readfirstlane(U);
  const int q_stride = __builtin_amdgcn_readfirstlane(M * U);
  uint32_t wide_bits = 0;  // bit m * UPL + i: unit i of activation row m is wide
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
      if (valid[i]) {
        const uint4 *xs = stage_x + unit[i] + m * rows_stride;
#pragma unroll
        for (int q = 0; q < 4; ++q, xs += q_stride) {
          const uint4 t = *xs;
          xh[m][i][4 * q + 0] = t.x;
          xh[m][i][4 * q + 1] = t.y;
          xh[m][i][4 * q + 2] = t.z;
          xh[m][i][4 * q + 3] = t.w;
        }
        const int sh = stage_sh[m * rows_stride + unit[i]];
        if (sh == kWideUnit) wide_bits |= 1u << (m * UPL + i);
        xf[m][i] = sh == kWideUnit ? 0.0f : ldexpf(1.0f, -sh);
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) xh[m][i][q] = 0;
        xf[m][i] = 0.0f;
      }
    }

  // ---- rows
  const uint32_t laneoff = lut_lane_offset(lane);
  auto compute_row = [&](int r, int step, const uint4 *c, const ScaleT *s) {
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.0f;
    // units outside the lane's slice: activations are 0, scale forced to 0
    float sc[UPL];
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
      uint32_t sbits;
      if constexpr (WS) {
        const uint32_t w = (uint32_t)__builtin_amdgcn_ds_bpermute(sperm[i], (int)s[0]);
        sbits = (lane & 2) ? (w >> 16) : (w & 0xffffu);
      } else {
        sbits = (uint32_t)__builtin_amdgcn_ds_bpermute(sperm[i], (int)(uint32_t)s[i >> 1]);
      }
      sc[i] = valid[i] ? f16_bits_to_f32(sbits) : 0.0f;
    }
    // table reads run two code words ahead of the dot products that consume them,
    // so the LDS latency overlaps the arithmetic
    constexpr int kWords = 4 * UPL;
    uint32_t q[kWords];
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
      q[4 * i + 0] = c[i].x;
      q[4 * i + 1] = c[i].y;
      q[4 * i + 2] = c[i].z;
      q[4 * i + 3] = c[i].w;
    }
    uint32_t lv[3][4];
    auto fetch = [&](int t, uint32_t *dst) __attribute__((always_inline)) {
      dst[0] = lds_load_u32(lut, lut_addr<0>(q[t], laneoff));
      dst[1] = lds_load_u32(lut, lut_addr<1>(q[t], laneoff));
      dst[2] = lds_load_u32(lut, lut_addr<2>(q[t], laneoff));
      dst[3] = lds_load_u32(lut, lut_addr<3>(q[t], laneoff));
    };
    fetch(0, lv[0]);
    if (kWords > 1) fetch(1, lv[1]);
    float p[M];
#pragma unroll
    for (int t = 0; t < kWords; ++t) {
      if (t + 2 < kWords) fetch(t + 2, lv[(t + 2) % 3]);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the dots below
      const int i = t >> 2, j = t & 3;
      if (j == 0) {
#pragma unroll
        for (int m = 0; m < M; ++m) p[m] = 0.0f;
      }
      const uint32_t *l = lv[t % 3];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        p[m] = dot2(l[0], xh[m][i][4 * j + 0], p[m]);
        p[m] = dot2(l[1], xh[m][i][4 * j + 1], p[m]);
        p[m] = dot2(l[2], xh[m][i][4 * j + 2], p[m]);
        p[m] = dot2(l[3], xh[m][i][4 * j + 3], p[m]);
      }
      if (j == 3) {
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m] = fmaf(p[m], sc[i] * xf[m][i], acc[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      // results wait in LDS until every row is done: a store inside the loop
      // would make later register reuse wait for it, and with it for every
      // load issued before it
      const float t = wave_sum(acc[m]);
      if (lane == 0) red[(m * rows_per_block + step * G + grp) * S + slice] = t;
    }
  };

  // Whole rounds of kDepth rows run without branches (rows past N compute on the
  // zeros their loads returned and are never stored), so the load waits stay
  // exact across the loop's back edge; the last partial round follows.
  int it = 0;
  for (; it + kDepth <= iters; it += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int r = row0 + grp + (it + d) * rstride;
      compute_row(r, it + d, cb[d], sb[d]);
      load_row(it + d + kDepth, r + kDepth * rstride, min(r, N - 1), cb[d], sb[d]);
    }
  }
#pragma unroll
  for (int d = 0; d < kDepth - 1; ++d)
    if (it + d < iters) compute_row(row0 + grp + (it + d) * rstride, it + d, cb[d], sb[d]);

  // ---- exact pass, only in waves holding a unit that f16 cannot hold exactly
  // (its activations span more than 2^28 in exponent; about 1e-8 of the units
  // of N(0, 1) data).  The row loop added nothing for such a unit; here each of
  // its weights is computed as (f16 level x fp32 group scale), exact, times the
  // bf16 activation with one fp32 fma, so every term is w~ * x rounded once and
  // no partial sum is formed before the scale is applied.  The wave's row sums
  // are then added to the row partials it left in LDS.
  if (__builtin_amdgcn_ballot_w64(wide_bits != 0) != 0) {
    for (int t = 0; t < iters; ++t) {
      const int r = row0 + grp + t * rstride;
      if (r >= N) break;  // uniform: rows grow with t
      float acc[M];
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = 0.0f;
#pragma unroll
      for (int i = 0; i < UPL; ++i) {
        uint32_t mine = 0;
#pragma unroll
        for (int m = 0; m < M; ++m) mine |= wide_bits & (1u << (m * UPL + i));
        if (mine) {
          const uint4 c = *reinterpret_cast<const uint4 *>(codes + (int64_t)r * row_bytes +
                                                           16 * unit[i]);
          const float sc = f16_bits_to_f32(scales[(int64_t)r * row_groups + (unit[i] >> 1)]);
          const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t lv[4];
            lv[0] = lds_load_u32(lut, lut_addr<0>(cw[j], laneoff));
            lv[1] = lds_load_u32(lut, lut_addr<1>(cw[j], laneoff));
            lv[2] = lds_load_u32(lut, lut_addr<2>(cw[j], laneoff));
            lv[3] = lds_load_u32(lut, lut_addr<3>(cw[j], laneoff));
#pragma unroll
            for (int m = 0; m < M; ++m) {
              if (wide_bits & (1u << (m * UPL + i))) {
                const uint32_t *xw =
                    reinterpret_cast<const uint32_t *>(X + (int64_t)m * K + 32 * unit[i]) + 4 * j;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                  const uint32_t x2 = xw[b];
                  acc[m] = fmaf(f16_bits_to_f32(lv[b] & 0xffffu) * sc, bf16_lo(x2), acc[m]);
                  acc[m] = fmaf(f16_bits_to_f32(lv[b] >> 16) * sc, bf16_hi(x2), acc[m]);
                }
              }
            }
          }
        }
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float tsum = wave_sum(acc[m]);
        if (lane == 0) red[(m * rows_per_block + t * G + grp) * S + slice] += tsum;
      }
    }
  }
  {
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
  if (U > kMaxUnits || M * U * kUnitStageBytes > kStageBytes) return false;
  int S = 1;  // a power of two, so that S * G covers the 8 waves exactly
  while (S < cdiv(U, 64 * upl_cap(M))) S *= 2;
  // where four units per lane fit a slice exactly, two units per lane in twice
  // the slices (half the activation registers, the same lane use) ran faster:
  // 8192x8192 9.5 -> 9.0 us, 57344x8192 42.4 -> 39.9 us
  if (M == 1 && U == 256 * S && 2 * S <= kWaves) S *= 2;
  if (S > kWaves) return false;
  // widen the K split while there are too few rows to give every CU a row group
  while (2 * S <= kWaves && cdiv(N, std::max(1, kWaves / S)) < kCUs) S *= 2;
  const int G = std::max(1, kWaves / S);
  const int Us = 4 * cdiv(U, 4 * S);  // whole pairs of groups per slice
  const int upl = cdiv(Us, 64);
  // rows per workgroup: G * iters, about N / (number of CUs)
  int iters = std::max(1, cdiv(N, (int64_t)G * kCUs));
  while (iters > 1 && M * G * iters * S > kRedFloats) --iters;
  if (M * G * iters * S > kRedFloats) return false;
  p.S = S;
  p.G = G;
  p.Us = Us;
  p.upl = upl;
  p.iters = iters;
  p.blocks = cdiv(N, (int64_t)G * iters);
  return upl <= upl_cap(M) && S * G == kWaves;
}

template <int M, int UPL, bool WS, bool NT>
void launch(const Plan &p, const uint8_t *codes, const uint16_t *scales, int N, int K,
            const uint16_t *X, float *Y, hipStream_t stream) {
  hipLaunchKernelGGL((gemv_valu_kernel<M, UPL, WS, NT>), dim3(p.blocks), dim3(kThreads), 0, stream,
                     codes, scales, X, Y, N, K, p.S | p.G << 4 | p.Us << 8, p.iters, p.blocks);
}

template <int M, int UPL>
hipError_t go(const Plan &p, const uint8_t *codes, const uint16_t *scales, int N, int K,
              const uint16_t *X, float *Y, hipStream_t stream) {
  // 32-bit scale words need an even group count and a 4-byte aligned array
  const bool ws = ((K >> 6) % 2 == 0) && ((reinterpret_cast<uintptr_t>(scales) & 3) == 0);
  // Code loads carry the non-temporal hint when each wave streams many rows:
  // measured on the Llama shapes, it gains 1-5 % at 8 or more rows per wave and
  // loses 1-5 % below (4096x11008: 7.58 us plain vs 7.90 us hinted).
  const bool nt = p.iters >= 8;
  if (ws && nt) launch<M, UPL, true, true>(p, codes, scales, N, K, X, Y, stream);
  else if (ws) launch<M, UPL, true, false>(p, codes, scales, N, K, X, Y, stream);
  else if (nt) launch<M, UPL, false, true>(p, codes, scales, N, K, X, Y, stream);
  else launch<M, UPL, false, false>(p, codes, scales, N, K, X, Y, stream);
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
