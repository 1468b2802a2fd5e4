// embed.hip -- packed embedding rows: only the requested rows of an NF4 matrix
// are decoded, into bf16 (deep-fold README, "Method": embeddings decode only
// the requested rows; the result feeds the first linear layer as activations).
//
// out[t][k] = bf16(L[code(id,k)] * s(id, k/64)), id = ids[t], one rounding of
// the exact product: p = the fp32 product, e = its exact error (one fma); p
// decides the bf16 rounding except on an exact bf16 tie, where the sign of e
// says on which side of it the exact product lies.  One thread writes 8
// outputs of a row (one 32-bit word of codes, 16 bytes of output), in 1, 2, 4
// or 8 consecutive rows.  The rows are written with non-temporal stores (they
// are 80 % of the bytes and are not read back here; T = 32768: 78 -> 65 us).
// An id outside [0, N) gives a zero row and sets bit NF4_EMBED_BAD_ID of the
// status word.
#include "nf4_device.h"
#include "nf4_launch.h"

namespace nf4 {

// bf16 bits of the exact value p + e (p = fp32 rounding of a product, e its
// exact rounding error); NaN gives the quiet NaN 0x7FC0.
__device__ __forceinline__ uint32_t bf16_of_exact(float p, float e) {
  const uint32_t b = __float_as_uint(p);
  if ((b & 0x7F800000u) == 0x7F800000u) return (b & 0x007FFFFFu) ? 0x7FC0u : (b >> 16);
  const uint32_t lo = b & 0xFFFFu;
  const uint32_t r = b >> 16;
  bool up;
  if (lo != 0x8000u)
    up = lo > 0x8000u;
  else if (e != 0.0f)
    up = (e > 0.0f) == (p > 0.0f);  // the exact value lies beyond the tie
  else
    up = (r & 1u) != 0u;            // exact tie: to even
  return r + (up ? 1u : 0u);
}

// levels from a 16-entry table in LDS: the entries sit in 16 distinct banks, so
// lanes reading different levels never conflict and equal ones broadcast
__device__ __forceinline__ uint32_t embed_pair(const float *lv, uint32_t byte, float s) {
  const float l0 = lv[byte & 15u], l1 = lv[byte >> 4];
  const float p0 = __fmul_rn(l0, s), p1 = __fmul_rn(l1, s);
  const float e0 = __fmaf_rn(l0, s, -p0), e1 = __fmaf_rn(l1, s, -p1);
  return bf16_of_exact(p0, e0) | (bf16_of_exact(p1, e1) << 16);
}

constexpr int kEmbedThreads = 256;

// One thread decodes chunk c (8 values) of RPT consecutive rows; the rows' loads
// are all issued before any is used, so a wave has RPT code words in flight
// instead of one.  Block b covers chunk block b % bpr of row group b / bpr.
template <int RPT>
__global__ void __launch_bounds__(kEmbedThreads)
    embed_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales, int N,
                 int K, const int64_t *__restrict__ ids, int64_t T, uint16_t *__restrict__ out,
                 int32_t *status, int blocks_per_row) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = level_f32(threadIdx.x);
  __syncthreads();
  const int g = blockIdx.x / blocks_per_row;
  const int c = (blockIdx.x - g * blocks_per_row) * kEmbedThreads + threadIdx.x;  // 8-value chunk
  if (c >= (K >> 3)) return;
  const int64_t t0 = (int64_t)g * RPT;
  uint32_t w[RPT];
  float s[RPT];
  bool ok[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int64_t id = t0 + j < T ? ids[t0 + j] : 0;
    ok[j] = id >= 0 && id < N;
    if (!ok[j] && t0 + j < T && c == 0 && status) atomicOr(status, 1);
    const int64_t r = ok[j] ? id : 0;  // a bad id reads row 0 and writes zeros
    w[j] = *reinterpret_cast<const uint32_t *>(codes + r * (int64_t)(K >> 1) + (int64_t)c * 4);
    s[j] = f16_bits_to_f32(scales[r * (int64_t)(K >> 6) + (c >> 3)]);
  }
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    if (t0 + j >= T) break;
    uint4 o = make_uint4(0u, 0u, 0u, 0u);
    if (ok[j]) {
      o.x = embed_pair(lv, w[j] & 0xFFu, s[j]);
      o.y = embed_pair(lv, (w[j] >> 8) & 0xFFu, s[j]);
      o.z = embed_pair(lv, (w[j] >> 16) & 0xFFu, s[j]);
      o.w = embed_pair(lv, w[j] >> 24, s[j]);
    }
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u32x4{o.x, o.y, o.z, o.w},
                                reinterpret_cast<u32x4 *>(out + (t0 + j) * K + (int64_t)c * 8));
  }
}

__global__ void clear_embed_status_kernel(int32_t *status) { *status = 0; }

hipError_t launch_embed(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                        const int64_t *ids, int64_t T, uint16_t *out, int32_t *status,
                        hipStream_t stream) {
  if (status) {
    hipLaunchKernelGGL(clear_embed_status_kernel, dim3(1), dim3(1), 0, stream, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (T == 0) return hipSuccess;
  const int chunks = (int)(K >> 3);
  const int bpr = (chunks + kEmbedThreads - 1) / kEmbedThreads;
  // rows per thread: keep about two waves' worth of blocks per SIMD before
  // trading blocks for loads in flight
  const int64_t blocks1 = T * bpr;
  const int rpt = blocks1 >= 8 * 2048 ? 8 : blocks1 >= 4 * 2048 ? 4 : blocks1 >= 2 * 2048 ? 2 : 1;
  const unsigned grid = (unsigned)(((T + rpt - 1) / rpt) * bpr);
  if (rpt == 8)
    hipLaunchKernelGGL(embed_kernel<8>, dim3(grid), dim3(kEmbedThreads), 0, stream, codes,
                       scales, (int)N, (int)K, ids, T, out, status, bpr);
  else if (rpt == 4)
    hipLaunchKernelGGL(embed_kernel<4>, dim3(grid), dim3(kEmbedThreads), 0, stream, codes,
                       scales, (int)N, (int)K, ids, T, out, status, bpr);
  else if (rpt == 2)
    hipLaunchKernelGGL(embed_kernel<2>, dim3(grid), dim3(kEmbedThreads), 0, stream, codes,
                       scales, (int)N, (int)K, ids, T, out, status, bpr);
  else
    hipLaunchKernelGGL(embed_kernel<1>, dim3(grid), dim3(kEmbedThreads), 0, stream, codes,
                       scales, (int)N, (int)K, ids, T, out, status, bpr);
  return hipGetLastError();
}

// A dispatch covers at most 2^32 - 1 work-items per dimension, so at most
// floor((2^32 - 1) / 256) blocks; T rows take ceil(T / rpt) * bpr blocks, with
// rpt = 8 rows per thread at every T near the limit.
int64_t embed_max_rows(int64_t K) {
  const int64_t bpr = ((K >> 3) + kEmbedThreads - 1) / kEmbedThreads;
  const int64_t max_blocks = ((int64_t(1) << 32) - 1) / kEmbedThreads;
  return 8 * (max_blocks / bpr);
}

}  // namespace nf4
