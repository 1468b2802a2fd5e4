// stream_probe.hip -- the streaming floor a product launch is measured against.
//
// A product of an N x K packed matrix must read its codes (N K / 2 bytes) and
// scales (N K / 32 bytes) once and write its M N fp32 outputs (Trapetum
// overview, "The bandwidth law": decode time follows the bytes read).  This
// kernel moves exactly those bytes with nothing else to do: every 16-byte chunk
// of the two input ranges is read once with a non-temporal load and folded into
// a per-thread XOR, and out_words 32-bit words are written.  Its time, at the
// same byte counts and in the same kind of launch (back to back in a HIP
// graph), is what a product launch cannot beat; the product's time over it is
// what its own work costs on top of the stream.
//
// Variants (`variant`), all plain: 0..3 -- one 16-byte load per thread per
// step, 1, 2, 4 or 8 loads in flight per thread, one pass (grid = chunks /
// (256 x loads)); 4 -- a grid of 4 workgroups of 256 threads per compute unit
// striding over the chunks, 4 loads in flight.  The caller times each and takes
// the fastest.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "stream_probe.h"

namespace {

constexpr int kThreads = 256;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold(u32x4_t v) { return v.x ^ v.y ^ v.z ^ v.w; }

// chunk c of the concatenation [a chunks | b chunks]
__device__ __forceinline__ const u32x4_t *chunk_ptr(const uint8_t *a, int64_t ac, const uint8_t *b,
                                                    int64_t c) {
  return reinterpret_cast<const u32x4_t *>(c < ac ? a + 16 * c : b + 16 * (c - ac));
}

template <int V>
__global__ void __launch_bounds__(kThreads)
    probe_pass(const uint8_t *__restrict__ a, int64_t ac, const uint8_t *__restrict__ b,
               int64_t bc, const uint8_t *__restrict__ btail, int btail_bytes,
               uint32_t *__restrict__ out, int64_t out_words) {
  const int64_t total = ac + bc;
  const int64_t base = (int64_t)blockIdx.x * kThreads * V + threadIdx.x;
  u32x4_t v[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int64_t c = base + (int64_t)j * kThreads;
    v[j] = c < total ? __builtin_nontemporal_load(chunk_ptr(a, ac, b, c)) : u32x4_t{0, 0, 0, 0};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < V; ++j) acc ^= fold(v[j]);
  if (blockIdx.x == 0 && (int)threadIdx.x < btail_bytes) acc ^= btail[threadIdx.x];
  const int64_t gtid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t nthreads = (int64_t)gridDim.x * kThreads;
  for (int64_t i = gtid; i < out_words; i += nthreads) out[i] = acc ^ (uint32_t)i;
}

__global__ void __launch_bounds__(kThreads)
    probe_persistent(const uint8_t *__restrict__ a, int64_t ac, const uint8_t *__restrict__ b,
                     int64_t bc, const uint8_t *__restrict__ btail, int btail_bytes,
                     uint32_t *__restrict__ out, int64_t out_words) {
  constexpr int V = 4;
  const int64_t total = ac + bc;
  const int64_t nthreads = (int64_t)gridDim.x * kThreads;
  const int64_t gtid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (int64_t c0 = gtid; c0 < total; c0 += nthreads * V) {
    u32x4_t v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t c = c0 + (int64_t)j * nthreads;
      v[j] = c < total ? __builtin_nontemporal_load(chunk_ptr(a, ac, b, c)) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < V; ++j) acc ^= fold(v[j]);
  }
  if (blockIdx.x == 0 && (int)threadIdx.x < btail_bytes) acc ^= btail[threadIdx.x];
  for (int64_t i = gtid; i < out_words; i += nthreads) out[i] = acc ^ (uint32_t)i;
}

}  // namespace

extern "C" int nf4_probe_variants(void) { return 5; }

extern "C" int nf4_probe_stream(const void *a, int64_t a_bytes, const void *b, int64_t b_bytes,
                                uint32_t *out, int64_t out_words, int variant, void *stream) {
  if ((a_bytes > 0 && !a) || (b_bytes > 0 && !b) || (out_words > 0 && !out)) return -1;
  if (a_bytes < 0 || b_bytes < 0 || out_words < 0 || a_bytes % 16 != 0) return -1;
  if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15) return -2;
  if (variant < 0 || variant >= nf4_probe_variants()) return -3;
  const int64_t ac = a_bytes / 16, bc = b_bytes / 16;
  const uint8_t *btail = static_cast<const uint8_t *>(b) + 16 * bc;
  const int btail_bytes = (int)(b_bytes - 16 * bc);
  const uint8_t *pa = static_cast<const uint8_t *>(a), *pb = static_cast<const uint8_t *>(b);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t total = ac + bc;
  if (variant < 4) {
    const int V = 1 << variant;
    const int64_t blocks = std::max<int64_t>(1, (total + kThreads * V - 1) / (kThreads * V));
    if (blocks > 0x7fffffff) return -3;
    switch (V) {
      case 1: hipLaunchKernelGGL(probe_pass<1>, dim3(blocks), dim3(kThreads), 0, s, pa, ac, pb, bc,
                                 btail, btail_bytes, out, out_words); break;
      case 2: hipLaunchKernelGGL(probe_pass<2>, dim3(blocks), dim3(kThreads), 0, s, pa, ac, pb, bc,
                                 btail, btail_bytes, out, out_words); break;
      case 4: hipLaunchKernelGGL(probe_pass<4>, dim3(blocks), dim3(kThreads), 0, s, pa, ac, pb, bc,
                                 btail, btail_bytes, out, out_words); break;
      default: hipLaunchKernelGGL(probe_pass<8>, dim3(blocks), dim3(kThreads), 0, s, pa, ac, pb,
                                  bc, btail, btail_bytes, out, out_words); break;
    }
  } else {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    hipLaunchKernelGGL(probe_persistent, dim3(4 * cus), dim3(kThreads), 0, s, pa, ac, pb, bc,
                       btail, btail_bytes, out, out_words);
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
