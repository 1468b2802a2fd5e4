// api.hip -- the C ABI of libnf4 (declared in include/nf4.h): argument checks,
// device check and kernel choice.  No allocation, no synchronization.
#include <atomic>
#include <cstring>
#include <mutex>

#include "../../include/nf4.h"
#include "nf4_device.h"
#include "nf4_launch.h"

namespace nf4 {
}

namespace {

constexpr int kMaxDevices = 64;
// per device: 0 = unknown, 1 = gfx950, 2 = other
std::atomic<int> g_arch[kMaxDevices];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NF4_ERANGE;
  int a = g_arch[dev].load(std::memory_order_relaxed);
  if (a == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return NF4_ERANGE;
    a = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch[dev].store(a, std::memory_order_relaxed);
  }
  return a == 1 ? NF4_OK : NF4_EDEVICE;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_shape(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || K % NF4_GROUP != 0) return NF4_EINVAL;
  if (K > NF4_MAX_K || N >= (int64_t(1) << 31)) return NF4_ERANGE;
  if (N * (K / 2) >= (int64_t(1) << 31)) return NF4_ERANGE;  // codes of one matrix < 2 GiB
  return NF4_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? NF4_OK : NF4_ELAUNCH; }

// ---- the library-owned scratch of nf4_gemm_smallm_noalloc: one array per
// device (each GPU the library runs on holds its own copy until the process
// ends), in place of a caller workspace.  The host never passes `scratch`
// itself to a kernel (in host code it is only a stand-in for the symbol): the
// device address is looked up once per device with hipGetSymbolAddress and kept.
constexpr int64_t kScratchBytes = int64_t(4) << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` per device, set once

__global__ void clear_counters_kernel(uint32_t *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The device's scratch address, set up on the device's first call: the lookup,
// then the counter area cleared by a kernel on the caller's stream (every
// completed split call leaves the counters zero again).
int scratch_for_current_device(void **out, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NF4_ERANGE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return NF4_ELAUNCH;
    constexpr int n = nf4::kSplitCounters;
    hipLaunchKernelGGL(clear_counters_kernel, dim3((n + 255) / 256), dim3(256), 0, stream,
                       static_cast<uint32_t *>(p), n);
    if (hipGetLastError() != hipSuccess) return NF4_ELAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return NF4_OK;
}

}  // namespace

namespace nf4 {
int device_status() { return check_device(); }
}  // namespace nf4

extern "C" {

int nf4_pack(const float *W, int64_t N, int64_t K, uint8_t *codes, uint16_t *scales,
             int32_t *dev_status, void *stream) {
  if (!W || !codes || !scales) return NF4_EINVAL;
  if (int r = check_shape(N, K)) return r;
  if (!aligned(W, 4) || !aligned(codes, 4) || !aligned(scales, 2) ||
      (dev_status && !aligned(dev_status, 4)))
    return NF4_EALIGN;
  if (int r = check_device()) return r;
  return launched(nf4::launch_pack(W, N, K, codes, scales, dev_status, (hipStream_t)stream));
}

int nf4_unpack(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K, float *W_out,
               void *stream) {
  if (!codes || !scales || !W_out) return NF4_EINVAL;
  if (int r = check_shape(N, K)) return r;
  if (!aligned(codes, 4) || !aligned(scales, 2) || !aligned(W_out, 16)) return NF4_EALIGN;
  if (int r = check_device()) return r;
  return launched(nf4::launch_unpack(codes, scales, N, K, W_out, (hipStream_t)stream));
}

int64_t nf4_gemm_smallm_workspace_bytes(int64_t N, int64_t K, int64_t M) {
  if (check_shape(N, K) || M < 1 || M > NF4_MAX_M) return -1;
  if (nf4::use_valu(N, K, (int)M)) return 0;
  return nf4::gemm_mfma_workspace_bytes(N, K, (int)M);
}

int nf4_gemm_smallm_ws(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                       const uint16_t *X, int64_t M, float *Y, void *workspace,
                       int64_t workspace_bytes, void *stream) {
  if (!codes || !scales || !X || !Y) return NF4_EINVAL;
  if (int r = check_shape(N, K)) return r;
  if (M < 1 || M > NF4_MAX_M) return NF4_ERANGE;
  if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(X, 16) || !aligned(Y, 4) ||
      (workspace && !aligned(workspace, 256)))
    return NF4_EALIGN;
  const int64_t need = nf4_gemm_smallm_workspace_bytes(N, K, M);
  if (need > 0 && (!workspace || workspace_bytes < need)) return NF4_ERANGE;
  if (int r = check_device()) return r;
  const int m = (int)M;
  hipStream_t s = (hipStream_t)stream;
  if (nf4::use_valu(N, K, m))
    return launched(nf4::launch_gemv_valu(codes, scales, N, K, X, m, Y, s));
  return launched(nf4::launch_gemm_mfma(codes, scales, N, K, X, m, Y,
                                        need > 0 ? workspace : nullptr, workspace_bytes, s));
}

int nf4_gemm_smallm(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                    const uint16_t *X, int64_t M, float *Y, void *stream) {
  if (!codes || !scales || !X || !Y) return NF4_EINVAL;
  if (int r = check_shape(N, K)) return r;
  if (M < 1 || M > NF4_MAX_M) return NF4_ERANGE;
  if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(X, 16) || !aligned(Y, 4))
    return NF4_EALIGN;
  if (int r = check_device()) return r;
  const int m = (int)M;
  hipStream_t s = (hipStream_t)stream;
  if (nf4::use_valu(N, K, m))
    return launched(nf4::launch_gemv_valu(codes, scales, N, K, X, m, Y, s));
  return launched(nf4::launch_gemm_mfma(codes, scales, N, K, X, m, Y, nullptr, 0, s));
}

int64_t nf4_gemm_smallm_noalloc_max_bytes(void) { return kScratchBytes; }

int nf4_gemm_smallm_noalloc(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                            const uint16_t *X, int64_t M, float *Y, void *stream) {
  if (!codes || !scales || !X || !Y) return NF4_EINVAL;
  if (int r = check_shape(N, K)) return r;
  if (M < 1 || M > NF4_MAX_M) return NF4_ERANGE;
  if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(X, 16) || !aligned(Y, 4))
    return NF4_EALIGN;
  const int64_t need = nf4_gemm_smallm_workspace_bytes(N, K, M);
  if (need > kScratchBytes) return NF4_ERANGE;
  if (int r = check_device()) return r;
  const int m = (int)M;
  hipStream_t s = (hipStream_t)stream;
  if (nf4::use_valu(N, K, m))
    return launched(nf4::launch_gemv_valu(codes, scales, N, K, X, m, Y, s));
  void *ws = nullptr;
  if (need > 0) {
    if (int r = scratch_for_current_device(&ws, s)) return r;
  }
  return launched(nf4::launch_gemm_mfma(codes, scales, N, K, X, m, Y, ws,
                                        need > 0 ? kScratchBytes : 0, s));
}

int64_t nf4_gemm_prefill_workspace_bytes(int64_t N, int64_t K, int64_t M) {
  if (check_shape(N, K) || M < 1 || M * K >= (int64_t(1) << 30)) return -1;
  return nf4::gemm_prefill_workspace_bytes(N, K, M);
}

int nf4_gemm_prefill_ws(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                        const uint16_t *X, int64_t M, float *Y, void *workspace,
                        int64_t workspace_bytes, void *stream) {
  if (!codes || !scales || !X || !Y) return NF4_EINVAL;
  if (int r = check_shape(N, K)) return r;
  if (M < 1 || M * K >= (int64_t(1) << 30)) return NF4_ERANGE;  // X below 2 GiB
  if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(X, 16) || !aligned(Y, 4) ||
      (workspace && !aligned(workspace, 256)))
    return NF4_EALIGN;
  const int64_t need = nf4::gemm_prefill_workspace_bytes(N, K, M);
  if (need > 0 && (!workspace || workspace_bytes < need)) return NF4_ERANGE;
  if (int r = check_device()) return r;
  return launched(nf4::launch_gemm_prefill(codes, scales, N, K, X, M, Y,
                                           need > 0 ? workspace : nullptr, workspace_bytes,
                                           (hipStream_t)stream));
}

int nf4_gemm_prefill(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                     const uint16_t *X, int64_t M, float *Y, void *stream) {
  if (!codes || !scales || !X || !Y) return NF4_EINVAL;
  if (int r = check_shape(N, K)) return r;
  if (M < 1 || M * K >= (int64_t(1) << 30)) return NF4_ERANGE;  // X below 2 GiB
  if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(X, 16) || !aligned(Y, 4))
    return NF4_EALIGN;
  if (int r = check_device()) return r;
  return launched(
      nf4::launch_gemm_prefill(codes, scales, N, K, X, M, Y, nullptr, 0, (hipStream_t)stream));
}

int nf4_gemv(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
             const uint16_t *x, float *y, void *stream) {
  return nf4_gemm_smallm(codes, scales, N, K, x, 1, y, stream);
}

int nf4_embed(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
              const int64_t *ids, int64_t T, uint16_t *out, int32_t *dev_status, void *stream) {
  if (!codes || !scales || T < 0 || (T > 0 && (!ids || !out))) return NF4_EINVAL;
  if (int r = check_shape(N, K)) return r;
  if (T > nf4::embed_max_rows(K)) return NF4_ERANGE;
  if (!aligned(codes, 4) || !aligned(scales, 2) || (T > 0 && (!aligned(ids, 8) ||
      !aligned(out, 16))) || (dev_status && !aligned(dev_status, 4)))
    return NF4_EALIGN;
  if (int r = check_device()) return r;
  return launched(nf4::launch_embed(codes, scales, N, K, ids, T, out, dev_status,
                                    (hipStream_t)stream));
}

void nf4_codebook(float out[16]) {
  if (!out) return;
  for (int i = 0; i < 16; ++i) std::memcpy(&out[i], &nf4::kLevelBits[i], 4);
}

const char *nf4_strerror(int status) {
  switch (status) {
    case NF4_OK: return "ok";
    case NF4_EINVAL: return "invalid argument (null pointer, N or K not positive, K % 64 != 0)";
    case NF4_EALIGN: return "misaligned pointer";
    case NF4_ERANGE: return "size out of range (M not in [1,32], K too large, N too large) or no device";
    case NF4_EDEVICE: return "current device is not gfx950";
    case NF4_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
