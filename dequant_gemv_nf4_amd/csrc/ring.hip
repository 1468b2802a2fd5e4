// ring.hip -- CopyRing: products over packed matrices that live in pinned host
// memory, staged through a pair of device buffers that are used in turn
// (deep-fold README, "Method", execution-path table and Figure 1: when a model
// does not fit on the card, some of its packed matrices stay in page-locked host
// memory and are copied into one of two device slots before the unchanged
// product kernel runs on them).
//
// Each nf4_ring_gemm call takes the next slot (0, 1, 0, ...), and enqueues
//   copy stream:    wait until the slot's previous product has finished reading
//                   it; copy codes then scales host -> slot; mark "copied";
//   compute stream: wait for "copied"; run the product from the slot (the same
//                   kernels as nf4_gemm_smallm); mark "done reading".
// So the copy of matrix i + 1 overlaps the product of matrix i, and a slot is
// never overwritten while a product reads it.  Everything is enqueued; nothing
// waits on the host.  The ring owns four HIP events (created and destroyed with
// it) and no device memory: the slots are the caller's.
#include <new>

#include "../../include/nf4.h"
#include "nf4_launch.h"

namespace nf4 {
int device_status();  // NF4_OK on a gfx950 device (api.hip)
}

struct nf4_ring {
  uint8_t *slot[2];
  int64_t slot_bytes;
  hipStream_t compute, copy;
  hipEvent_t copied[2], read_done[2];
  bool used[2];
  int next;
  int device;
};

namespace {

constexpr int64_t kScaleAlign = 256;  // scales start on a 256-byte boundary of the slot

int64_t scale_offset(int64_t N, int64_t K) {
  return (N * (K / 2) + kScaleAlign - 1) / kScaleAlign * kScaleAlign;
}

bool is_pinned_host(const void *p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the error a pageable pointer leaves
    return false;
  }
  return a.type == hipMemoryTypeHost;
}

}  // namespace

extern "C" {

int nf4_ring_create(nf4_ring **ring, void *slot0, void *slot1, int64_t slot_bytes,
                    void *compute_stream, void *copy_stream) {
  if (!ring || !slot0 || !slot1 || slot_bytes <= 0) return NF4_EINVAL;
  *ring = nullptr;
  if ((reinterpret_cast<uintptr_t>(slot0) & 255) || (reinterpret_cast<uintptr_t>(slot1) & 255))
    return NF4_EALIGN;
  if (int st = nf4::device_status()) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NF4_ERANGE;
  nf4_ring *r = new (std::nothrow) nf4_ring();
  if (!r) return NF4_ERANGE;
  r->slot[0] = static_cast<uint8_t *>(slot0);
  r->slot[1] = static_cast<uint8_t *>(slot1);
  r->slot_bytes = slot_bytes;
  r->compute = (hipStream_t)compute_stream;
  r->copy = (hipStream_t)copy_stream;
  r->used[0] = r->used[1] = false;
  r->next = 0;
  r->device = dev;
  int made = 0;
  bool ok = true;
  for (int s = 0; s < 2 && ok; ++s) {
    ok = hipEventCreateWithFlags(&r->copied[s], hipEventDisableTiming) == hipSuccess;
    made += ok;
    if (ok) {
      ok = hipEventCreateWithFlags(&r->read_done[s], hipEventDisableTiming) == hipSuccess;
      made += ok;
    }
  }
  if (!ok) {
    hipEvent_t *ev[4] = {&r->copied[0], &r->read_done[0], &r->copied[1], &r->read_done[1]};
    for (int i = 0; i < made; ++i) (void)hipEventDestroy(*ev[i]);
    delete r;
    return NF4_ELAUNCH;
  }
  *ring = r;
  return NF4_OK;
}

int nf4_ring_gemm(nf4_ring *r, const uint8_t *host_codes, const uint16_t *host_scales, int64_t N,
                  int64_t K, const uint16_t *X, int64_t M, float *Y) {
  if (!r || !host_codes || !host_scales || !X || !Y) return NF4_EINVAL;
  if (N <= 0 || K <= 0 || K % NF4_GROUP != 0) return NF4_EINVAL;
  if (K > NF4_MAX_K || N >= (int64_t(1) << 31) || N * (K / 2) >= (int64_t(1) << 31))
    return NF4_ERANGE;
  if (M < 1 || M > NF4_MAX_M) return NF4_ERANGE;
  const int64_t soff = scale_offset(N, K);
  const int64_t sbytes = N * (K / NF4_GROUP) * 2;
  if (soff + sbytes > r->slot_bytes) return NF4_ERANGE;
  if ((reinterpret_cast<uintptr_t>(X) & 15) || (reinterpret_cast<uintptr_t>(Y) & 3)) return NF4_EALIGN;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != r->device) return NF4_EDEVICE;
  if (!is_pinned_host(host_codes) || !is_pinned_host(host_scales)) return NF4_EINVAL;

  const int s = r->next;
  uint8_t *codes = r->slot[s];
  uint16_t *scales = reinterpret_cast<uint16_t *>(r->slot[s] + soff);
  auto fail = [](hipError_t e) { return e == hipSuccess ? NF4_OK : NF4_ELAUNCH; };
  if (r->used[s] && hipStreamWaitEvent(r->copy, r->read_done[s], 0) != hipSuccess)
    return NF4_ELAUNCH;
  if (int e = fail(hipMemcpyAsync(codes, host_codes, N * (K / 2), hipMemcpyHostToDevice, r->copy)))
    return e;
  if (int e = fail(hipMemcpyAsync(scales, host_scales, sbytes, hipMemcpyHostToDevice, r->copy)))
    return e;
  if (int e = fail(hipEventRecord(r->copied[s], r->copy))) return e;
  if (int e = fail(hipStreamWaitEvent(r->compute, r->copied[s], 0))) return e;
  const int m = (int)M;
  hipError_t le = nf4::use_valu(N, K, m)
                      ? nf4::launch_gemv_valu(codes, scales, N, K, X, m, Y, r->compute)
                      : nf4::launch_gemm_mfma(codes, scales, N, K, X, m, Y, nullptr, 0, r->compute);
  if (int e = fail(le)) return e;
  if (int e = fail(hipEventRecord(r->read_done[s], r->compute))) return e;
  r->used[s] = true;
  r->next = s ^ 1;
  return NF4_OK;
}

int64_t nf4_ring_slot_bytes(int64_t N, int64_t K) {
  // the shape limits of every product call, checked before any arithmetic
  if (N <= 0 || K <= 0 || K % NF4_GROUP != 0) return -1;
  if (K > NF4_MAX_K || N >= (int64_t(1) << 31) || N * (K / 2) >= (int64_t(1) << 31)) return -1;
  return scale_offset(N, K) + N * (K / NF4_GROUP) * 2;
}

int nf4_ring_destroy(nf4_ring *r) {
  if (!r) return NF4_EINVAL;
  int st = NF4_OK;
  for (int s = 0; s < 2; ++s) {
    if (hipEventSynchronize(r->read_done[s]) != hipSuccess) st = NF4_ELAUNCH;
    if (hipEventDestroy(r->copied[s]) != hipSuccess) st = NF4_ELAUNCH;
    if (hipEventDestroy(r->read_done[s]) != hipSuccess) st = NF4_ELAUNCH;
  }
  delete r;
  return st;
}

}  // extern "C"
