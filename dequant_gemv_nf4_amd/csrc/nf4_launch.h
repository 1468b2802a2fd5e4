// nf4_launch.h -- host-side launchers behind the C ABI (internal to libnf4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4 {

hipError_t launch_pack(const float *W, int64_t N, int64_t K, uint8_t *codes, uint16_t *scales,
                       int32_t *status, hipStream_t stream);
hipError_t launch_unpack(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                         float *out, hipStream_t stream);

// VALU product, 1 <= M <= 7 (the GEMV is M = 1), for the shapes its plan fits.
hipError_t launch_gemv_valu(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                            const uint16_t *X, int M, float *Y, hipStream_t stream);
bool valu_supported(int64_t N, int64_t K, int M);

// Whether the MFMA product of this shape runs in the streaming form (several
// column tiles per workgroup, activation fragments kept in registers).
bool gemm_mfma_streams(int64_t N, int64_t K, int M);

// Which kernel a batch of M rows runs on: the vector-ALU kernel (one weight
// decode shared by M dot products) for M <= 2, and for M = 3 and 4 on matrices
// of more than 5120 rows, except M = 4 above 16384 rows where the streaming
// MFMA form takes it; the MFMA kernel otherwise.  Measured on the Llama-3.1-8B
// shapes (graph replays): MFMA wins from M = 5 everywhere and at M = 3 and 4 on
// 4096 rows (4096x4096 at M = 4: 5.5 vs 7.1 us); VALU at M = 3 and 4 on 6144
// rows (M = 4: 8.6 vs 8.9 us) and at M = 3 on 28672 rows (18.4 vs 18.9); the
// streaming MFMA form at M = 4 on 28672 rows (18.2 vs 21.3).
inline bool use_valu(int64_t N, int64_t K, int M) {
  if (M == 4 && N > 16384 && gemm_mfma_streams(N, K, M)) return false;
  return (M <= 2 || (M <= 4 && N > 5120)) && valu_supported(N, K, M);
}

// Workspace layout of every K-splitting call (small-batch and prefill): the
// first kSplitCounterBytes hold one 32-bit counter per tile group (at most
// kSplitCounters groups split), the partial tiles start right after.  The
// counter area has the same place and size for every shape, and each call
// leaves its counters zero, so one workspace serves calls of any shape in turn.
constexpr int kSplitCounters = 1024;
constexpr int kSplitCounterBytes = kSplitCounters * 4;

// MFMA product, 1 <= M <= 32.  With a workspace (workspace_bytes at least
// gemm_mfma_workspace_bytes, its counter area zero before first use), K may be
// split over workgroups; without one (nullptr), never.
hipError_t launch_gemm_mfma(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                            const uint16_t *X, int M, float *Y, void *workspace,
                            int64_t workspace_bytes, hipStream_t stream);
int64_t gemm_mfma_workspace_bytes(int64_t N, int64_t K, int M);

// MFMA product with 64 x 64 .. 128 x 128 workgroup tiles, any M >= 1 (prefill);
// with a workspace (as for launch_gemm_mfma), small grids split K over workgroups.
hipError_t launch_gemm_prefill(const uint8_t *codes, const uint16_t *scales, int64_t N,
                               int64_t K, const uint16_t *X, int64_t M, float *Y, void *workspace,
                               int64_t workspace_bytes, hipStream_t stream);
int64_t gemm_prefill_workspace_bytes(int64_t N, int64_t K, int64_t M);

// Packed embedding rows into bf16; status (may be null) is cleared first.
hipError_t launch_embed(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                        const int64_t *ids, int64_t T, uint16_t *out, int32_t *status,
                        hipStream_t stream);
// largest T one launch of the embedding kernel covers for this K
int64_t embed_max_rows(int64_t K);

}  // namespace nf4
