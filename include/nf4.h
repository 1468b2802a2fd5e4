/*
 * nf4.h -- C ABI of libnf4: NF4 weight packing and the fused dequant
 * matrix-vector / small-batch products for MI355X (gfx950).
 *
 * Problem statement (the sources):
 *  - deep-fold README, "Method": weights are 4-bit NF4 codes in groups of 64
 *    consecutive weights, one FP16 scale per group; packed codes and scales stay
 *    in GPU memory and the linear kernels rebuild the values of the current tile
 *    while multiplying, never writing a dense matrix back.  Decode is an N=1
 *    GEMV; prefill runs the same product on chunks of at most 32 positions.
 *  - Trapetum home page: the 4-bit weights are decoded inside the matmul, so the
 *    full-precision matrix is never materialized.
 *  - NF4 levels: QLoRA's 4-bit NormalFloat (named by the deep-fold README).
 *  So every product computes  Y[m][n] = sum_k L[code(n,k)] * s(n, k/64) * X[m][k].
 *
 * Data layout (all row-major, contiguous, no padding or leading dimensions):
 *  - W      fp32 [N][K]              input to nf4_pack only.
 *  - codes  uint8 [N][K/2]           byte j of row n = code(n,2j) | code(n,2j+1) << 4
 *                                    (low nibble = even k).
 *  - scales uint16 [N][K/64]         IEEE binary16 bit patterns.
 *  - x / X  uint16 bf16 bits [M][K]  (x is M = 1).
 *  - y / Y  fp32 [M][N].
 *  K must be a multiple of 64; every group lies inside one row.
 *
 * Ownership and execution:
 *  - Every array argument is a device pointer owned by the caller.  The library
 *    never frees or keeps a pointer and never writes its inputs.  The only
 *    state it keeps between calls is a per-device cache of "is this device
 *    gfx950" (filled on a device's first call, read-only afterwards), so calls
 *    on different streams may run concurrently.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    call only enqueues work on it and returns; there is no synchronization.
 *  - Outputs are fully overwritten (no accumulation into y / Y).
 *
 * Errors: each call validates its arguments on the host before launching and
 * returns one of the nf4_status codes; on any error nothing is enqueued and no
 * memory is touched.  Asynchronous GPU faults surface on the stream as usual.
 *
 * Numerics: nf4_pack and nf4_unpack are exact (bit-for-bit defined below).
 * The products accumulate in fp32.  On the vector-ALU kernel (M <= 2, and
 * M = 3 or 4 on matrices of more than 5120 rows) the levels are f16 and each
 * 32-value activation block is scaled by a power of two into f16 where that is
 * exact (every non-zero value of the block within 2^28 of its largest in
 * binary exponent, and the largest at least 2^-98); the blocks that are not
 * are computed as f16 level x fp32 scale (exact) times the bf16 activation in
 * fp32 instead.  The MFMA product that walks 5 or more 16-column tiles per
 * workgroup (M <= 32 on matrices of 16385 to 32768 rows, K a multiple of 256 up
 * to 8192, up to 4096 above M = 8) takes f16 levels and f16 activations
 * scaled by a power of two per 64-value group shared by all rows, under the
 * same exactness rule over the group's values of every row; a group that fails
 * is computed the same exact way.  The other MFMA kernels (every other M, and
 * nf4_gemm_prefill) split the levels into bf16 hi + lo and use the bf16
 * activations as they are.  Per output element
 *   |Y - Y_exact| <= 2e-3 * sum_k |w~(n,k) X[m][k]| + 1e-5
 * for finite inputs with every |X[m][k]| <= 2^120 and every
 * sum_k |w~(n,k) X[m][k]| <= 2^120 (w~ = the dequantized weight).  Results are
 * deterministic: the same call on the same device gives the same bits.
 */
#ifndef NF4_H
#define NF4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NF4_GROUP 64      /* weights per scale group, along K */
#define NF4_MAX_M 32      /* largest activation batch of nf4_gemm_smallm */
#define NF4_MAX_K 32768   /* largest supported K */

enum nf4_status {
  NF4_OK = 0,
  NF4_EINVAL = -1,  /* null pointer, N <= 0, K <= 0, K % 64 != 0 */
  NF4_EALIGN = -2,  /* codes / x / X not 16-byte aligned, scales / y not 2 / 4 */
  NF4_ERANGE = -3,  /* M outside [1, 32], K > NF4_MAX_K, N * K / 2 >= 2^31, or no device */
  NF4_EDEVICE = -4, /* current device is not gfx950 */
  NF4_ELAUNCH = -5  /* the HIP launch itself failed */
};

/* bits OR-ed into *dev_status by nf4_pack */
#define NF4_PACK_NONFINITE 1      /* a group holds NaN or +-inf */
#define NF4_PACK_SCALE_OVERFLOW 2 /* group absmax rounds to fp16 infinity (>= 65520) */

/*
 * nf4_pack -- quantize fp32 W [N][K] to NF4 codes and fp16 group scales.
 * Source: deep-fold README, "Method" (group of 64, NF4 codes, one FP16 scale).
 * Per group of 64 along K:
 *   s = binary16(max |w|), round to nearest even;
 *   code(w) = number of i in 0..14 with w > (L[i] + L[i+1]) / 2 * s, evaluated
 *             exactly (fp64) -- the nearest level L[c]*s to w, ties to the lower
 *             code; if s == 0 every code is 7 (the zero level).
 * A group holding a non-finite value, or whose absmax rounds to fp16 infinity,
 * is written as scale 0 and codes 7, and the matching NF4_PACK_* bit is OR-ed
 * into *dev_status (device int32).  dev_status may be NULL; if given, the call
 * first clears it to 0 on the stream.
 * Alignment: W 4 bytes, codes 4 bytes, scales 2 bytes.
 */
int nf4_pack(const float *W, int64_t N, int64_t K, uint8_t *codes, uint16_t *scales,
             int32_t *dev_status, void *stream);

/*
 * nf4_unpack -- dequantize to fp32 W_out [N][K]:  W_out = fp32(L[c] * s), one
 * correctly rounded fp32 multiply.  Exists to check the format bit for bit; the
 * products never call it.  Source: deep-fold README, "Method".
 * Alignment: codes 4 bytes, scales 2 bytes, W_out 16 bytes.
 */
int nf4_unpack(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
               float *W_out, void *stream);

/*
 * nf4_gemv -- y[n] = sum_k L[code(n,k)] * s(n,k/64) * x[k]  (M = 1, decode).
 * Source: deep-fold README, "Method" (N=1 GEMV of resident decode); Trapetum
 * overview, "The bandwidth law" (the cost is reading the packed weights).
 * The dense matrix is never formed: codes are expanded in registers.
 * Alignment: codes 16 bytes, scales 2, x 16, y 4.
 */
int nf4_gemv(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
             const uint16_t *x, float *y, void *stream);

/*
 * nf4_gemm_smallm -- Y[m][n] = sum_k L[code(n,k)] * s(n,k/64) * X[m][k] for
 * 1 <= M <= 32 (prefill chunks, speculative verification batches).
 * Source: deep-fold README, "Method" (prompt chunks of up to 32 positions on a
 * tensor-core NF4 GEMM).  M = 1 is the GEMV; from M = 5 (M = 3 and 4 on
 * matrices of up to 5120 rows) the product runs on MFMA.
 * Alignment: codes 16 bytes, scales 2, X 16, Y 4.
 */
int nf4_gemm_smallm(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                    const uint16_t *X, int64_t M, float *Y, void *stream);

/*
 * nf4_gemm_smallm_ws -- nf4_gemm_smallm with a caller-owned device workspace
 * that lets the MFMA kernel split K over workgroups (wider column tiles share
 * each activation fragment while every CU still gets work).  Each split writes
 * its partial tile to the workspace; the last split of a tile group to finish
 * adds the partials in split order, so results are deterministic (they may
 * differ in the last bits from nf4_gemm_smallm, whose sums are grouped
 * differently; both meet the stated tolerance).
 *  - workspace: device memory, 256-byte aligned, at least
 *    nf4_gemm_smallm_workspace_bytes(N, K, M) bytes (0 bytes: the call is
 *    nf4_gemm_smallm and workspace may be NULL).  Its first 4 KiB are counters
 *    that must be zero before the workspace's first use; every completed call
 *    leaves them zero again, so one zero-fill at allocation suffices.  The
 *    counter area has the same place and size for every shape (partial tiles
 *    follow it), so one workspace serves calls of any shapes, of this function
 *    and of nf4_gemm_prefill_ws, one after another.  Calls that share a
 *    workspace must not run concurrently (e.g. use one per stream).
 *  - Errors: as nf4_gemm_smallm; NF4_ERANGE if the workspace is missing or too
 *    small; NF4_EALIGN if it is not 256-byte aligned.
 * Source: deep-fold README, "Method" (prompt chunks of up to 32 positions).
 * nf4_gemm_smallm_workspace_bytes: the bytes needed for (N, K, M), 0 if the
 * call would not split, -1 if the shape or M is invalid.  Host only.
 */
int64_t nf4_gemm_smallm_workspace_bytes(int64_t N, int64_t K, int64_t M);
int nf4_gemm_smallm_ws(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                       const uint16_t *X, int64_t M, float *Y, void *workspace,
                       int64_t workspace_bytes, void *stream);

/*
 * nf4_gemm_smallm_noalloc -- nf4_gemm_smallm_ws without a caller workspace and
 * without any allocation: the K-split partial tiles and counters live in a
 * library-owned device array of nf4_gemm_smallm_noalloc_max_bytes() bytes
 * (4 MiB; every valid small-batch shape needs at most about 2 MiB), one per
 * device, held until the process ends.  For callers that cannot allocate
 * device memory at the point of the call: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same kernels, plans and
 * bits as nf4_gemm_smallm_ws with a workspace.
 *  - The first call on a device looks up the array's address (hipGetSymbolAddress)
 *    and clears its counter area with a kernel on `stream`; make that first call
 *    outside graph capture.  No call allocates or frees memory.
 *  - Every call on one device shares that device's array and leaves its
 *    counters zero: calls that overlap on one GPU (concurrent streams, or host
 *    threads) race on it and must be serialized by the caller.
 *  - Errors: as nf4_gemm_smallm; NF4_ERANGE if the shape would need more than
 *    nf4_gemm_smallm_noalloc_max_bytes() of scratch.
 * nf4_gemm_smallm_noalloc_max_bytes: the array's size in bytes.  Host only.
 */
int64_t nf4_gemm_smallm_noalloc_max_bytes(void);
int nf4_gemm_smallm_noalloc(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                            const uint16_t *X, int64_t M, float *Y, void *stream);

/*
 * nf4_gemm_prefill -- the same product, Y[m][n] = sum_k L[code(n,k)] *
 * s(n,k/64) * X[m][k], for any batch 1 <= M with M * K < 2^30 (prefill chunks
 * beyond 32 positions), on 32 x 32 x 16 bf16 MFMA tiles of 64 x 64 to 128 x 128
 * outputs per workgroup.  Source: deep-fold README, "Method" (prefill on the
 * NF4 matrix-core product); Trapetum overview, "The fine print" (at prefill
 * sizes the product is bound by arithmetic, not by the weight stream).
 * Alignment: codes 16 bytes, scales 2, X 16, Y 4.  Errors: NF4_ERANGE for
 * M < 1 or M * K >= 2^30, otherwise as nf4_gemm_smallm.
 */
int nf4_gemm_prefill(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                     const uint16_t *X, int64_t M, float *Y, void *stream);

/*
 * nf4_gemm_prefill_ws -- nf4_gemm_prefill with a caller-owned device workspace
 * that lets a grid of fewer output tiles than CUs split K over workgroups (each
 * tile's S partial tiles are added in split order by the last to finish:
 * deterministic; bits may differ from nf4_gemm_prefill's, both within the
 * tolerance).  Workspace rules as for nf4_gemm_smallm_ws: 256-byte aligned, at
 * least nf4_gemm_prefill_workspace_bytes(N, K, M) bytes (0: no split, NULL
 * allowed), the same 4 KiB counter area (zero before first use, re-armed by
 * every completed call; shareable with nf4_gemm_smallm_ws calls of any shape),
 * no concurrent calls sharing one.  Errors: as nf4_gemm_prefill; NF4_ERANGE for
 * a missing or short workspace, NF4_EALIGN for a misaligned one.
 * Source: deep-fold README, "Method" (prefill on the NF4 matrix-core product).
 * nf4_gemm_prefill_workspace_bytes: bytes needed (0: no split), -1 if invalid.
 */
int64_t nf4_gemm_prefill_workspace_bytes(int64_t N, int64_t K, int64_t M);
int nf4_gemm_prefill_ws(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                        const uint16_t *X, int64_t M, float *Y, void *workspace,
                        int64_t workspace_bytes, void *stream);

/* bit OR-ed into *dev_status by nf4_embed */
#define NF4_EMBED_BAD_ID 1 /* an id outside [0, N): its output row is all +0 */

/*
 * nf4_embed -- packed embedding rows: decode only the rows ids[0..T-1] of the
 * NF4 matrix (codes, scales) [N][K] into bf16:
 *   out[t][k] = bf16(L[code(ids[t],k)] * s(ids[t],k/64)), the exact product
 *   rounded once to nearest, ties to even (NaN scales give 0x7FC0).
 * Source: deep-fold README, "Method" (embeddings decode only the requested
 * rows; the rows then feed the first linear layer as bf16 activations).
 *  - ids: device int64 [T]; repeated ids are allowed.  An id outside [0, N)
 *    writes a zero row and OR-s NF4_EMBED_BAD_ID into *dev_status (device
 *    int32, may be NULL; if given, the call first clears it to 0 on the stream).
 *  - out: device bf16 bits [T][K].  T = 0 is valid and writes nothing.
 * Alignment: codes 4 bytes, scales 2, ids 8, out 16.  Errors: NF4_EINVAL for a
 * null pointer or T < 0, NF4_ERANGE if T is too large for one launch
 * (T > 8 * floor(floor((2^32 - 1) / 256) / ceil(K / 2048)), e.g. 134217720 rows
 * for K <= 2048), plus the shape rules of every call; all checked before the
 * status word is cleared.
 */
int nf4_embed(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
              const int64_t *ids, int64_t T, uint16_t *out, int32_t *dev_status,
              void *stream);

/*
 * CopyRing -- products over packed matrices held in pinned host memory, staged
 * through two device slots used in turn.  Source: deep-fold README, "Method",
 * execution-path table and Figure 1 (for models larger than the card, some
 * packed matrices stay in page-locked host memory and are copied into one of two
 * device slots, where the same product kernel reads them).
 *
 * nf4_ring_create: slot0 / slot1 are caller-owned device buffers of slot_bytes
 * each (256-byte aligned); compute_stream and copy_stream are two hipStreams
 * (void*; NULL = null stream, but two distinct streams are needed for overlap).
 * The ring object and its four HIP events are created here and released by
 * nf4_ring_destroy, which first waits until the ring's last product is done.
 * The ring keeps the slot pointers and streams until then; a ring is used by
 * one host thread at a time.
 *
 * nf4_ring_gemm: Y[m][n] = sum_k L[code(n,k)] s(n,k/64) X[m][k] exactly as
 * nf4_gemm_smallm (same kernels, same bits), with codes [N][K/2] and scales
 * [N][K/64] in pinned host memory (allocated with hipHostMalloc or an equivalent;
 * a pageable pointer is rejected with NF4_EINVAL).  The call takes the next slot,
 * enqueues on the copy stream a wait for the slot's previous product, the copy
 * of codes (slot offset 0) and scales (offset rounded up to 256 bytes), and on the
 * compute stream a wait for that copy and the product; it returns at once.
 * X and Y are device memory, read / written on the compute stream.  The host
 * buffers must stay valid until the copy has run.  Errors: NF4_ERANGE if the
 * matrix does not fit a slot (see nf4_ring_slot_bytes) or M is outside [1, 32];
 * NF4_EDEVICE if the current device is not the ring's; the shape and alignment
 * rules of nf4_gemm_smallm otherwise.
 *
 * nf4_ring_slot_bytes: bytes a slot needs for an N x K matrix (-1 if the shape
 * is invalid or beyond the limits of the product calls).
 */
typedef struct nf4_ring nf4_ring;
int nf4_ring_create(nf4_ring **ring, void *slot0, void *slot1, int64_t slot_bytes,
                    void *compute_stream, void *copy_stream);
int nf4_ring_gemm(nf4_ring *ring, const uint8_t *host_codes, const uint16_t *host_scales,
                  int64_t N, int64_t K, const uint16_t *X, int64_t M, float *Y);
int64_t nf4_ring_slot_bytes(int64_t N, int64_t K);
int nf4_ring_destroy(nf4_ring *ring);

/* The 16 NF4 levels L[0..15] (fp32) this library decodes with.  Host only. */
void nf4_codebook(float out[16]);

/* Static string for an nf4_status code.  Host only. */
const char *nf4_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* NF4_H */
