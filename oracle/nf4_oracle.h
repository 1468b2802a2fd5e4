/*
 * nf4_oracle.h -- plain, slow, fp64 CPU reference for the NF4 dequant-GEMV path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes, links or
 * calls this code; only the tests, the package's smoke check and the bench's CPU
 * baseline leg do.  It shares no code, header, table or constant with the HIP
 * implementation: the codebook is regenerated here from its definition.
 *
 * Method (sources):
 *  - deep-fold README, "Method" section: weights are stored as 4-bit NF4 codes
 *    in groups of 64 consecutive weights, each group carrying one FP16 scale;
 *    linear kernels rebuild the values they need while they multiply and never
 *    write a dense weight matrix back.
 *  - deep-fold README, "Method" section: NF4 is the data type of QLoRA
 *    (Dettmers et al., 2023, section on 4-bit NormalFloat quantization), whose
 *    construction the codebook below follows.
 *  - Trapetum overview, "In one sentence" / "The bandwidth law": decode is a
 *    matrix-vector product whose cost is reading the weights.
 *
 * Layout (identical reading on both sides; the README's layout page is missing):
 *  - W is [N][K] row-major fp32, K a multiple of 64; groups run along K.
 *  - packed codes: [N][K/2] bytes; byte j of row n holds code(n, 2j) in its low
 *    nibble and code(n, 2j+1) in its high nibble.
 *  - scales: [N][K/64] IEEE binary16 bit patterns, row-major.
 *  - x / X: bf16 bit patterns, X is [M][K] row-major; y / Y fp64 [M][N].
 *
 * All functions are single-threaded, allocate nothing the caller must free,
 * and never touch a GPU.
 */
#ifndef NF4_ORACLE_H
#define NF4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status bits written by orc_quantize (per call, OR of all groups) */
#define ORC_STATUS_NONFINITE 1      /* a group holds NaN or +-inf            */
#define ORC_STATUS_SCALE_OVERFLOW 2 /* group absmax rounds to fp16 infinity  */

/* Standard normal quantile: the x with Phi(x) = p, 0 < p < 1.  Safeguarded
 * Newton iteration on Phi(x) = erfc(-x/sqrt 2)/2 (libm erfc). */
double orc_normal_quantile(double p);

/* QLoRA NF4 codebook: lv64 = the 16 levels in fp64, lv32 = each rounded to
 * fp32 (round to nearest even).  The fp32 values are the stored table. */
void orc_codebook(double lv64[16], float lv32[16]);

/* IEEE binary32 -> binary16, round to nearest, ties to even; returns bits. */
uint16_t orc_f32_to_f16_bits(float f);
/* binary16 bits -> exact value; bf16 bits -> exact value. */
double orc_f16_bits_to_f64(uint16_t h);
double orc_bf16_bits_to_f64(uint16_t b);

/* Quantize W [N][K] to one code per byte (unpacked, codes[N][K]) and fp16
 * scales [N][K/64].  Returns the OR of ORC_STATUS_* bits over all groups;
 * a flagged group gets scale bits 0 and every code 7. */
int32_t orc_quantize(const float *W, int64_t N, int64_t K, uint8_t *codes,
                     uint16_t *scales);

/* Two codes per byte, low nibble = even k. */
void orc_pack(const uint8_t *codes, int64_t N, int64_t K, uint8_t *packed);
void orc_unpack_codes(const uint8_t *packed, int64_t N, int64_t K, uint8_t *codes);

/* Dequantize: w~ = L[c] * s exactly in fp64, and its fp32 rounding. */
void orc_dequant_f64(const uint8_t *packed, const uint16_t *scales, int64_t N,
                     int64_t K, double *Wt);
void orc_dequant_f32(const uint8_t *packed, const uint16_t *scales, int64_t N,
                     int64_t K, float *Wt);

/* Y[m][r] = sum_k w~[rows[r]][k] * X[m][k] (fp64, k ascending), and
 * A[m][r] = sum_k |w~[rows[r]][k] * X[m][k]| for the tolerance.  rows == NULL
 * means every row 0..N-1 (nrows must then equal N).  A may be NULL. */
void orc_gemm_rows(const uint8_t *packed, const uint16_t *scales, int64_t N,
                   int64_t K, const uint16_t *X, int64_t M, const int64_t *rows,
                   int64_t nrows, double *Y, double *A);

/* exact value -> bfloat16 bits, one rounding to nearest, ties to even (8
 * significant bits, binary32 exponent range, subnormals kept); any NaN gives
 * the quiet NaN 0x7FC0. */
uint16_t orc_f64_to_bf16_bits(double v);

/* status bit written by orc_embed */
#define ORC_EMBED_BAD_ID 1 /* an id outside [0, N): that output row is zero */

/* Packed embedding rows (deep-fold README: embeddings decode only the requested
 * rows): out[t][k] = bf16(w~[ids[t]][k]) for t < T, w~ = L[c] * s exact, one
 * rounding.  out is bf16 bits [T][K].  Returns ORC_EMBED_BAD_ID if any id is
 * out of range (those rows are all +0), else 0. */
int32_t orc_embed(const uint8_t *packed, const uint16_t *scales, int64_t N, int64_t K,
                  const int64_t *ids, int64_t T, uint16_t *out);

#ifdef __cplusplus
}
#endif
#endif
