// nf4_oracle.cpp -- plain fp64 CPU reference for the NF4 dequant-GEMV path.
//
// TEST INFRASTRUCTURE ONLY (see nf4_oracle.h): used by the tests, the smoke
// check and the bench's CPU-baseline leg, never by the product library.  It is
// written for a reader checking it against the sources by eye: no blocking, no
// fusion, no reordering beyond the plain definitions.
//
// Readings of points the sources leave open are stated where they are taken.
#include "nf4_oracle.h"

#include <cmath>
#include <cstring>

// ---------------------------------------------------------------------------
// Normal quantile.  QLoRA builds NF4 from quantiles of N(0,1).  The quantile is
// the root of a tail probability written with libm's erfc: below 1/2 the lower
// tail Phi(x) = erfc(-x/sqrt 2)/2 equals p; above 1/2 the upper tail
// erfc(x/sqrt 2)/2 equals 1 - p (exact in fp64 there).  Working on the tail
// keeps full relative precision away from the centre.  Newton steps fall back
// to bisection whenever a step leaves the bracket.
// ---------------------------------------------------------------------------
static double normal_pdf(double x) {
  const double pi = 3.14159265358979323846;
  return std::exp(-0.5 * x * x) / std::sqrt(2.0 * pi);
}

extern "C" double orc_normal_quantile(double p) {
  if (!(p > 0.0 && p < 1.0)) return std::nan("");
  if (p == 0.5) return 0.0;
  const bool upper = p > 0.5;
  const double target = upper ? 1.0 - p : p;  // tail probability, < 1/2
  // g(x) = tail(x) - target is increasing in x for the lower tail and
  // decreasing for the upper tail
  double lo = upper ? 0.0 : -40.0, hi = upper ? 40.0 : 0.0;
  double x = upper ? 1.0 : -1.0;
  for (int it = 0; it < 300; ++it) {
    double tail = upper ? 0.5 * std::erfc(x / std::sqrt(2.0))
                        : 0.5 * std::erfc(-x / std::sqrt(2.0));
    double f = tail - target;
    if (f == 0.0) return x;
    double slope = upper ? -normal_pdf(x) : normal_pdf(x);
    // root lies where f changes sign
    if ((f < 0.0) == !upper) lo = x; else hi = x;
    double nx = x - f / slope;
    if (!(nx > lo && nx < hi)) nx = 0.5 * (lo + hi);  // keep inside the bracket
    if (nx == x) break;
    x = nx;
  }
  return x;
}

// ---------------------------------------------------------------------------
// Codebook (QLoRA, 4-bit NormalFloat).  Reading of the construction:
//   delta = (1 - 1/30 + 1 - 1/32) / 2 (the average of the two tail offsets);
//   8 positive levels: quantiles at 8 probabilities evenly spaced from delta
//     down towards 1/2 on a 9-point grid, the 1/2 end point dropped;
//   7 negative levels: minus the quantiles on an 8-point grid from delta to
//     1/2, the 1/2 end point dropped;
//   an exact 0; all 16 sorted ascending and divided by the largest magnitude.
// The stored table is each level rounded to fp32 (round to nearest even, the
// C conversion).  Quantizer and dequantizer both use the fp32 values.
// ---------------------------------------------------------------------------
extern "C" void orc_codebook(double lv64[16], float lv32[16]) {
  const double delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0));
  double v[16];
  int n = 0;
  // positive side: 9-point grid from delta to 1/2, keep the first 8 points
  for (int i = 0; i < 8; ++i) {
    double p = delta + (0.5 - delta) * (double)i / 8.0;
    v[n++] = orc_normal_quantile(p);
  }
  // negative side: 8-point grid from delta to 1/2, keep the first 7 points
  for (int i = 0; i < 7; ++i) {
    double p = delta + (0.5 - delta) * (double)i / 7.0;
    v[n++] = -orc_normal_quantile(p);
  }
  v[n++] = 0.0;
  // sort ascending (insertion sort: 16 values)
  for (int i = 1; i < 16; ++i) {
    double t = v[i];
    int j = i - 1;
    while (j >= 0 && v[j] > t) { v[j + 1] = v[j]; --j; }
    v[j + 1] = t;
  }
  double mx = 0.0;
  for (int i = 0; i < 16; ++i) mx = std::fmax(mx, std::fabs(v[i]));
  for (int i = 0; i < 16; ++i) {
    lv64[i] = v[i] / mx;
    lv32[i] = (float)lv64[i];
  }
}

// ---------------------------------------------------------------------------
// binary16 helpers.  Rounding is written out from the definition: the value is
// the nearest multiple of the binade's spacing, ties to the even multiple
// (nearbyint under the default rounding mode).
// ---------------------------------------------------------------------------
extern "C" uint16_t orc_f32_to_f16_bits(float f) {
  uint32_t fb;
  std::memcpy(&fb, &f, 4);
  uint16_t sign = (uint16_t)((fb >> 16) & 0x8000u);
  double a = std::fabs((double)f);
  if (std::isnan(a)) return (uint16_t)(sign | 0x7E00u);
  if (a == 0.0) return sign;
  // binade exponent E with 2^E <= a < 2^(E+1)
  int e2;
  std::frexp(a, &e2);
  int E = e2 - 1;
  int Eq = E < -14 ? -14 : E;               // subnormals share the 2^-14 spacing
  double quantum = std::ldexp(1.0, Eq - 10);  // 10 fraction bits
  double r = std::nearbyint(a / quantum) * quantum;
  if (r >= 65536.0) return (uint16_t)(sign | 0x7C00u);  // rounds past the max
  if (r == 0.0) return sign;
  if (r < std::ldexp(1.0, -14)) {  // subnormal: value = m * 2^-24
    uint16_t m = (uint16_t)(r / std::ldexp(1.0, -24));
    return (uint16_t)(sign | m);
  }
  std::frexp(r, &e2);
  int Er = e2 - 1;
  uint16_t mant = (uint16_t)(r / std::ldexp(1.0, Er - 10) - 1024.0);
  return (uint16_t)(sign | (uint16_t)((Er + 15) << 10) | mant);
}

extern "C" double orc_f16_bits_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 0x1F;
  int mant = h & 0x3FF;
  double v;
  if (ex == 0) v = std::ldexp((double)mant, -24);
  else if (ex == 31) v = mant ? std::nan("") : INFINITY;
  else v = std::ldexp(1024.0 + (double)mant, ex - 25);
  return sign ? -v : v;
}

extern "C" double orc_bf16_bits_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;  // bf16 is the top half of a binary32
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// ---------------------------------------------------------------------------
// Quantize (deep-fold README, Method: one FP16 scale per group of 64; NF4
// codes).  Readings:
//   scale s = fp16(absmax of the group), round to nearest even;
//   code   = index of the level L[c]*s nearest in value to w; the boundary
//            between codes c and c+1 sits at T_c = (L[c]+L[c+1])/2 * s, and a
//            weight exactly on a boundary takes the lower code.  In fp64 the
//            midpoint and the product are exact (fp32 levels of one binade or
//            adjacent to 0, times an 11-bit scale), so the count below is the
//            exact nearest-level rule;
//   s = 0 (all-zero group, or absmax below half the smallest fp16 subnormal):
//            every dequantized weight is 0 whatever the code; the code is the
//            zero level, 7;
//   NaN/inf in the group, or absmax rounding to fp16 infinity: flagged in the
//            returned status; the group is written as scale 0, codes 7.
// ---------------------------------------------------------------------------
extern "C" int32_t orc_quantize(const float *W, int64_t N, int64_t K, uint8_t *codes,
                                uint16_t *scales) {
  double lv64[16];
  float L[16];
  orc_codebook(lv64, L);
  int32_t status = 0;
  const int64_t G = K / 64;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t g = 0; g < G; ++g) {
      const float *w = W + n * K + g * 64;
      uint8_t *c = codes + n * K + g * 64;
      int bad = 0;
      float amax = 0.0f;
      for (int k = 0; k < 64; ++k) {
        if (!std::isfinite(w[k])) bad |= ORC_STATUS_NONFINITE;
        else amax = std::fmax(amax, std::fabs(w[k]));
      }
      uint16_t sb = 0;
      if (!bad) {
        sb = orc_f32_to_f16_bits(amax);
        if ((sb & 0x7C00u) == 0x7C00u) bad |= ORC_STATUS_SCALE_OVERFLOW;
      }
      if (bad) {
        status |= bad;
        scales[n * G + g] = 0;
        for (int k = 0; k < 64; ++k) c[k] = 7;
        continue;
      }
      scales[n * G + g] = sb;
      double s = orc_f16_bits_to_f64(sb);
      for (int k = 0; k < 64; ++k) {
        if (s == 0.0) { c[k] = 7; continue; }
        int code = 0;
        for (int i = 0; i < 15; ++i) {
          double T = (((double)L[i] + (double)L[i + 1]) / 2.0) * s;
          if ((double)w[k] > T) code += 1;
        }
        c[k] = (uint8_t)code;
      }
    }
  }
  return status;
}

extern "C" void orc_pack(const uint8_t *codes, int64_t N, int64_t K, uint8_t *packed) {
  for (int64_t n = 0; n < N; ++n)
    for (int64_t j = 0; j < K / 2; ++j) {
      uint8_t lo = codes[n * K + 2 * j] & 0xF;
      uint8_t hi = codes[n * K + 2 * j + 1] & 0xF;
      packed[n * (K / 2) + j] = (uint8_t)(lo | (hi << 4));
    }
}

extern "C" void orc_unpack_codes(const uint8_t *packed, int64_t N, int64_t K,
                                 uint8_t *codes) {
  for (int64_t n = 0; n < N; ++n)
    for (int64_t j = 0; j < K / 2; ++j) {
      uint8_t b = packed[n * (K / 2) + j];
      codes[n * K + 2 * j] = b & 0xF;
      codes[n * K + 2 * j + 1] = b >> 4;
    }
}

// code of weight (n, k) from the packed bytes
static int code_at(const uint8_t *packed, int64_t K, int64_t n, int64_t k) {
  uint8_t b = packed[n * (K / 2) + k / 2];
  return (k % 2 == 0) ? (b & 0xF) : (b >> 4);
}

// ---------------------------------------------------------------------------
// Dequantize (deep-fold README, Method: the value of a weight is its level
// times its group's scale; NF4 has an exact zero level, so no offset).
// ---------------------------------------------------------------------------
extern "C" void orc_dequant_f64(const uint8_t *packed, const uint16_t *scales, int64_t N,
                                int64_t K, double *Wt) {
  double lv64[16];
  float L[16];
  orc_codebook(lv64, L);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      double s = orc_f16_bits_to_f64(scales[n * (K / 64) + k / 64]);
      Wt[n * K + k] = (double)L[code_at(packed, K, n, k)] * s;
    }
}

extern "C" void orc_dequant_f32(const uint8_t *packed, const uint16_t *scales, int64_t N,
                                int64_t K, float *Wt) {
  double lv64[16];
  float L[16];
  orc_codebook(lv64, L);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      double s = orc_f16_bits_to_f64(scales[n * (K / 64) + k / 64]);
      // the fp64 product is exact, so this is one correctly rounded fp32 multiply
      Wt[n * K + k] = (float)((double)L[code_at(packed, K, n, k)] * s);
    }
}

// ---------------------------------------------------------------------------
// Product (Trapetum overview: decode is y = W x over the stored weights;
// deep-fold README: prefill runs the same product on chunks of up to 32 rows of
// activations).  y = dequant(codes, scales) . x, in fp64, k ascending.  Each
// term is exact in fp64; only the running sum rounds.
// ---------------------------------------------------------------------------
extern "C" void orc_gemm_rows(const uint8_t *packed, const uint16_t *scales, int64_t N,
                              int64_t K, const uint16_t *X, int64_t M, const int64_t *rows,
                              int64_t nrows, double *Y, double *A) {
  double lv64[16];
  float L[16];
  orc_codebook(lv64, L);
  for (int64_t m = 0; m < M; ++m)
    for (int64_t r = 0; r < nrows; ++r) {
      int64_t n = rows ? rows[r] : r;
      double acc = 0.0, aacc = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double s = orc_f16_bits_to_f64(scales[n * (K / 64) + k / 64]);
        double w = (double)L[code_at(packed, K, n, k)] * s;
        double x = orc_bf16_bits_to_f64(X[m * K + k]);
        acc += w * x;
        aacc += std::fabs(w * x);
      }
      Y[m * nrows + r] = acc;
      if (A) A[m * nrows + r] = aacc;
    }
  (void)N;
}

// ---------------------------------------------------------------------------
// Rounding to bfloat16 (8 significant bits, the binary32 exponent range): the
// nearest bf16 value to v, ties to the even significand.  Written out on the
// exact value: the significand scaled to an integer range, rounded by hand.
extern "C" uint16_t orc_f64_to_bf16_bits(double v) {
  if (std::isnan(v)) return 0x7FC0;
  const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  const double a = std::fabs(v);
  if (std::isinf(a)) return sign | 0x7F80;
  if (a == 0.0) return sign;
  // a = q * 2^e2 with q an integer multiple of the bf16 spacing at a's binade:
  // normal range (a >= 2^-126): 8 significant bits; below, spacing 2^-133.
  int e = 0;
  (void)std::frexp(a, &e);                 // a in [2^(e-1), 2^e)
  int e2 = (e - 1 >= -126) ? (e - 8) : -133;  // spacing of bf16 values near a
  const double q = std::ldexp(a, -e2);     // exact: a power-of-two scaling
  double fl = std::floor(q);
  const double rem = q - fl;               // exact
  if (rem > 0.5 || (rem == 0.5 && std::fmod(fl, 2.0) != 0.0)) fl += 1.0;
  const double r = std::ldexp(fl, e2);     // the rounded value, exactly a bf16
  if (r >= std::ldexp(1.0, 128)) return sign | 0x7F80;  // rounds past the largest
  const float f = (float)r;                // exact: every bf16 value is a binary32
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

// ---------------------------------------------------------------------------
// Packed embedding rows: decode only the requested rows (deep-fold README,
// Method: embeddings decode the requested rows), w~ = L[c] * s exact in fp64,
// then one rounding to bf16.  An id outside [0, N) yields a zero row and the
// status bit.
extern "C" int32_t orc_embed(const uint8_t *packed, const uint16_t *scales, int64_t N,
                             int64_t K, const int64_t *ids, int64_t T, uint16_t *out) {
  double lv64[16];
  float lv32[16];
  orc_codebook(lv64, lv32);
  int32_t status = 0;
  const int64_t G = K / 64;
  for (int64_t t = 0; t < T; ++t) {
    const int64_t n = ids[t];
    uint16_t *o = out + t * K;
    if (n < 0 || n >= N) {
      status |= ORC_EMBED_BAD_ID;
      for (int64_t k = 0; k < K; ++k) o[k] = 0;
      continue;
    }
    for (int64_t k = 0; k < K; ++k) {
      const uint8_t byte = packed[n * (K / 2) + k / 2];
      const int c = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
      const double s = orc_f16_bits_to_f64(scales[n * G + k / 64]);
      o[k] = orc_f64_to_bf16_bits((double)lv32[c] * s);
    }
  }
  return status;
}
