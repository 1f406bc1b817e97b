// CPU oracle for C = A x B.  TEST INFRASTRUCTURE ONLY.
//
// Only the test suite, the smoke check and the benchmark's CPU-baseline leg
// load this library.  The product (the HIP library) never calls it, shares no
// code, header, table or helper with it, and is compiled by a different
// compiler (this file is built with g++ -O2 -fopenmp, no fast-math).
//
// What it computes is the plain definition of the product, not an algorithm to
// mirror:
//   * "Optimizing GEMM in HIP" (ROCm optimization guide), section "GEMM
//     fundamentals": C_ij is the inner product of row i of A and column j of
//     B; a CPU implementation is three nested loops, 2*M*N*K operations.
//   * "FP16 GEMM Optimization on AMD RDNA 3 and RDNA 4", section "What We Are
//     Computing": the TN storage pairing (A row-major, B column-major, C
//     column-major with leading dimension M).
//   * "FP8 GEMM Optimization on AMD RDNA 4", section "What Changes at FP8":
//     E4M3 operands, FP32 accumulation and FP32 output, no scale factors.
//
// For every output element (i, j):
//   1. decode a(i,k), b(k,j) exactly from their storage format;
//   2. s   = sum_k a(i,k) * b(k,j)    in FP64, one accumulator, k ascending;
//   3. sab = sum_k |a(i,k) * b(k,j)|  in FP64, same pass;
//   4. c   = s rounded ONCE, round-to-nearest-even, to the output format.
// Products of two FP32 (or narrower) values are exact in FP64 (24+24 <= 53
// significand bits), so the only rounding before step 4 is FP64 addition.
//
// Threads split the rows; every (i, j) is summed by one thread in one fixed
// order, so the result does not depend on the thread count.
//
// Parity status: pinned (brute force against exact rationals, closed forms,
// identity, +-1 exactness, exhaustive codec checks against library casts).

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>
#include <omp.h>

namespace {

enum Fmt { FMT_F32 = 0, FMT_F16 = 1, FMT_BF16 = 2, FMT_E4M3 = 3 };
enum Layout { LAYOUT_NN = 0, LAYOUT_TN = 1 };

// ---- exact decoders (format definitions) ----------------------------------

// IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
double dec_f16(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
  double v;
  if (e == 0)        v = std::ldexp((double)m, -24);              // subnormal
  else if (e == 31)  v = m ? NAN : INFINITY;
  else               v = std::ldexp((double)(1024 + m), e - 25);  // (1.m) * 2^(e-15)
  return s ? -v : v;
}

// bfloat16: the upper half of an IEEE binary32.
double dec_bf16(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// OCP FP8 E4M3 ("E4M3FN"): 1 sign, 4 exponent (bias 7), 3 fraction bits,
// exponent field 0 is subnormal (m * 2^-9), S.1111.111 is NaN, no infinity.
double dec_e4m3(uint8_t b) {
  const int s = b >> 7, e = (b >> 3) & 0xf, m = b & 7;
  double v;
  if (e == 0)                 v = std::ldexp((double)m, -9);
  else if (e == 15 && m == 7) v = NAN;
  else                        v = std::ldexp((double)(8 + m), e - 10);  // (1.m) * 2^(e-7)
  return s ? -v : v;
}

double dec_f32(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

double decode(int fmt, const void* base, int64_t idx) {
  switch (fmt) {
    case FMT_F32:  return dec_f32(((const uint32_t*)base)[idx]);
    case FMT_F16:  return dec_f16(((const uint16_t*)base)[idx]);
    case FMT_BF16: return dec_bf16(((const uint16_t*)base)[idx]);
    default:       return dec_e4m3(((const uint8_t*)base)[idx]);
  }
}

// ---- round-to-nearest-even encoders from FP64 ------------------------------
// Both narrow formats are handled the same way: write |x| = q * 2^(E - P + 1)
// with E = floor(log2|x|) and P significand bits, round q to an integer with
// ties to even (std::nearbyint under the default rounding mode), and renormalise
// if the rounding carried into the next binade.  Below the smallest normal
// exponent the quantum is fixed at the subnormal spacing.

uint16_t enc_narrow(double x, int P, int emin, int emax, int ebias, uint16_t nan_bits) {
  const uint16_t sign = std::signbit(x) ? (uint16_t)(1u << 15) : 0;
  const int fbits = P - 1;
  const uint16_t inf_bits = (uint16_t)(((emax + ebias + 1) << fbits));
  if (std::isnan(x)) return nan_bits;
  double a = std::fabs(x);
  if (std::isinf(a)) return sign | inf_bits;
  if (a == 0.0) return sign;
  int e2;
  std::frexp(a, &e2);                 // a = f * 2^e2, f in [0.5, 1)
  int E = e2 - 1;                     // a in [2^E, 2^(E+1))
  if (E < emin) {                     // subnormal range: quantum 2^(emin - fbits)
    double q = std::nearbyint(std::ldexp(a, fbits - emin));
    // q == 2^fbits lands exactly on the smallest normal, whose encoding is q.
    return sign | (uint16_t)q;
  }
  double q = std::nearbyint(std::ldexp(a, fbits - E));   // in [2^fbits, 2^P]
  if (q == std::ldexp(1.0, P)) { q = std::ldexp(1.0, fbits); ++E; }
  if (E > emax) return sign | inf_bits;
  return sign | (uint16_t)((E + ebias) << fbits) | (uint16_t)(q - std::ldexp(1.0, fbits));
}

uint16_t enc_f16(double x)  { return enc_narrow(x, 11, -14, 15, 15, 0x7e00); }
uint16_t enc_bf16(double x) { return enc_narrow(x, 8, -126, 127, 127, 0x7fc0); }

uint32_t enc_f32(double x) {
  const float f = (float)x;           // IEEE conversion, default rounding (nearest-even)
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

int in_bytes(int fmt) { return fmt == FMT_F32 ? 4 : (fmt == FMT_E4M3 ? 1 : 2); }

}  // namespace

extern "C" {

// Core entry point.
//   in_fmt  : 0 f32, 1 f16, 2 bf16, 3 e4m3 (both operands)
//   out_fmt : 0 f32, 1 f16, 2 bf16
//   layout  : 0 NN (A[i*lda+k], B[k*ldb+j]), 1 TN (A[i*lda+k], B[j*ldb+k])
//   rows    : the row indices i to compute (nrows of them); NULL means all M
//   c_bits  : [nrows][N] output-format bit patterns (4 or 2 bytes each), or NULL
//   s, sab  : [nrows][N] FP64 sums and absolute sums, or NULL
//   nthreads: OpenMP threads, <= 0 for the runtime default
// Returns 0, or -1 on a bad argument.
int oracle_gemm(int in_fmt, int out_fmt, int layout, int64_t M, int64_t N, int64_t K,
                const void* A, int64_t lda, const void* B, int64_t ldb,
                const int64_t* rows, int64_t nrows,
                void* c_bits, double* s, double* sab, int nthreads) {
  if (in_fmt < 0 || in_fmt > 3 || out_fmt < 0 || out_fmt > 2) return -1;
  if (layout != LAYOUT_NN && layout != LAYOUT_TN) return -1;
  if (M < 0 || N < 0 || K < 0) return -1;
  if (!rows) nrows = M;
  if (nrows == 0 || N == 0) return 0;
  if (rows)
    for (int64_t r = 0; r < nrows; ++r)
      if (rows[r] < 0 || rows[r] >= M) return -1;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  (void)in_bytes;

  // Exact widening to FP32 storage with K contiguous (every f16, bf16 and
  // E4M3 value is an FP32 value, so this changes no value).
  std::vector<float> a((size_t)nrows * (size_t)K), b((size_t)N * (size_t)K);
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t i = rows ? rows[r] : r;
    for (int64_t k = 0; k < K; ++k) a[(size_t)r * K + k] = (float)decode(in_fmt, A, i * lda + k);
  }
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t j = 0; j < N; ++j)
    for (int64_t k = 0; k < K; ++k) {
      const int64_t idx = layout == LAYOUT_NN ? k * ldb + j : j * ldb + k;
      b[(size_t)j * K + k] = (float)decode(in_fmt, B, idx);
    }

  // Rows in groups of 4 so each streamed column of B serves four rows.  The
  // order of operations for any single (i, j) is the same as in the plain
  // triple loop: one FP64 accumulator, k ascending.
  const int64_t ngroups = (nrows + 3) / 4;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
  for (int64_t g = 0; g < ngroups; ++g) {
    const int64_t r0 = g * 4;
    const int64_t rn = (nrows - r0) < 4 ? (nrows - r0) : 4;
    for (int64_t j = 0; j < N; ++j) {
      double acc[4] = {0, 0, 0, 0}, aab[4] = {0, 0, 0, 0};
      const float* bj = b.data() + (size_t)j * K;   // (no element when K == 0)
      for (int64_t k = 0; k < K; ++k) {
        const double bv = (double)bj[k];
        for (int64_t q = 0; q < rn; ++q) {
          const double p = (double)a[(size_t)(r0 + q) * K + k] * bv;
          acc[q] += p;
          aab[q] += std::fabs(p);
        }
      }
      for (int64_t q = 0; q < rn; ++q) {
        const size_t o = (size_t)(r0 + q) * (size_t)N + (size_t)j;
        if (s) s[o] = acc[q];
        if (sab) sab[o] = aab[q];
        if (c_bits) {
          if (out_fmt == FMT_F32)       ((uint32_t*)c_bits)[o] = enc_f32(acc[q]);
          else if (out_fmt == FMT_F16)  ((uint16_t*)c_bits)[o] = enc_f16(acc[q]);
          else                          ((uint16_t*)c_bits)[o] = enc_bf16(acc[q]);
        }
      }
    }
  }
  return 0;
}

// Single-threaded, unblocked i-j-k triple loop with the same per-element
// arithmetic.  Used only to show that the row-grouped, threaded loop above
// produces the same bits.
int oracle_gemm_plain(int in_fmt, int out_fmt, int layout, int64_t M, int64_t N, int64_t K,
                      const void* A, int64_t lda, const void* B, int64_t ldb,
                      void* c_bits, double* s, double* sab) {
  if (in_fmt < 0 || in_fmt > 3 || out_fmt < 0 || out_fmt > 2) return -1;
  if (layout != LAYOUT_NN && layout != LAYOUT_TN) return -1;
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < N; ++j) {
      double acc = 0, aab = 0;
      for (int64_t k = 0; k < K; ++k) {
        const double av = decode(in_fmt, A, i * lda + k);
        const double bv = decode(in_fmt, B, layout == LAYOUT_NN ? k * ldb + j : j * ldb + k);
        acc += av * bv;
        aab += std::fabs(av * bv);
      }
      const size_t o = (size_t)i * (size_t)N + (size_t)j;
      if (s) s[o] = acc;
      if (sab) sab[o] = aab;
      if (c_bits) {
        if (out_fmt == FMT_F32)       ((uint32_t*)c_bits)[o] = enc_f32(acc);
        else if (out_fmt == FMT_F16)  ((uint16_t*)c_bits)[o] = enc_f16(acc);
        else                          ((uint16_t*)c_bits)[o] = enc_bf16(acc);
      }
    }
  return 0;
}

// Codec access for the self-tests and the library-product check.  Each
// element is converted on its own; threads only split the range.
void oracle_decode(int fmt, const void* src, int64_t n, double* dst) {
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t i = 0; i < n; ++i) dst[i] = decode(fmt, src, i);
}

// fmt: 0 f32 (uint32 out), 1 f16, 2 bf16 (uint16 out)
void oracle_encode(int fmt, const double* src, int64_t n, void* dst) {
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t i = 0; i < n; ++i) {
    if (fmt == FMT_F32)      ((uint32_t*)dst)[i] = enc_f32(src[i]);
    else if (fmt == FMT_F16) ((uint16_t*)dst)[i] = enc_f16(src[i]);
    else                     ((uint16_t*)dst)[i] = enc_bf16(src[i]);
  }
}

int oracle_max_threads(void) { return omp_get_max_threads(); }

}  // extern "C"
