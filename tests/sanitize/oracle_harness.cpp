// Host-only harness for the CPU oracle, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitizers.py.  It drives every
// exported oracle function over edge shapes (empty, one element, odd sizes,
// padded leading dimensions, row subsets with repeats) in both layouts and
// all formats, and checks that the threaded row-grouped loop and the plain
// triple loop agree bit for bit.  Exit status 0 on success.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

extern "C" {
int oracle_gemm(int in_fmt, int out_fmt, int layout, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                const void* B, int64_t ldb, const int64_t* rows, int64_t nrows, void* c_bits, double* s, double* sab,
                int nthreads);
int oracle_gemm_plain(int in_fmt, int out_fmt, int layout, int64_t M, int64_t N, int64_t K, const void* A,
                      int64_t lda, const void* B, int64_t ldb, void* c_bits, double* s, double* sab);
void oracle_decode(int fmt, const void* src, int64_t n, double* dst);
void oracle_encode(int fmt, const double* src, int64_t n, void* dst);
}

namespace {

int fails = 0;

void expect(bool ok, const char* what, int a, int b, int c) {
  if (!ok) {
    std::fprintf(stderr, "FAIL %s at %d %d %d\n", what, a, b, c);
    ++fails;
  }
}

// Random storage bits of the given width; NaN patterns are allowed.
std::vector<uint8_t> random_bytes(std::mt19937& g, size_t n) {
  std::vector<uint8_t> v(n);
  for (auto& x : v) x = (uint8_t)(g() & 0x7b);   // keep exponents moderate
  return v;
}

}  // namespace

int main() {
  std::mt19937 g(12345);
  const int in_bytes[4] = {4, 2, 2, 1};
  const int64_t dims[] = {0, 1, 2, 7, 16, 33};
  for (int fmt = 0; fmt < 4; ++fmt)
    for (int layout = 0; layout < 2; ++layout)
      for (int64_t M : dims)
        for (int64_t N : dims)
          for (int64_t K : dims) {
            const int out_fmt = fmt == 3 ? 0 : fmt;
            const int ob = out_fmt == 0 ? 4 : 2;
            const int64_t lda = K + 3, ldb = (layout == 0 ? N : K) + 5;
            const int64_t brows = layout == 0 ? K : N;
            auto A = random_bytes(g, (size_t)(M * lda + 1) * in_bytes[fmt]);
            auto B = random_bytes(g, (size_t)(brows * ldb + 1) * in_bytes[fmt]);
            std::vector<uint8_t> c1((size_t)(M * N + 1) * ob), c2((size_t)(M * N + 1) * ob);
            std::vector<double> s1(M * N + 1), s2(M * N + 1), a1(M * N + 1), a2(M * N + 1);
            int r1 = oracle_gemm(fmt, out_fmt, layout, M, N, K, A.data(), lda, B.data(), ldb, nullptr, 0,
                                 c1.data(), s1.data(), a1.data(), 3);
            int r2 = oracle_gemm_plain(fmt, out_fmt, layout, M, N, K, A.data(), lda, B.data(), ldb, c2.data(),
                                       s2.data(), a2.data());
            expect(r1 == 0 && r2 == 0, "status", (int)M, (int)N, (int)K);
            expect(std::memcmp(c1.data(), c2.data(), (size_t)(M * N) * ob) == 0, "bits", (int)M, (int)N, (int)K);
            expect(std::memcmp(s1.data(), s2.data(), (size_t)(M * N) * 8) == 0, "sums", (int)M, (int)N, (int)K);
            if (M > 1) {
              // a row subset with a repeat, against the full run
              const int64_t rows[3] = {M - 1, 0, M - 1};
              std::vector<uint8_t> c3((size_t)(3 * N + 1) * ob);
              std::vector<double> s3(3 * N + 1);
              int r3 = oracle_gemm(fmt, out_fmt, layout, M, N, K, A.data(), lda, B.data(), ldb, rows, 3,
                                   c3.data(), s3.data(), nullptr, 2);
              expect(r3 == 0, "rows status", (int)M, (int)N, (int)K);
              for (int r = 0; r < 3; ++r)
                expect(std::memcmp(&s3[(size_t)r * N], &s1[(size_t)rows[r] * N], (size_t)N * 8) == 0, "rows",
                       (int)M, (int)N, (int)K);
              // a row index out of range is refused (with N == 0 there is no work to refuse)
              const int64_t bad[1] = {M};
              expect(oracle_gemm(fmt, out_fmt, layout, M, N, K, A.data(), lda, B.data(), ldb, bad, 1, c3.data(),
                                 nullptr, nullptr, 1) == (N > 0 ? -1 : 0), "row out of range", (int)M, (int)N, (int)K);
            }
          }
  // invalid formats and layouts are refused without touching memory
  expect(oracle_gemm(7, 0, 0, 1, 1, 1, nullptr, 1, nullptr, 1, nullptr, 0, nullptr, nullptr, nullptr, 1) == -1,
         "format", 0, 0, 0);
  expect(oracle_gemm(0, 0, 5, 1, 1, 1, nullptr, 1, nullptr, 1, nullptr, 0, nullptr, nullptr, nullptr, 1) == -1,
         "layout", 0, 0, 0);
  expect(oracle_gemm(0, 0, 0, -1, 1, 1, nullptr, 1, nullptr, 1, nullptr, 0, nullptr, nullptr, nullptr, 1) == -1,
         "dims", 0, 0, 0);
  // codecs over every 16-bit pattern and back
  std::vector<uint16_t> h(65536);
  for (int i = 0; i < 65536; ++i) h[i] = (uint16_t)i;
  std::vector<double> d(65536);
  std::vector<uint16_t> back(65536);
  for (int fmt = 1; fmt <= 2; ++fmt) {
    oracle_decode(fmt, h.data(), 65536, d.data());
    oracle_encode(fmt, d.data(), 65536, back.data());
    for (int i = 0; i < 65536; ++i) {
      const bool nan = d[i] != d[i];
      expect(nan || back[i] == h[i] || ((back[i] | h[i]) & 0x7fff) == 0, "codec round trip", fmt, i, 0);
    }
  }
  std::vector<uint8_t> e8(256);
  for (int i = 0; i < 256; ++i) e8[i] = (uint8_t)i;
  oracle_decode(3, e8.data(), 256, d.data());
  std::vector<uint32_t> f32(256);
  oracle_encode(0, d.data(), 256, f32.data());
  std::printf("oracle harness: %d failures\n", fails);
  return fails == 0 ? 0 : 1;
}
