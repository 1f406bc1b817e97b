// Host-only harness for the C ABI's argument handling, built with
// AddressSanitizer and UndefinedBehaviorSanitizer (host code only) by
// tests/test_sanitizers.py.  It runs every check the header documents with
// arguments that are refused before any launch (no GPU is needed), the tile
// and kernel choice of dgemm_kernel_config over many shapes of every format
// and layout, the tile map over whole grids, and the sizing helpers.  Exit
// status 0 when every returned status is the documented one.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "dgemm.h"

namespace {

int fails = 0;

void expect(int got, int want, const char* what, long long a = 0, long long b = 0) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s (%lld %lld): got %d want %d\n", what, a, b, got, want);
    ++fails;
  }
}

}  // namespace

int main() {
  alignas(16) static uint16_t buf16[64];
  alignas(16) static uint8_t buf8[64];
  alignas(16) static float buf32[64];
  alignas(16) static float out32[64];
  uint16_t* p = buf16;
  // check order: layout, dims, pointers, ld, alignment
  expect(gemm_bf16(4, 4, 4, p, 8, p, 8, p, 4, 7, nullptr), DGEMM_ERR_INVALID_LAYOUT, "layout");
  expect(gemm_bf16(-1, 4, 4, p, 8, p, 8, p, 4, DGEMM_TN, nullptr), DGEMM_ERR_INVALID_DIM, "neg M");
  expect(gemm_bf16(4, 4, -4, p, 8, p, 8, p, 4, DGEMM_TN, nullptr), DGEMM_ERR_INVALID_DIM, "neg K");
  expect(gemm_bf16(0, 4, 4, nullptr, 8, nullptr, 8, nullptr, 4, DGEMM_TN, nullptr), DGEMM_OK, "M = 0");
  expect(gemm_f32(4, 0, 4, nullptr, 8, nullptr, 8, nullptr, 4, DGEMM_NN, nullptr), DGEMM_OK, "N = 0");
  expect(gemm_f16(4, 4, 4, nullptr, 8, p, 8, p, 4, DGEMM_TN, nullptr), DGEMM_ERR_NULL_POINTER, "null A");
  expect(gemm_f16(4, 4, 4, p, 8, p, 8, nullptr, 4, DGEMM_TN, nullptr), DGEMM_ERR_NULL_POINTER, "null C");
  expect(gemm_f16(4, 4, 8, p, 7, p, 8, p, 4, DGEMM_TN, nullptr), DGEMM_ERR_INVALID_LD, "lda < K");
  expect(gemm_f16(4, 4, 8, p, 8, p, 8, p, 3, DGEMM_TN, nullptr), DGEMM_ERR_INVALID_LD, "ldc < M");
  expect(gemm_f16(4, 9, 8, p, 8, p, 8, p, 9, DGEMM_NN, nullptr), DGEMM_ERR_INVALID_LD, "NN ldb < N");
  expect(gemm_f16(4, 4, 4, p + 1, 8, p, 8, p, 4, DGEMM_TN, nullptr), DGEMM_ERR_MISALIGNED, "A base");
  expect(gemm_f16(4, 4, 4, p, 12, p, 8, p, 4, DGEMM_TN, nullptr), DGEMM_ERR_MISALIGNED, "lda pitch");
  expect(gemm_fp8(4, 4, 4, buf8, 8, buf8, 16, out32, 4, DGEMM_TN, nullptr), DGEMM_ERR_MISALIGNED, "fp8 pitch");
  expect(gemm_f32(4, 4, 4, buf32, 4, buf32, 4, (float*)((char*)out32 + 2), 4, DGEMM_NN, nullptr),
         DGEMM_ERR_MISALIGNED, "C element");
  // descriptor limits
  // (every tile has at least 128 rows of a K-contiguous operand)
  const int64_t big = (int64_t(1) << 31) / 128 / 2 + 64;
  expect(gemm_bf16(512, 512, 128, p, big, p, 128, p, 512, DGEMM_TN, nullptr), DGEMM_ERR_UNSUPPORTED, "lda limit");
  // scale factors and MX block scales
  expect(gemm_fp8_scaled(4, 4, 16, buf8, 16, buf8, 16, out32, 4, buf32, 2, buf32, 1, DGEMM_TN, nullptr),
         DGEMM_ERR_INVALID_DIM, "factor count");
  expect(gemm_fp8_scaled(4, 4, 16, buf8, 16, buf8, 16, out32, 4, nullptr, 1, buf32, 1, DGEMM_TN, nullptr),
         DGEMM_ERR_NULL_POINTER, "null factor");
  expect(gemm_mxfp8(4, 4, 48, buf8, 48, buf8, 48, out32, 4, buf8, 16, buf8, 16, DGEMM_TN, nullptr),
         DGEMM_ERR_INVALID_DIM, "MX K % 32");
  expect(gemm_mxfp8(4, 4, 64, buf8, 64, buf8, 64, out32, 4, buf8, 1, buf8, 16, DGEMM_TN, nullptr),
         DGEMM_ERR_INVALID_LD, "MX ld");
  expect(gemm_mxfp8(4, 4, 64, buf8, 64, buf8, 64, out32, 4, buf8 + 1, 16, buf8, 16, DGEMM_TN, nullptr),
         DGEMM_ERR_MISALIGNED, "MX base");
  expect(dgemm_trace_clock((unsigned long long*)buf32, -1), DGEMM_ERR_INVALID_DIM, "trace count");
  expect(dgemm_trace_clock(nullptr, 0), DGEMM_OK, "trace off");
  for (int s = -1; s < 10; ++s) expect(gemm_strerror(s) != nullptr, 1, "strerror", s);
  // kernel choice over many shapes (host planning only)
  char desc[512];
  const int64_t dims[] = {1, 7, 16, 17, 32, 33, 255, 256, 257, 1000, 4096, 8191, 8192, 14336, 28672};
  const int64_t ks[] = {0, 1, 16, 100, 128, 256, 400, 4096, 4112, 8200};
  long long configs = 0;
  for (int dt = 0; dt <= 5; ++dt)
    for (int layout = 0; layout < 2; ++layout)
      for (int64_t M : dims)
        for (int64_t N : dims)
          for (int64_t K : ks) {
            const int st = dgemm_kernel_config(dt, layout, M, N, K, desc, sizeof desc);
            const bool mx_bad = dt == 5 && K % 32 != 0;
            expect(st, mx_bad ? DGEMM_ERR_INVALID_DIM : DGEMM_OK, "kernel_config", M * 100000 + N, K);
            if (st == DGEMM_OK) expect(std::strlen(desc) > 0, 1, "description", M, N);
            ++configs;
          }
  expect(dgemm_kernel_config(1, 1, 8, 8, 8, desc, 4), DGEMM_OK, "short buffer");
  expect((int)std::strlen(desc), 3, "truncated description");
  // the tile map is a bijection on whole grids
  for (int64_t tp = 1; tp <= 40; tp += 13)
    for (int64_t tq = 1; tq <= 37; tq += 9) {
      static unsigned char seen[40 * 37];
      std::memset(seen, 0, sizeof seen);
      for (int64_t pid = 0; pid < tp * tq; ++pid) {
        int64_t a = -1, b = -1;
        expect(dgemm_tile_map(tp, tq, 8, pid, &a, &b), 0, "tile_map", tp, tq);
        if (a >= 0 && a < tp && b >= 0 && b < tq) seen[a * tq + b]++;
      }
      for (int64_t i = 0; i < tp * tq; ++i) expect(seen[i], 1, "bijection", tp, tq);
    }
  expect(dgemm_tile_map(4, 4, 8, 16, nullptr, nullptr), -1, "tile_map range");
  expect((int)dgemm_lds_bytes(256, 256, 64, 2, 0, 2), 131072, "lds bytes");
  expect((int)dgemm_lds_bytes(-1, 256, 64, 2, 0, 2), -1, "lds negative");
  std::printf("abi harness: %lld configurations, %d failures\n", configs, fails);
  return fails == 0 ? 0 : 1;
}
