/*
 * dgemm.h -- C ABI of libdgemm.so: tiled dense GEMM C = A x B on MI355X (gfx950).
 *
 * Operation.  Every entry point computes C = A x B, C_ij = sum_k A_ik * B_kj,
 * 2*M*N*K flops ("Optimizing GEMM in HIP", ROCm optimization guide, section
 * "GEMM fundamentals"), with products and sums in FP32 (FP32 accumulation for
 * every input format) and one conversion of each FP32 result to the output
 * format with round-to-nearest-even.  C is overwritten (no alpha/beta).
 *
 * Layouts (leading dimensions are in ELEMENTS):
 *   DGEMM_NN  A is M x K row-major       A(i,k) = A[i*lda + k],  lda >= K
 *             B is K x N row-major       B(k,j) = B[k*ldb + j],  ldb >= N
 *             C is M x N row-major       C(i,j) = C[i*ldc + j],  ldc >= N
 *   DGEMM_TN  the pairing named TN in "FP16 GEMM Optimization on AMD RDNA 3
 *             and RDNA 4", section "What We Are Computing": both operands
 *             contiguous along K, C column-major.
 *             A is M x K row-major       A(i,k) = A[i*lda + k],  lda >= K
 *             B is K x N column-major    B(k,j) = B[j*ldb + k],  ldb >= K
 *             C is M x N column-major    C(i,j) = C[j*ldc + i],  ldc >= M
 *
 * Formats: FP32 = IEEE binary32; FP16 = IEEE binary16 bits; BF16 = bfloat16
 * bits; FP8 = OCP E4M3 ("E4M3FN": bias 7, max 448, no infinity) bytes, used
 * raw with no scale factors ("FP8 GEMM Optimization on AMD RDNA 4", section
 * "What Changes at FP8"), producing FP32 output.
 *
 * Memory and ownership.  A, B and C are DEVICE pointers owned by the caller;
 * the library never allocates, frees or retains them and keeps no mutable
 * global state (beyond two thread-local diagnostics: the last HIP error code
 * and the clock-trace buffer set with dgemm_trace_clock), so calls are
 * reentrant.
 * A and B must not overlap C, and must be readable over whole rows of
 * their pitch: A over M*lda elements, B over K*ldb (NN) or N*ldb (TN); the
 * kernels copy 16-byte pieces and may read the padding of the last row.
 * Alignment: A and B must be 16-byte aligned and lda*elem, ldb*elem must be
 * multiples of 16 bytes (elem = bytes per input element); C needs only its
 * element alignment (wider stores are used when C and ldc allow them).
 * Size limits: the bytes one block tile addresses in an operand must stay
 * below 2^31 (for a K-contiguous operand: 256 rows * ld * elem; for the NN
 * B operand: K * ldb * elem); beyond that the call returns DGEMM_ERR_UNSUPPORTED.
 *
 * Streams.  The work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and the call returns without synchronising.  Faults inside the
 * kernel surface at the caller's next synchronisation.
 *
 * Errors.  Each call returns a dgemm_status and never prints or aborts; the
 * code of the last HIP failure is kept per thread (dgemm_last_hip_error).
 * Checks, in this order: layout -> DGEMM_ERR_INVALID_LAYOUT; any of M, N, K
 * negative -> DGEMM_ERR_INVALID_DIM; M == 0 or N == 0 -> DGEMM_OK with no
 * work; a NULL A or B (when K > 0) or NULL C -> DGEMM_ERR_NULL_POINTER; a
 * leading dimension below its minimum -> DGEMM_ERR_INVALID_LD; misaligned A
 * or B base or pitch -> DGEMM_ERR_MISALIGNED; size limits ->
 * DGEMM_ERR_UNSUPPORTED; a HIP launch error -> DGEMM_ERR_HIP.
 * K == 0 is valid: C is filled with zeros (the empty sum).
 */
#ifndef DGEMM_H
#define DGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DGEMM_NN = 0, DGEMM_TN = 1 } dgemm_layout;

typedef enum {
  DGEMM_OK = 0,
  DGEMM_ERR_INVALID_DIM = 1,
  DGEMM_ERR_NULL_POINTER = 2,
  DGEMM_ERR_INVALID_LD = 3,
  DGEMM_ERR_INVALID_LAYOUT = 4,
  DGEMM_ERR_MISALIGNED = 5,
  DGEMM_ERR_UNSUPPORTED = 6,
  DGEMM_ERR_HIP = 7
} dgemm_status;

/* FP32 x FP32 -> FP32. */
int gemm_f32(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
             const float* B, int64_t ldb, float* C, int64_t ldc, int layout, void* stream);

/* FP16 x FP16 -> FP16 (binary16 bit patterns), FP32 accumulation. */
int gemm_f16(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
             const uint16_t* B, int64_t ldb, uint16_t* C, int64_t ldc, int layout, void* stream);

/* BF16 x BF16 -> BF16 (bfloat16 bit patterns), FP32 accumulation. */
int gemm_bf16(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
              const uint16_t* B, int64_t ldb, uint16_t* C, int64_t ldc, int layout, void* stream);

/* OCP FP8 E4M3 x E4M3 -> FP32, FP32 accumulation, no scale factors. */
int gemm_fp8(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
             const uint8_t* B, int64_t ldb, float* C, int64_t ldc, int layout, void* stream);

/*
 * OCP FP8 E4M3 x E4M3 -> FP32 with scale factors, the per-tensor or per-row
 * factors a quantized kernel carries on top of the raw FP8 product ("FP8
 * GEMM Optimization on AMD RDNA 4", section "What Changes at FP8"):
 *   C_ij = (sum_k A_ik * B_kj) * (sa_i * sb_j)
 * with the sum accumulated in FP32 as in gemm_fp8 and each of the two
 * products rounded to FP32 (round-to-nearest-even); IEEE rules apply to
 * zero, infinite and NaN factors (K == 0 gives 0 * sa_i * sb_j).
 * scale_a: DEVICE pointer to n_scale_a FP32 values, n_scale_a = 1 (sa_i =
 *          scale_a[0] for every i) or M (sa_i = scale_a[i], one per row of A);
 * scale_b: DEVICE pointer to n_scale_b FP32 values, 1 or N (one per column
 *          of B, whatever the layout).
 * Both are read by the kernel at run time (stream-ordered like A and B), must
 * be 4-byte aligned, and are owned by the caller.  Other arguments, layouts
 * and checks as gemm_fp8; additionally a count other than those above ->
 * DGEMM_ERR_INVALID_DIM (checked with the dimensions), a NULL factor pointer
 * -> DGEMM_ERR_NULL_POINTER, a misaligned one -> DGEMM_ERR_MISALIGNED.
 */
int gemm_fp8_scaled(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                    const uint8_t* B, int64_t ldb, float* C, int64_t ldc,
                    const float* scale_a, int64_t n_scale_a, const float* scale_b, int64_t n_scale_b,
                    int layout, void* stream);

/*
 * MXFP8: OCP E4M3 x E4M3 -> FP32 with one E8M0 scale per 32 consecutive k of
 * each row of A and of each column of B (the block scales of the OCP
 * Microscaling (MX) format, fed to the scale operands of the gfx950 MFMA;
 * the scaled successor that "FP8 GEMM Optimization on AMD RDNA 4", section
 * "What Changes at FP8", leaves for later work):
 *   C_ij = sum over blocks b of 2^(sa_ib - 127) * 2^(sb_jb - 127)
 *          * sum_{k = 32b}^{32b + 31} A_ik * B_kj
 * accumulated in FP32.  K must be a multiple of 32 (else
 * DGEMM_ERR_INVALID_DIM, checked with the dimensions).
 * scale_a: DEVICE pointer to M*ldsa bytes; sa_ib is scale_a[i*ldsa + b],
 *          ldsa >= K/32 (the kernels read whole 16-byte groups of a row).
 * scale_b: DEVICE pointer to N*ldsb bytes; sb_jb is scale_b[j*ldsb + b],
 *          ldsb >= K/32 (one row of scales per column j of B, in either
 *          layout).  With K == 0 neither is read (and may be NULL).
 * Both must be 16-byte aligned with ldsa, ldsb multiples of 16
 * (else DGEMM_ERR_MISALIGNED); an ld below K/32 -> DGEMM_ERR_INVALID_LD;
 * 256*ldsa or 256*ldsb at or above 2^31 -> DGEMM_ERR_UNSUPPORTED.  The scale
 * byte 255 (NaN in the format) is not supported: its result is unspecified.
 * Other arguments, layouts and checks as gemm_fp8.
 */
int gemm_mxfp8(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
               const uint8_t* B, int64_t ldb, float* C, int64_t ldc,
               const uint8_t* scale_a, int64_t ldsa, const uint8_t* scale_b, int64_t ldsb,
               int layout, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* gemm_strerror(int status);

/*
 * dgemm_last_hip_error: the hipError_t code behind the calling thread's most
 * recent DGEMM_ERR_HIP (0 if there was none); dgemm_hip_error_string: HIP's
 * static description of such a code.  For diagnostics only.
 */
int dgemm_last_hip_error(void);
const char* dgemm_hip_error_string(int code);

/*
 * Host-side introspection (no GPU work; used by host-only tests and reports).
 *
 * dgemm_tile_map: the block -> output-tile mapping the kernels use, for a grid
 * of tiles_p x tiles_q tiles, grouping `group` tiles along p ("FP16 GEMM
 * Optimization on AMD RDNA 3 and RDNA 4", section "Step 6: Block Scheduling
 * for Cache Reuse") after spreading consecutive tiles over the 8 XCDs.
 * Writes the tile coordinates of block `pid`; returns 0, or -1 for pid out of
 * range or non-positive sizes.
 *
 * dgemm_lds_bytes: LDS footprint (BM + BN) * (BK * elem + pad_bytes) * buffers
 * of a block tile, the sizing rule behind the LDS tables of "FP16 GEMM
 * Optimization on AMD RDNA 3 and RDNA 4" (Step 5, Table 9) and "FP8 GEMM
 * Optimization on AMD RDNA 4" (Configs 1-4).  Returns -1 for negative inputs.
 *
 * dgemm_kernel_config: writes a one-line description (kernel name, tile, wave
 * grid, LDS bytes, grid size) of the kernel a call with these arguments would
 * launch into buf (at most len bytes, NUL-terminated).  dtype: 0 f32, 1 f16,
 * 2 bf16, 3 fp8, 4 fp8 with scale factors, 5 MXFP8.  Returns 0, or a
 * dgemm_status for invalid arguments.
 */
/*
 * dgemm_trace_clock (diagnostics, used to report the engine clock the GEMM
 * itself ran at): while `buf` is set, every launch of the four-wave kernels
 * made by later calls from the calling thread records, for each workgroup
 * w < n_workgroups, four 64-bit values at buf[4w .. 4w + 3]: the core clock
 * counter and the 100 MHz real-time counter when the workgroup started, and
 * both again when it finished.  Engine clock in Hz over the workgroup =
 * (buf[4w+2] - buf[4w]) / (buf[4w+3] - buf[4w+1]) * 1e8 (the counters of
 * different XCDs have different origins: compare stamps of one workgroup
 * only).  `buf` is a DEVICE pointer to 4*n_workgroups values owned by the
 * caller, written asynchronously on the call's stream; later launches
 * overwrite it.  NULL turns the trace off.  Only the main launch of a call
 * is traced (not the second launch of a split call); other kernels (FP32,
 * skinny, ragged K) ignore it.  Returns DGEMM_ERR_INVALID_DIM for n_workgroups < 0.
 */
int dgemm_trace_clock(unsigned long long* buf, int64_t n_workgroups);

int dgemm_tile_map(int64_t tiles_p, int64_t tiles_q, int64_t group, int64_t pid,
                   int64_t* tile_p, int64_t* tile_q);
int64_t dgemm_lds_bytes(int bm, int bn, int bk, int elem, int pad_bytes, int buffers);
int dgemm_kernel_config(int dtype, int layout, int64_t M, int64_t N, int64_t K, char* buf, int64_t len);

#ifdef __cplusplus
}
#endif

#endif /* DGEMM_H */
