// Shared device/host pieces of the gfx950 GEMM kernels: vector types, buffer
// resource descriptors, the block -> tile scheduler and LDS sizing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Number of XCDs on MI355X; workgroups are dispatched round-robin over them.
constexpr int kXcds = 8;

// Offset used to force a buffer load out of range.  Every descriptor built by
// these kernels has num_records < 2^31, so this offset always reads zero.
constexpr uint32_t kOobOffset = 0x80000000u;

// s_waitcnt immediate that waits for vmcnt == 0 only (gfx9 encoding: vmcnt
// bits [3:0] and [15:14] zero, expcnt [6:4] and lgkmcnt [11:8] at their
// maxima).  Direct global -> LDS copies are counted by vmcnt.
constexpr int kWaitVmcnt0 = 0x0F70;
// ... and for lgkmcnt == 0 only (vmcnt 63, expcnt 7).
constexpr int kWaitLgkmcnt0 = 0xC07F;
// vmcnt <= n: kWaitVmcntBase | vmcnt_bits(n), n in [0, 63].
constexpr int kWaitVmcntBase = 0x0F70;
constexpr int vmcnt_bits(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14); }

// Raw (untyped, stride 0) buffer descriptor, word 3 of the gfx9-family
// encoding (data format 32-bit; the RDNA word printed on the pages does not
// apply to CDNA).  Loads at offsets >= num_records return zero instead of
// faulting ("FP16 GEMM Optimization on AMD RDNA 3 and RDNA 4", section
// "Step 4: Buffer Resource Descriptors for Global Loads").
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_records) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_records, kBufferWord3);
}

// The same descriptor as four dwords (gfx9 layout: base, base[47:32] with
// stride 0, num_records, word 3), for inline assembly.
__device__ __forceinline__ i32x4 make_desc(const void* base, uint32_t num_records) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return i32x4{(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xffffu), (int)num_records, kBufferWord3};
}

// Direct global -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ...
// lds) written as inline assembly.  The compiler does not see it as an LDS
// write, so it adds no waits of its own for it: the caller waits (vmcnt)
// before anything reads the destination, as the kernels here do before
// every barrier that publishes a stage.  (Issued through the builtin, the
// copy makes the compiler drain all copies in flight before every
// transposing LDS read, which it cannot prove independent of them.)
// M0 holds the LDS destination; one wait state separates its write from the
// load that consumes it.
__device__ __forceinline__ void copy16_lds(i32x4 desc, uint32_t voff, const void* lds_dst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_dst;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(desc), "s"(m0)
               : "memory", "m0");
}

// The same with 4 bytes per lane (buffer_load_dword ... lds): lane l lands
// at M0 + 4*l.
__device__ __forceinline__ void copy4_lds(i32x4 desc, uint32_t voff, const void* lds_dst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_dst;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(desc), "s"(m0)
               : "memory", "m0");
}

// This lane's index in its wave, computed afresh (mbcnt) rather than taken
// from threadIdx: code after a long loop that uses it then keeps no thread
// index register live across the loop.
__device__ __forceinline__ int lane_id() {
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
}

// ---- block -> tile scheduler -------------------------------------------------
// 1. XCD spread: block `pid` runs on XCD pid % 8.  Renumber blocks so that
//    each XCD receives a contiguous range of logical tile ids; neighbouring
//    tiles then share that XCD's private L2.  Ranges differ in length by at
//    most one when the block count is not a multiple of 8, keeping the map a
//    bijection.
// 2. Grouping ("FP16 GEMM Optimization on AMD RDNA 3 and RDNA 4", Step 6):
//    logical ids walk `group` tiles along p, then step along q, so blocks in
//    flight at the same time reuse the same operand panels; the last group
//    may be shorter.
__host__ __device__ inline void tile_map(int64_t tiles_p, int64_t tiles_q, int64_t group, int64_t pid,
                                         int64_t* tp, int64_t* tq) {
  const int64_t total = tiles_p * tiles_q;
  const int64_t per = total / kXcds, extra = total % kXcds;
  const int64_t xcd = pid % kXcds, local = pid / kXcds;
  const int64_t lid = (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + local;
  const int64_t width = group * tiles_q;
  const int64_t g = lid / width;
  const int64_t first = g * group;
  const int64_t rest = tiles_p - first;
  const int64_t gsz = rest < group ? rest : group;
  const int64_t in = lid - g * width;
  *tp = first + in % gsz;
  *tq = in / gsz;
}

// LDS bytes of a block tile: (BM + BN) rows of BK*elem bytes plus a per-row pad,
// times the number of buffers.
__host__ __device__ constexpr int64_t lds_bytes(int bm, int bn, int bk, int elem, int pad, int bufs) {
  return (int64_t)(bm + bn) * (int64_t)(bk * elem + pad) * (int64_t)bufs;
}

constexpr int64_t kLdsLimit = 163840;  // 160 KiB per workgroup on gfx950

// Kernel arguments shared by every GEMM kernel.  The kernels compute
// D[p][q] = sum_k P(p,k) * Q(q,k) and store D[p][q] at C[q*ldc + p]:
//   TN: P = A (p = i), Q = B (q = j), C column-major  -> C[j*ldc + i]
//   NN: P = B^T (p = j), Q = A (q = i), C row-major   -> C[i*ldc + j]
// so p is always the contiguous direction of C.
struct GemmArgs {
  const char* P;     // operand P base
  const char* Q;     // operand Q base
  void* C;
  int64_t ldp;       // bytes between consecutive rows of P's storage
  int64_t ldq;       // bytes between consecutive rows of Q's storage
  int64_t ldc;       // elements between consecutive q of C
  int64_t Pn, Qn, K; // extents of p, q and k
  int64_t tiles_p, tiles_q, group;
  int vec_store;     // C and ldc allow 4-element vector stores
  int vec16;         // C and ldc allow 16-byte stores
  // Scale factors (FP8 scaled entry point only): D[p][q] is multiplied by
  // sp[p] * sq[q] (sp_row / sq_row = 1) or by sp[0] / sq[0] (= 0).
  const float* sp;
  const float* sq;
  int sp_row, sq_row;
  // E8M0 block scales (MXFP8 entry point only): row p of P has K/32 scale
  // bytes at msp + p*ldsp, row q of Q at msq + q*ldsq.
  const uint8_t* msp;
  const uint8_t* msq;
  int64_t ldsp, ldsq;
  // Clock trace (diagnostics, four-wave kernels only): workgroup w <
  // trace_n writes its start and end stamps of the core clock counter and
  // of the 100 MHz real-time counter to trace[4w .. 4w + 3].
  unsigned long long* trace;
  int64_t trace_n;
};

}  // namespace dg
