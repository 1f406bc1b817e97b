// Skinny TN GEMM (at most 32 rows of A), 16-bit operands, gfx950.
//
// With M = 16 the product is a matrix-vector-like stream: every element of B
// is used by only M rows of A, so time goes into reading B once from HBM
// ("FP16 GEMM Optimization on AMD RDNA 3 and RDNA 4", Where That Leaves Us:
// a skinny GEMM is the wrong shape for the large-tile kernel).  The large-tile
// kernel would launch N/256 workgroups -- 32 at N = 8192 -- far too few to
// pull HBM bandwidth.  This kernel instead:
//  * gives each workgroup 32 rows of B (so N/32 workgroups, one per CU at
//    N = 8192) and splits K over its 8 waves;
//  * loads B and A straight from global memory into MFMA operand registers
//    (no LDS staging), keeping DEPTH k-steps of loads in flight per wave so
//    enough bytes are outstanding to cover HBM latency;
//  * multiplies with v_mfma_f32_16x16x32_{f16,bf16}: 16 rows of A per MFMA,
//    which is exactly the skinny extent (the matrix pipe is far from busy);
//  * reduces the 8 waves' partial sums through LDS, parked in register
//    layout, and stores four consecutive elements of a column of C at once
//    with the round-to-nearest-even convert.
// Rows of A past M and rows of B past N read zero through the buffer
// descriptors' num_records; k past K is pushed out of range, and a 16-byte
// chunk straddling K is masked in registers.
#pragma once

#include "common.hpp"
#include "gemm_mfma.hpp"

namespace dg {

typedef float f32x4v __attribute__((ext_vector_type(4)));

template <class Op> struct Mma16;
template <> struct Mma16<OpF16> {
  __device__ static f32x4v mma(u32x4 a, u32x4 b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
};
template <> struct Mma16<OpBF16> {
  __device__ static f32x4v mma(u32x4 a, u32x4 b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
};

template <class Op, int PF>
struct SkinnyCfg {
  static constexpr int NW = 8;                  // waves, each owning a slice of K
  static constexpr int NT = NW * 64;
  static constexpr int BQ = 32;                 // rows of B (columns of C) per workgroup
  static constexpr int QF = BQ / 16;            // 16-wide MFMA tiles along q
  static constexpr int KS = 32;                 // k per MFMA (16x16x32)
  // k-steps of loads in flight per wave.  Measured at 16 x 8192 x 8192: 8
  // steps 36.5 us, 12 steps 38.0, 16 steps 40.0 (more bytes in flight push
  // A, which every workgroup re-reads, out of the L2).
  static constexpr int DEPTH = 8;
  static constexpr int LPS = QF + PF;           // loads per k-step
  static constexpr int E = Op::ELEM;
  static_assert(Op::ELEM == 2, "16-bit operands");
  static_assert(PF == 1 || PF == 2, "up to 32 rows of A");
  static_assert((DEPTH - 1) * LPS <= 63, "vmcnt range");
};

template <class Op, int PF>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_skinny_kernel(const GemmArgs a) {
  using Cfg = SkinnyCfg<Op, PF>;
  constexpr int NW = Cfg::NW, BQ = Cfg::BQ, QF = Cfg::QF, KS = Cfg::KS, DEPTH = Cfg::DEPTH, E = Cfg::E;
  constexpr int LPS = Cfg::LPS, CPE = 16 / E;

  // Partial sums of every wave, tile and lane: one 16-byte slot per lane,
  // so each wave's writes and each summing thread's reads are contiguous.
  __shared__ f32x4v red[NW][PF * QF][64];
  static_assert(BQ % 16 == 0, "whole 16-wide q tiles");
  static_assert(PF * QF * 64 <= NW * 64, "one summing thread per tile lane");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int64_t q0 = (int64_t)blockIdx.x * BQ;
  const int64_t K = a.K;
  const uint32_t kbytes16 = (uint32_t)(((K * E) + 15) & ~(int64_t)15);

  // Descriptors over the workgroup's 32 rows of B and all (<= 32) rows of A.
  const int64_t qrows = (a.Qn - q0) < BQ ? (a.Qn - q0) : BQ;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.Q + q0 * a.ldq, (uint32_t)((qrows - 1) * a.ldq) + kbytes16);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.P, (uint32_t)((a.Pn - 1) * a.ldp) + kbytes16);

  // MFMA 16x16x32 operand layout: lane l holds row (l % 16) and k elements
  // 8*(l/16) .. 8*(l/16)+7 of the k-step (the same k-set for both operands).
  const int r16 = lane & 15, kg = lane >> 4;
  uint32_t qoff[QF], poff[PF];
#pragma unroll
  for (int j = 0; j < QF; ++j) qoff[j] = (uint32_t)((16 * j + r16) * a.ldq + kg * 16);
#pragma unroll
  for (int i = 0; i < PF; ++i) poff[i] = (uint32_t)((16 * i + r16) * a.ldp + kg * 16);

  // This wave's k-steps.
  const int nks = (int)((K + KS - 1) / KS);
  const int t0 = (int)((int64_t)wave_u * nks / NW), t1 = (int)((int64_t)(wave_u + 1) * nks / NW);
  const int nt = t1 - t0;

  u32x4 qb[DEPTH][QF], pb[DEPTH][PF];
  // Step t of this wave (any t >= 0): loads for t >= nt or k >= K are pushed
  // out of range and read zero, so the loop below needs no bounds branches
  // (a branch would make every wait drain all loads in flight).
  auto issue = [&](int t, int slot) {
    const int64_t k = (int64_t)(t0 + t) * KS + kg * CPE;        // first k of this lane's chunk
    const uint32_t kill = (t >= nt || k >= K) ? kOobOffset : 0u;
    const uint32_t koff = (uint32_t)((t0 + t) * KS * E);
#pragma unroll
    for (int j = 0; j < QF; ++j) qb[slot][j] = load16(rq, (qoff[j] + koff) | kill);
#pragma unroll
    for (int i = 0; i < PF; ++i) pb[slot][i] = load16(rp, (poff[i] + koff) | kill);
  };
  f32x4v acc[PF][QF];
#pragma unroll
  for (int i = 0; i < PF; ++i)
#pragma unroll
    for (int j = 0; j < QF; ++j) acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};
  auto consume = [&](int t, int slot) {
    // Keep only the bytes below K: all 16 for a full chunk, none past K,
    // the leading ones for a chunk that straddles K (computed, not branched).
    const int64_t k = (int64_t)(t0 + t) * KS + kg * CPE;
    const int64_t rem = K - k;
    const int vb = rem >= CPE ? 16 : (rem <= 0 ? 0 : (int)rem * E);
#pragma unroll
    for (int j = 0; j < QF; ++j) qb[slot][j] = mask_tail(qb[slot][j], vb);
#pragma unroll
    for (int i = 0; i < PF; ++i) pb[slot][i] = mask_tail(pb[slot][i], vb);
#pragma unroll
    for (int i = 0; i < PF; ++i)
#pragma unroll
      for (int j = 0; j < QF; ++j) acc[i][j] = Mma16<Op>::mma(pb[slot][i], qb[slot][j], acc[i][j]);
  };

  // Register ring of DEPTH k-steps: step t lives in slot t % DEPTH.  Every
  // iteration issues one step, so exactly DEPTH - 1 later steps are in flight
  // when a step is consumed (loads complete in issue order).
#pragma unroll
  for (int u = 0; u < DEPTH; ++u) issue(u, u);
  for (int t = 0; t < nt; t += DEPTH) {
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      __builtin_amdgcn_s_waitcnt(kWaitVmcntBase | vmcnt_bits((DEPTH - 1) * LPS));
      consume(t + u, u);
      issue(t + u + DEPTH, u);
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // Cross-wave reduction.  16x16 accumulator layout: lane l holds column
  // (l % 16) and rows 4*(l/16) .. 4*(l/16)+3, four consecutive elements of
  // a column of C.  Thread (t, l) sums lane l of tile t over the waves, in
  // wave order, and stores those four elements.
#pragma unroll
  for (int i = 0; i < PF; ++i)
#pragma unroll
    for (int j = 0; j < QF; ++j) red[wave_u][i * QF + j][lane] = acc[i][j];
  __syncthreads();
  if (tid < PF * QF * 64) {
    const int t = tid >> 6;
    const int64_t p = 16 * (t / QF) + 4 * kg, q = q0 + 16 * (t % QF) + r16;
    f32x4v s = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) s += red[w][t][lane];
    if (q < a.Qn) store4<Op>(a, q, p, s[0], s[1], s[2], s[3]);
  }
}

}  // namespace dg
