// Skinny TN GEMM (at most 32 rows of A), 16-bit operands, gfx950.
//
// With M = 16 the product is a matrix-vector-like stream: every element of B
// is used by only M rows of A, so time goes into reading B once from HBM
// ("FP16 GEMM Optimization on AMD RDNA 3 and RDNA 4", Where That Leaves Us:
// a skinny GEMM is the wrong shape for the large-tile kernel).  The large-tile
// kernel would launch N/256 workgroups -- 32 at N = 8192 -- far too few to
// pull HBM bandwidth.  This kernel instead:
//  * gives each workgroup 32 rows of B (N/32 workgroups, one per CU at
//    N = 8192) and splits K over its 8 waves, which run independently (no
//    barrier until the final reduction);
//  * loads B straight from global memory into MFMA operand registers, 256
//    bytes of each of the 32 rows per step (four 16 x 64-byte loads per
//    16-row tile, whole 128-byte lines), one step per wave in flight;
//  * loads A in 4-row x 256-byte pieces (whole lines, one row per 16
//    lanes) and turns them into MFMA operand layout through a private LDS
//    area of the wave (XOR-swizzled by row, so both the writes and the
//    fragment reads are free of bank conflicts); every A fragment serves
//    both 16-row tiles of B;
//  * multiplies with v_mfma_f32_16x16x32_{f16,bf16}: 16 rows of A per MFMA,
//    which is exactly the skinny extent (the matrix pipe is far from busy);
//  * reduces the 8 waves' partial sums through LDS, in wave order, and
//    stores four consecutive elements of a column of C at once with the
//    round-to-nearest-even convert.
// Rows of A past M and rows of B past N read zero through their offsets
// (pushed past num_records); k past K likewise, and a 16-byte chunk
// straddling K is masked in registers.
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
  static constexpr int QF = BQ / 16;            // 16-row tiles of B
  static constexpr int PR = 16 * PF;            // rows of A
  static constexpr int E = Op::ELEM;
  static constexpr int CPE = 16 / E;            // elements per 16-byte chunk
  static constexpr int KS = 32;                 // k per MFMA
  static constexpr int NI = 4;                  // MFMA k-steps per step
  static constexpr int STEPB = NI * KS * E;     // bytes of a row per step
  static constexpr int ALPR = STEPB / 16;       // lanes per row of an A load
  static constexpr int ARPL = 64 / ALPR;        // rows per A load
  static constexpr int ALD = PR / ARPL;         // A loads per step
  // Steps of loads in flight per wave.  Measured at 16 x 8192 x 8192 BF16
  // (one launch, B read from HBM): 1 step 28.8 us, 2 steps 31.6 us, 3 steps
  // 33.4 us; 512 bytes of a row per step (NI = 8) with 2 steps 36.8 us.
  // Beyond about 100 KiB in flight per CU the stream slows down.
  static constexpr int DEPTH = 1;
  static constexpr int LPS = QF * NI + ALD;     // loads per step
  static constexpr int ASCR = PR * STEPB;       // LDS bytes of a wave's A step
  static constexpr int LDS = NW * ASCR > NW * PF * QF * 64 * 16 ? NW * ASCR : NW * PF * QF * 64 * 16;
  static_assert(Op::ELEM == 2, "16-bit operands");
  static_assert(PF == 1 || PF == 2, "up to 32 rows of A");
  static_assert(ALPR <= 64 && 64 % ALPR == 0 && PR % ARPL == 0, "whole rows per A load");
  static_assert(STEPB / 16 >= 16, "the row swizzle permutes 16 chunks");
  static_assert(DEPTH >= 1 && (DEPTH - 1) * LPS <= 63, "vmcnt range");
};

template <class Op, int PF>
__device__ __forceinline__ void gemm_skinny_body(const GemmArgs& a) {
  using Cfg = SkinnyCfg<Op, PF>;
  constexpr int NW = Cfg::NW, BQ = Cfg::BQ, QF = Cfg::QF, KS = Cfg::KS, DEPTH = Cfg::DEPTH, E = Cfg::E;
  constexpr int NI = Cfg::NI, ALD = Cfg::ALD, LPS = Cfg::LPS, STEPB = Cfg::STEPB, CPE = Cfg::CPE;

  __shared__ __attribute__((aligned(1024))) char smem[Cfg::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t q0 = (int64_t)blockIdx.x * BQ;
  const int64_t K = a.K;
  const uint32_t kbytes16 = (uint32_t)(((K * E) + 15) & ~(int64_t)15);

  // Descriptors over the workgroup's 32 rows of B and all (<= 32) rows of A.
  const int64_t qrows = (a.Qn - q0) < BQ ? (a.Qn - q0) : BQ;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.Q + q0 * a.ldq, (uint32_t)((qrows - 1) * a.ldq) + kbytes16);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.P, (uint32_t)((a.Pn - 1) * a.ldp) + kbytes16);

  // B, MFMA 16x16x32 operand layout: lane l holds row (l % 16) of its tile
  // and chunk l / 16 of a 32-k step (8 k, the same k-set as A's fragment).
  // Load i of a step covers k-step i: 64 bytes of each of 16 rows.
  const int r16 = lane & 15, kg = lane >> 4;
  uint32_t qoff[QF];
#pragma unroll
  for (int j = 0; j < QF; ++j) qoff[j] = (16 * j + r16) < qrows ? (uint32_t)((16 * j + r16) * a.ldq + kg * 16) : kOobOffset;
  // A, load i of a step: rows 4 i + l / 16, 16-byte chunk l % 16 of the
  // step's 256 bytes.
  constexpr int ALPR = Cfg::ALPR, ARPL = Cfg::ARPL;
  const int arow = lane / ALPR, ach = lane % ALPR;
  uint32_t poff[ALD];
#pragma unroll
  for (int i = 0; i < ALD; ++i)
    poff[i] = (ARPL * i + arow) < a.Pn ? (uint32_t)((ARPL * i + arow) * a.ldp + ach * 16) : kOobOffset;

  // This wave's steps (128 k each).
  const int nks = (int)((K + NI * KS - 1) / (NI * KS));
  const int t0 = (int)((int64_t)wave * nks / NW), t1 = (int)((int64_t)(wave + 1) * nks / NW);
  const int nt = t1 - t0;

  u32x4 qb[DEPTH][QF][NI], pa[DEPTH][ALD];
  // Step t of this wave (any t >= 0): loads for t >= nt or k >= K are pushed
  // out of range and read zero, so the loop below needs no bounds branches
  // (a branch would make every wait drain all loads in flight).
  auto issue = [&](int t, int slot) {
    const int64_t kb = (int64_t)(t0 + t) * (NI * KS);           // first k of the step
    const uint32_t boff = (uint32_t)(t0 + t) * STEPB;
    const bool dead = t >= nt;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t kill = (dead || kb + KS * i + kg * CPE >= K) ? kOobOffset : 0u;
#pragma unroll
      for (int j = 0; j < QF; ++j) qb[slot][j][i] = load16(rq, (qoff[j] + boff + i * (KS * E)) | kill);
    }
    const uint32_t akill = (dead || kb + ach * CPE >= K) ? kOobOffset : 0u;
#pragma unroll
    for (int i = 0; i < ALD; ++i) pa[slot][i] = load16(rp, (poff[i] + boff) | akill);
  };

  // The wave's A area: PR rows of 256 bytes, chunk c of row r at physical
  // chunk c ^ (r % 16).
  char* ascr = smem + wave * Cfg::ASCR;
  f32x4v acc[PF][QF];
#pragma unroll
  for (int i = 0; i < PF; ++i)
#pragma unroll
    for (int j = 0; j < QF; ++j) acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};
  auto consume = [&](int t, int slot) {
#pragma unroll
    for (int i = 0; i < ALD; ++i) {
      const int r = ARPL * i + arow;
      *(u32x4*)(ascr + r * STEPB + ((ach ^ (r & 15)) << 4)) = pa[slot][i];
    }
    const int64_t kb = (int64_t)(t0 + t) * (NI * KS);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      // Keep only the bytes below K: all 16 for a full chunk, none past K,
      // the leading ones for a chunk that straddles K.
      const int64_t rem = K - (kb + KS * i + kg * CPE);
      const int vb = rem >= CPE ? 16 : (rem <= 0 ? 0 : (int)rem * E);
      const int c = (KS / CPE) * i + kg;
      u32x4 af[PF];
#pragma unroll
      for (int f = 0; f < PF; ++f) {
        const int r = 16 * f + r16;
        af[f] = mask_tail(*(const u32x4*)(ascr + r * STEPB + ((c ^ (r & 15)) << 4)), vb);
      }
#pragma unroll
      for (int j = 0; j < QF; ++j) {
        const u32x4 b = mask_tail(qb[slot][j][i], vb);
#pragma unroll
        for (int f = 0; f < PF; ++f) acc[f][j] = Mma16<Op>::mma(af[f], b, acc[f][j]);
      }
    }
  };

  // Register ring of DEPTH steps: step t lives in slot t % DEPTH.  Every
  // iteration issues one step, so exactly DEPTH - 1 later steps are in flight
  // when a step is consumed (loads complete in issue order).
#pragma unroll
  for (int u = 0; u < DEPTH; ++u) {
    issue(u, u);
    __builtin_amdgcn_sched_barrier(0);   // slots in issue order
  }
  for (int t = 0; t < nt; t += DEPTH) {
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      __builtin_amdgcn_s_waitcnt(kWaitVmcntBase | vmcnt_bits((DEPTH - 1) * LPS));
      consume(t + u, u);
      // (Kept after the step's MFMAs: hoisted above them, the loads into
      // this slot would force its values to be copied first.)
      __builtin_amdgcn_sched_barrier(0);
      issue(t + u + DEPTH, u);
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();

  // Cross-wave reduction.  16x16 accumulator layout: lane l holds column
  // (l % 16) and rows 4*(l/16) .. 4*(l/16)+3, four consecutive elements of
  // a column of C.  Thread (t, l) sums lane l of tile t over the waves, in
  // wave order, and stores those four elements.
  f32x4v* red = (f32x4v*)smem;   // [NW][PF * QF][64]
#pragma unroll
  for (int i = 0; i < PF; ++i)
#pragma unroll
    for (int j = 0; j < QF; ++j) red[(wave * PF * QF + i * QF + j) * 64 + lane] = acc[i][j];
  __syncthreads();
  if (tid < PF * QF * 64) {
    const int t = tid >> 6;
    const int64_t p = 16 * (t / QF) + 4 * kg, q = q0 + 16 * (t % QF) + r16;
    f32x4v s = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) s += red[(w * PF * QF + t) * 64 + lane];
    if (q < a.Qn) store4<Op>(a, q, p, s[0], s[1], s[2], s[3]);
  }
}

template <class Op, int PF>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_skinny_kernel(const GemmArgs a) {
  gemm_skinny_body<Op, PF>(a);
}

}  // namespace dg
