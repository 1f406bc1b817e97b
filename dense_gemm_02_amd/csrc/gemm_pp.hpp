// Eight-wave "ping-pong" GEMM for 16-bit and 8-bit K-contiguous operands
// (TN) on gfx950: two waves on every SIMD, in two groups of four, take
// turns.  While one group issues nothing but MFMAs, the other reads its
// fragments for its next turn from LDS and (group 0) issues the global ->
// LDS copies; at each workgroup barrier the roles swap.  A SIMD's MFMA pipe
// therefore never waits for a fragment read, a copy issue or a wave that is
// late to a barrier while the other wave has work ("An Educational GEMM
// Ladder for Helios GPUs", Level 12, two waves per SIMD; its summary names
// the eight-wave ping-pong as the MI355X schedule).
//
// Operation and (P, Q, D) mapping as gemm_mfma.hpp: D[p][q] = sum_k P(p,k)
// Q(q,k), stored at C[q*ldc + p].  Block tile 256 x 256; SIMD s owns the
// 128 x 128 quadrant (p half s / 2, q half s % 2) and its two waves split
// it along q: the wave of group g computes 128 (p) x 64 (q) as 8 x 4 MFMA
// tiles of 16 x 16 (x 32 for FP16/BF16, x 128 for FP8) with 128
// accumulator registers, which leaves 128 for the fragments of one whole
// stage (96) and addressing at two waves per SIMD.
//
// LDS: 128 bytes of k per row per stage, XOR-swizzled as in the four-wave
// kernel; two slots for the P rows of a stage (256 x 128 B, 32 KiB each) and
// three for the Q rows (32 KiB each): 160 KiB.  Copies are direct global ->
// LDS through buffer descriptors (rows past the edge and k past K read zero).
//
// Per stage t each wave runs R(t) (read its fragments of stage t), a
// barrier, C(t) (all MFMAs of the stage), a wait for its own copies, a
// barrier; group 1 runs one barrier behind group 0, so that one group's C
// overlaps the other's R.  Ahead of its R(t), group 0 copies the P rows of
// stage t + 1 and group 1 the Q rows of stage t + 2, each into the slot that
// both groups finished reading a barrier earlier; each copy has two turns
// (its issuer's R and C) to land before the barrier that publishes it, and
// every turn carries half a stage of copies (32 KiB), which keeps the copy
// path at about half of what it delivers per CU.  The barriers wait only for
// LDS reads, so copies stay in flight across them.
#pragma once

#include "common.hpp"
#include "gemm_mfma.hpp"

namespace dg {

template <class Op>
struct PpCfg {
  static constexpr int BP = 256, BQ = 256;
  static constexpr int NW = 8, NT = 512, NSIMD = 4;
  static constexpr int E = Op::ELEM, FC = Op::FC;
  static constexpr int ROWB = 128;                 // bytes of k per LDS row per stage
  static constexpr int BK = ROWB / E;              // k per stage
  static constexpr int CPE = 16 / E;               // elements per 16-byte chunk
  static constexpr int P_LDS = BP * ROWB;          // one P slot
  static constexpr int Q_LDS = BQ * ROWB;          // one Q slot
  static constexpr int Q_BASE = 2 * P_LDS;         // Q slots after the two P slots
  static constexpr int LDS = 2 * P_LDS + 3 * Q_LDS;
  static constexpr int QSEG = BQ / 8 / NSIMD;      // copies per wave per stage of its operand
  static constexpr int PSEG = BP / 8 / NSIMD;
  static constexpr int WTP = BP / 2, WTQ = BQ / 4; // wave tile
  static constexpr int MT = 16;
  static constexpr int KI = E == 2 ? 32 : 128;     // k per MFMA
  static constexpr int TP = WTP / MT, TQ = WTQ / MT;
  static constexpr int KSTEPS = BK / KI;
  static constexpr int CPK = KI * E / 16;          // 16-byte chunks of k per k-step
  static_assert(LDS <= kLdsLimit, "LDS budget");
  static_assert((TP / (Op::OE == 4 ? 2 : 1)) * MT * Op::OE == 256, "staged epilogue rows of 256 bytes");
  static_assert(WTQ * 256 * NW <= LDS, "epilogue staging fits the stage buffers");
};

// KT: K ends inside a stage, so the copies carry per-lane tail masks.
template <class Op, bool KT>
__device__ __forceinline__ void gemm_pp_body(const GemmArgs& a) {
  using Cfg = PpCfg<Op>;
  constexpr int E = Cfg::E, FC = Cfg::FC, ROWB = Cfg::ROWB, BK = Cfg::BK, CPE = Cfg::CPE;
  constexpr int TP = Cfg::TP, TQ = Cfg::TQ, MT = Cfg::MT, CPK = Cfg::CPK, KSTEPS = Cfg::KSTEPS;

  __shared__ __attribute__((aligned(1024))) char smem[Cfg::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, simd = wave & 3;
  const int wp = simd >> 1, wq = simd & 1;
  const int64_t K = a.K;
  const int nst = (int)((K + BK - 1) / BK);
  const uint32_t kbytes16 = (uint32_t)(((K * E) + 15) & ~(int64_t)15);
  const int64_t ntiles = a.tiles_p * a.tiles_q;
  const int64_t tile = blockIdx.x;
  if (tile >= ntiles) return;   // (the whole workgroup)

  auto stamp = [&](int at) {
    if (a.trace != nullptr && tid == 0 && tile < a.trace_n) {
      unsigned long long* t = a.trace + 4 * tile + at;
      t[0] = __builtin_amdgcn_s_memtime();
      t[1] = __builtin_amdgcn_s_memrealtime();
    }
  };
  stamp(0);

  int64_t tp, tq;
  tile_map(a.tiles_p, a.tiles_q, a.group, tile, &tp, &tq);
  const int64_t p0 = tp * Cfg::BP, q0 = tq * Cfg::BQ;
  const int64_t qrows = (a.Qn - q0) < Cfg::BQ ? (a.Qn - q0) : Cfg::BQ;
  const int64_t prows = (a.Pn - p0) < Cfg::BP ? (a.Pn - p0) : Cfg::BP;
  const char* qsrc = a.Q + q0 * a.ldq;
  const char* psrc = a.P + p0 * a.ldp;
  const uint32_t qn = (uint32_t)((qrows - 1) * a.ldq) + kbytes16;
  const uint32_t pn = (uint32_t)((prows - 1) * a.ldp) + kbytes16;

  // ---- copies: P rows by group 0, Q rows by group 1 ----
  // One copy instruction fills one 1 KiB LDS segment = 8 rows of 128 bytes;
  // the wave on SIMD s fills segments 4i + s of its operand's slot.  Lane l
  // lands at byte 16 l: row 8 (4i + s) + l / 8, physical chunk l % 8, which
  // holds logical chunk (l % 8) ^ key(row), key(row) = (row / 2) mod 8 =
  // (4 (s % 2) + l / 16) mod 8.  Rows past the edge need no test: their
  // offsets are at least rows * ld >= num_records.
  const int dkc = (lane & 7) ^ ((4 * (simd & 1) + (lane >> 4)) & 7);
  const char* csrc = grp == 0 ? psrc : qsrc;
  const uint32_t cn = grp == 0 ? pn : qn;
  const int64_t cld = grp == 0 ? a.ldp : a.ldq;
  const uint32_t cv0 = (uint32_t)((8 * simd + (lane >> 3)) * cld + dkc * 16);
  const uint32_t cstep = (uint32_t)(32 * cld);
  auto p_slot = [&](int t) { return smem + (t & 1) * Cfg::P_LDS; };
  auto q_slot = [&](int t) { return smem + Cfg::Q_BASE + (t % 3) * Cfg::Q_LDS; };
  // Stage t of this wave's operand into its slot.
  auto copies = [&](int t) {
    char* sb = grp == 0 ? p_slot(t) : q_slot(t);
    const uint32_t at = (uint32_t)t * ROWB;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(csrc + at, cn - at);
    uint32_t kill = 0;
    if constexpr (KT) {
      // Chunks at or past K read zero (bit 31 puts the offset past num_records).
      const int64_t rem64 = K - (int64_t)t * BK;
      const int rem = (int)(rem64 < BK ? rem64 : BK);
      kill = dkc * CPE >= rem ? kOobOffset : 0u;
    }
    static_assert(Cfg::PSEG == Cfg::QSEG, "both operands take the same number of copies");
#pragma unroll
    for (int i = 0; i < Cfg::PSEG; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(sb + (i * Cfg::NSIMD + simd) * 1024), 16,
          (cv0 + i * cstep) | kill, 0, 0, 0);
  };

  // ---- fragments ----
  // Lane l holds row l % 16 of its P and Q tiles; lane group l / 16 selects
  // its k: 16-bit, chunk 4 kk + l / 16 of the stage row (8 k); FP8, chunks
  // l / 16 and l / 16 + 4 (16 k each), which keeps the order of the
  // four-wave kernel's FP8 fragments.
  const int lr = lane & 15, lg = lane >> 4;
  const int sw = (lr >> 1) & 7;
  const uint32_t pf = (uint32_t)((wp * Cfg::WTP + lr) * ROWB);
  const uint32_t qf = (uint32_t)((wq * (Cfg::BQ / 2) + grp * Cfg::WTQ + lr) * ROWB);
  u32x4 fa[KSTEPS][TP][FC], fb[KSTEPS][TQ][FC];
  auto read_frags = [&](int t) {
    const char* sp = p_slot(t);
    const char* sq = q_slot(t);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
      for (int f = 0; f < FC; ++f) {
        const uint32_t off = (uint32_t)(((kk * CPK + f * (CPK / FC) + lg) ^ sw) << 4);
#pragma unroll
        for (int j = 0; j < TQ; ++j) fb[kk][j][f] = *(const u32x4*)(sq + qf + j * MT * ROWB + off);
#pragma unroll
        for (int i = 0; i < TP; ++i) fa[kk][i][f] = *(const u32x4*)(sp + pf + i * MT * ROWB + off);
      }
  };

  f32x4 acc[TP][TQ];
#pragma unroll
  for (int i = 0; i < TP; ++i)
#pragma unroll
    for (int j = 0; j < TQ; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&]() {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
      for (int j = 0; j < TQ; ++j)
#pragma unroll
        for (int i = 0; i < TP; ++i) acc[i][j] = Op::mma16(fa[kk][i], fb[kk][j], acc[i][j]);
  };
  // Workgroup barrier after this wave's LDS reads have returned; global ->
  // LDS copies stay in flight across it (a fence on LDS would also wait for
  // them, as they write LDS).  Written as assembly with a memory clobber so
  // that the compiler moves no memory access across it; copies become
  // visible through the explicit vmcnt waits of the waves that issued them,
  // each followed by one of these barriers.
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // Prologue: P of stage 0 (group 0), Q of stages 0 and 1 (group 1), all
  // landed before the first barrier; group 1 then runs one barrier behind.
  // Every wave passes 2 nst + 2 barriers in all.
  if (nst > 0) copies(0);
  if (grp == 1 && nst > 1) copies(1);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  barrier();
  if (grp == 1) barrier();
  const int ahead = grp == 0 ? 1 : 2;   // stages ahead this group copies
  for (int t = 0; t < nst; ++t) {
    if (t + ahead < nst) copies(t + ahead);
    read_frags(t);
    barrier();
    compute();
    // This wave's copies have landed before the next barrier publishes
    // them.  (Fenced off from the MFMAs, so that the compiler cannot move
    // the wait ahead of them.)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    barrier();
  }
  if (grp == 0) barrier();

  // Epilogue: every wave is past its last LDS read; each stages its own
  // 64 rows of C (64 x 256 bytes) through LDS.
  staged_epilogue<Op, Cfg::WTP, Cfg::WTQ, TP, TQ, MT, f32x4>(
      a, smem + wave * (Cfg::WTQ * 256), acc, lane, p0 + wp * Cfg::WTP,
      q0 + wq * (Cfg::BQ / 2) + grp * Cfg::WTQ);
  stamp(2);
}

template <class Op, bool KT>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_pp_kernel(const GemmArgs a) {
  gemm_pp_body<Op, KT>(a);
}

}  // namespace dg
