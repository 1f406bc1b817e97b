// Tiled FP32 GEMM on gfx950 matrix cores (v_mfma_f32_32x32x2_f32).
//
// "Optimizing GEMM in HIP" builds its FP32 kernel out of scalar FMAs with LDS
// and register tiling; CDNA4 has FP32 matrix instructions, so the same
// block/LDS/double-buffer structure feeds MFMA instead.  D[p][q] = sum_k
// P(p,k) Q(q,k) with the GemmArgs mapping (p contiguous in C).
//
// One MFMA consumes two k per lane pair: lane l supplies P(p = l % 32, k) and
// Q(q = l % 32, k) for one k chosen by l / 32.  Which k goes with which lane
// half is free as long as P and Q agree, so each block of 8 k is split as
// k = 8b + 4h + t (h = lane half, t = 0..3, one MFMA per t).  A lane then
// needs 4 consecutive k of its row: one 16-byte LDS read from a K-contiguous
// tile, or 4 scalar reads from a p-contiguous tile.  That lets both operands
// stay in LDS in the layout they have in memory; no transpose anywhere.
//
// LDS layouts per stage (BK = 32):
//  * K-contiguous operand: 128-byte rows, 16-byte chunks XOR-swizzled with
//    key (row / 2) mod 8, as in the 16-bit kernel.
//  * p-contiguous operand (the NN B matrix as P): BK rows of BP floats, each
//    row padded by 32 bytes so that the two lane halves (k and k + 4) land
//    in opposite halves of the 64 banks.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace dg {

template <int BP, int BQ, int WP, int WQ, bool P_TRANS>
struct F32Cfg {
  static constexpr int NT = WP * WQ * 64;
  static constexpr int BK = 32;
  static constexpr int ROWB = 128;                          // K-contiguous row bytes
  static constexpr int PT_STRIDE = BP * 4 + 32;             // p-contiguous row bytes (padded)
  static constexpr int P_LDS = P_TRANS ? BK * PT_STRIDE : BP * ROWB;
  static constexpr int Q_LDS = BQ * ROWB;
  static constexpr int STAGE = P_LDS + Q_LDS;
  static constexpr int PT_CPR = BP / 4;                     // 16-byte chunks per p-contiguous row
  static constexpr int PCH = (P_TRANS ? BK * PT_CPR : BP * 8) / NT;
  static constexpr int QCH = BQ * 8 / NT;
  static constexpr int WTP = BP / WP, WTQ = BQ / WQ;
  static constexpr int TP = WTP / 32, TQ = WTQ / 32;
  static_assert((P_TRANS ? BK * PT_CPR : BP * 8) % NT == 0 && BQ * 8 % NT == 0, "chunks divide over threads");
  static_assert(NT % 8 == 0 && (NT / 8) % 16 == 0, "swizzle key is per-thread invariant");
  static_assert(WTP % 32 == 0 && WTQ % 32 == 0, "whole MFMA tiles");
  static_assert(2 * STAGE <= kLdsLimit, "LDS budget");
};

// Stage s of a K-contiguous FP32 tile: this thread's chunks all start at
// k = s*BK + kc*4; in the last stage chunks past K read zero and a chunk that
// straddles K keeps only its first K - k floats.
template <int N, int BK>
__device__ __forceinline__ void load_kcontig_f32(const char* blk, uint32_t nrec, const uint32_t (&vo)[N],
                                                 u32x4 (&dst)[N], int s, bool tail, int64_t K, int kc) {
  const uint32_t adv = (uint32_t)s * (BK * 4);
  const __amdgpu_buffer_rsrc_t r = make_rsrc(blk + adv, nrec - adv);
  const int64_t kst = (int64_t)s * BK + kc * 4;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    uint32_t off = vo[i];
    if (tail && kst >= K) off = kOobOffset;
    u32x4 v = load16(r, off);
    if (tail && kst + 4 > K) {
      const int64_t valid = K - kst;
#pragma unroll
      for (int d = 0; d < 4; ++d) if (d >= valid) v[d] = 0u;
    }
    dst[i] = v;
  }
}

template <int BP, int BQ, int WP, int WQ, bool P_TRANS>
__global__ void __launch_bounds__(WP * WQ * 64)
gemm_f32_kernel(const GemmArgs a) {
  using Cfg = F32Cfg<BP, BQ, WP, WQ, P_TRANS>;
  constexpr int NT = Cfg::NT, BK = Cfg::BK, ROWB = Cfg::ROWB;
  constexpr int PCH = Cfg::PCH, QCH = Cfg::QCH, TP = Cfg::TP, TQ = Cfg::TQ;

  __shared__ __attribute__((aligned(1024))) char smem[2 * Cfg::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wp = wave / WQ, wq = wave % WQ;

  int64_t tp, tq;
  tile_map(a.tiles_p, a.tiles_q, a.group, blockIdx.x, &tp, &tq);
  const int64_t p0 = tp * BP, q0 = tq * BQ;
  const int64_t K = a.K;
  const int nst = (int)((K + BK - 1) / BK);
  const uint32_t kbytes16 = (uint32_t)(((K * 4) + 15) & ~(int64_t)15);

  const int kc = tid & 7, lrow = tid >> 3;
  const int sw_w = (lrow >> 1) & 7;
  const uint32_t lds_kc = (uint32_t)(lrow * ROWB + ((kc ^ sw_w) << 4));

  const char* qblk = a.Q + q0 * a.ldq;
  const int64_t qrows = (a.Qn - q0) < BQ ? (a.Qn - q0) : BQ;
  const uint32_t qnrec = (uint32_t)((qrows - 1) * a.ldq) + kbytes16;
  uint32_t qvo[QCH];
#pragma unroll
  for (int i = 0; i < QCH; ++i) {
    const int row = i * (NT / 8) + lrow;
    qvo[i] = (row < qrows) ? (uint32_t)(row * a.ldq + kc * 16) : kOobOffset;
  }

  const char* pblk;
  uint32_t pnrec;
  uint32_t pvo[PCH];
  if constexpr (!P_TRANS) {
    pblk = a.P + p0 * a.ldp;
    const int64_t prows = (a.Pn - p0) < BP ? (a.Pn - p0) : BP;
    pnrec = (uint32_t)((prows - 1) * a.ldp) + kbytes16;
#pragma unroll
    for (int i = 0; i < PCH; ++i) {
      const int row = i * (NT / 8) + lrow;
      pvo[i] = (row < prows) ? (uint32_t)(row * a.ldp + kc * 16) : kOobOffset;
    }
  } else {
    pblk = a.P + p0 * 4;
    const int64_t pcols = (a.Pn - p0) < BP ? (a.Pn - p0) : BP;
    pnrec = (uint32_t)((K - 1) * a.ldp) + (uint32_t)(((pcols * 4) + 15) & ~(int64_t)15);
#pragma unroll
    for (int i = 0; i < PCH; ++i) {
      const int c = i * NT + tid;
      const int krow = c / Cfg::PT_CPR, pc = c % Cfg::PT_CPR;
      pvo[i] = (pc * 4 < pcols) ? (uint32_t)(krow * a.ldp + pc * 16) : kOobOffset;
    }
  }

  u32x4 pst[PCH], qst[QCH];

  auto load_stage = [&](int s, auto tail_tag) {
    constexpr bool tail = decltype(tail_tag)::value;
    load_kcontig_f32<QCH, BK>(qblk, qnrec, qvo, qst, s, tail, K, kc);
    if constexpr (!P_TRANS) {
      load_kcontig_f32<PCH, BK>(pblk, pnrec, pvo, pst, s, tail, K, kc);
    } else {
      const uint32_t adv = (uint32_t)((int64_t)s * BK * a.ldp);
      const __amdgpu_buffer_rsrc_t r = make_rsrc(pblk + (int64_t)s * BK * a.ldp, pnrec - adv);
#pragma unroll
      for (int i = 0; i < PCH; ++i) {
        uint32_t off = pvo[i];
        const int krow = (i * NT + tid) / Cfg::PT_CPR;
        if (tail && (int64_t)s * BK + krow >= K) off = kOobOffset;
        pst[i] = load16(r, off);
      }
    }
  };

  auto commit_stage = [&](int buf) {
    char* sp = smem + buf * Cfg::STAGE;
    char* sq = sp + Cfg::P_LDS;
#pragma unroll
    for (int i = 0; i < QCH; ++i) *(u32x4*)(sq + lds_kc + i * (NT / 8) * ROWB) = qst[i];
    if constexpr (!P_TRANS) {
#pragma unroll
      for (int i = 0; i < PCH; ++i) *(u32x4*)(sp + lds_kc + i * (NT / 8) * ROWB) = pst[i];
    } else {
#pragma unroll
      for (int i = 0; i < PCH; ++i) {
        const int c = i * NT + tid;
        const int krow = c / Cfg::PT_CPR, pc = c % Cfg::PT_CPR;
        *(u32x4*)(sp + krow * Cfg::PT_STRIDE + pc * 16) = pst[i];
      }
    }
  };

  const int l32 = lane & 31, h = lane >> 5;
  const int sw_r = (l32 >> 1) & 7;
  const uint32_t qf_base = (uint32_t)(Cfg::P_LDS + (wq * Cfg::WTQ + l32) * ROWB);
  const uint32_t pf_base = P_TRANS ? (uint32_t)((4 * h) * Cfg::PT_STRIDE + (wp * Cfg::WTP + l32) * 4)
                                   : (uint32_t)((wp * Cfg::WTP + l32) * ROWB);

  f32x16 acc[TP][TQ];
#pragma unroll
  for (int i = 0; i < TP; ++i)
#pragma unroll
    for (int j = 0; j < TQ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto compute_stage = [&](int buf) {
    const char* sb = smem + buf * Cfg::STAGE;
#pragma unroll
    for (int kb = 0; kb < BK / 8; ++kb) {
      const uint32_t off = (uint32_t)(((2 * kb + h) ^ sw_r) << 4);
      f32x4 qf[TQ], pf[TP];
#pragma unroll
      for (int j = 0; j < TQ; ++j) qf[j] = *(const f32x4*)(sb + qf_base + j * 32 * ROWB + off);
#pragma unroll
      for (int i = 0; i < TP; ++i) {
        if constexpr (!P_TRANS) {
          pf[i] = *(const f32x4*)(sb + pf_base + i * 32 * ROWB + off);
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            pf[i][t] = *(const float*)(sb + pf_base + (8 * kb + t) * Cfg::PT_STRIDE + i * 32 * 4);
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < TP; ++i)
#pragma unroll
          for (int j = 0; j < TQ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(pf[i][t], qf[j][t], acc[i][j], 0, 0, 0);
    }
  };

  // Stage s is computed from buffer s % 2 while stage s + 1 is fetched into
  // registers and then committed to the other buffer.  Only the last stage can
  // be partial in K, so only its load carries the K-tail checks.
  if (nst > 0) {
    if (nst == 1) load_stage(0, std::true_type{});
    else load_stage(0, std::false_type{});
    commit_stage(0);
    __syncthreads();
    int s = 0;
    // The scheduling fences keep the next stage's global loads ahead of the
    // MFMAs (so their latency hides behind a whole stage of math) and the LDS
    // commit after them; left alone, the compiler sinks the loads to the
    // commit to shorten register live ranges, exposing the full latency.
    for (; s < nst - 2; ++s) {
      load_stage(s + 1, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      compute_stage(s & 1);
      __builtin_amdgcn_sched_barrier(0);
      commit_stage((s + 1) & 1);
      __syncthreads();
    }
    if (s < nst - 1) {
      load_stage(s + 1, std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
      compute_stage(s & 1);
      __builtin_amdgcn_sched_barrier(0);
      commit_stage((s + 1) & 1);
      __syncthreads();
      ++s;
    }
    compute_stage(s & 1);
  }


#pragma unroll
  for (int i = 0; i < TP; ++i) {
#pragma unroll
    for (int j = 0; j < TQ; ++j) {
      const int64_t q = q0 + wq * Cfg::WTQ + 32 * j + l32;
      if (q >= a.Qn) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t p = p0 + wp * Cfg::WTP + 32 * i + 8 * g + 4 * h;
        float* c = (float*)a.C + q * a.ldc + p;
        const float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
        const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
        if (a.vec_store && p + 3 < a.Pn) {
          *(f32x4*)c = f32x4{v0, v1, v2, v3};
        } else {
          if (p + 0 < a.Pn) c[0] = v0;
          if (p + 1 < a.Pn) c[1] = v1;
          if (p + 2 < a.Pn) c[2] = v2;
          if (p + 3 < a.Pn) c[3] = v3;
        }
      }
    }
  }
}

}  // namespace dg
