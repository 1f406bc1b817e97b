// TN (and NN) GEMM for 16-bit and 8-bit operands on gfx950: four waves, one
// per SIMD, each owning a quarter of the block tile (128 x 128 of 256 x 256)
// as 16 x 16 MFMA tiles.
//
// Same operation and P/Q/D mapping as gemm_mfma.hpp (D[p][q] = sum_k
// P(p,k) Q(q,k), stored at C[q*ldc + p]), for K-contiguous Q, K a whole
// number of 16-byte chunks and at least two stages.  Differences:
//
//  * 128 x 128 wave tiles read half as much LDS per flop as the eight-wave
//    128 x 64 split, and one wave per SIMD leaves all 512 registers to it
//    (accumulators in AGPRs).
//  * One tile per workgroup; tiles follow the XCD-aware order of tile_map.
//  * Copies of a stage are split: NA go out after the barrier two stages
//    ahead, the other NDMA - NA over the first NBSPAN MFMA slots of the stage
//    before, so the texture unit sees them spread out.
//  * NS LDS stages: with NS > 2 (small tiles, one workgroup per CU) every
//    copy goes out NS stages ahead, so a stage's copy latency hides behind
//    NS - 1 stages of MFMAs.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "gemm_mfma.hpp"

namespace dg {

template <class Op, bool PKM, int BP_ = 256, int BQ_ = 256, int NS_ = 2>
struct TnCfg {
  static constexpr int BP = BP_, BQ = BQ_, WP = 2, WQ = 2, NW = 4, NT = 256;
  static constexpr int NS = NS_;                  // LDS stages (a power of two)
  static_assert(NS == 2 || NS == 4, "two or four stages");
  static constexpr int E = Op::ELEM, FC = Op::FC;
  static constexpr int ROWB = 128;                // bytes of k per LDS row per stage
  static constexpr int BK = ROWB / E;             // k per stage
  static constexpr int CPE = 16 / E;              // elements per 16-byte chunk
  static constexpr int P_LDS = BP * ROWB;
  static constexpr int STAGE = (BP + BQ) * ROWB;  // 64 KiB
  // MX: after the NS stages, a ring of two scale groups; a group holds four
  // stages' block scales (16 bytes, 16 blocks of 32 k) of every P row, then
  // of every Q row.
  static constexpr int SC_ROWS = Op::MX ? BP + BQ : 0;
  static constexpr int SG_STAGES = 4;             // stages per scale group
  static constexpr int SG_BYTES = 16 * SC_ROWS;
  static constexpr int SC_INST = SC_ROWS / 64;    // 64-row copies per group
  static constexpr int LDS = NS * STAGE + 2 * SG_BYTES;
  static constexpr int QSEG = BQ / 8 / NW, PSEG = BP / 8 / NW;
  static constexpr int NDMA = QSEG + PSEG;        // copy instructions per wave per stage
  static constexpr int WTP = BP / WP, WTQ = BQ / WQ;
  // MFMA tile: 16 x 16 (x 32 for FP16/BF16, x 128 for FP8 and MXFP8), which
  // sustains 10-13% more throughput than the 32 x 32 shapes on the same wave
  // tile once the chip runs at its power limit (random operands; equal at
  // zero data).
  static constexpr int MT = 16;
  static constexpr int KI = E == 2 ? 32 : 128;    // k per MFMA
  static constexpr int ACC = MT * MT / 64;         // accumulator registers per tile
  using Acc = f32x4;
  static constexpr int TP = WTP / MT, TQ = WTQ / MT;
  static constexpr int KSTEPS = BK / KI;
  static constexpr int CPK = KI * E / 16;          // 16-byte chunks of k per k-step
  // One k-step per stage (FP8 16 x 16 x 128): fragments cannot be double
  // buffered next to the accumulators, so the stage runs "rolling": P tiles
  // 0 .. TP/2-1 against every Q tile before the barrier while P tiles TP/2 ..
  // come in, the rest after it, Q tile by Q tile, each fragment register
  // refilled with the next stage's data right after its last use.
  static constexpr bool ROLL = KSTEPS == 1;
  static_assert(!ROLL || TP % 2 == 0, "two halves of P tiles");
  static_assert(!Op::MX || ROLL, "MX block scales follow the 16 x 16 x 128 stage");
  // LDS reads per k-step: 16-byte reads of Q fragments, and of P fragments
  // either 16-byte reads (K-contiguous P) or twice as many 8-byte
  // transposing reads (p-contiguous P).
  static constexpr int PRD = PKM ? 2 * FC : FC;   // reads per P fragment
  static constexpr int NREAD = TQ * FC + TP * PRD;
  // p-contiguous P: LDS rows of k, BP*E bytes, in units of 32 p (UB bytes)
  // XOR-swizzled by a key of k below KEYM: (k mod 8) ^ 4 ((k / 16) mod 2)
  // (FP8) or (k mod 4) ^ 2 ((k / 8) mod 2) (16-bit), so that the fragment's
  // lane groups 0 and 1, which read k rows sixteen (eight) apart, meet
  // different banks.
  static constexpr int PROWB = BP * E;            // bytes of one LDS row of P (one k)
  static constexpr int UB = 32 * E;
  static constexpr int KEYM = 256 / UB;
  static constexpr int RPSG = 1024 / PROWB;       // rows of P per 1 KiB copy segment
  static constexpr int NMFMA = TP * TQ;           // MFMAs per k-step
  // MFMA slots before and after the barrier
  static constexpr int SLOTS1 = ROLL ? NMFMA / 2 : (KSTEPS - 1) * NMFMA;
  static constexpr int SLOTS2 = ROLL ? NMFMA / 2 : NMFMA;
  // Copy split: FP16/BF16 issue three quarters of a stage's copies after the
  // barrier two stages ahead, over the first NASPAN MFMA slots, and the rest
  // over the first NBSPAN slots of the stage before; FP8 issues them all
  // after the barrier, over every slot.  (16 x 16 tiles, measured against an
  // even split: +3-4%; the after-barrier copies within three quarters of the
  // slots: +1%.)
  static constexpr int NA = (Op::ELEM == 2 && NS == 2) ? 3 * NDMA / 4 : NDMA;
  static constexpr int NB = NDMA - NA;
  static constexpr int NASPAN = Op::ELEM == 2 ? 3 * SLOTS2 / 4 : SLOTS2;
  static constexpr int NBSPAN = NMFMA / 4;
  static_assert(NB == 0 || NBSPAN <= SLOTS1, "part-B copies go out before the barrier");
  static_assert(LDS <= kLdsLimit, "LDS budget");
  // The scale ring relies on every mid-stage wait draining all copies.
  static_assert(!Op::MX || NS == 2, "MX scale groups need two stages");
  // Copies in flight when a stage's data must have landed: those of the
  // NS - 2 later stream positions.
  static constexpr int VM_MID = (NS - 2) * NDMA;
  static_assert(!PKM || (PROWB / UB) % KEYM == 0, "swizzle keys stay within a row of P");
  // FP8: lane groups 0 and 1 read k rows sixteen apart.
  __device__ static int pkey(int k) {
    if constexpr (E == 2) return (k & 3) ^ (((k >> 3) & 1) << 1);
    else return (k & 7) ^ (((k >> 4) & 1) << 2);
  }
  // The LDS-staged epilogue needs 256-byte staged rows; smaller wave tiles
  // store straight from the accumulators.
  static constexpr bool STAGED_EPI = (TP / (Op::OE == 4 ? 2 : 1)) * MT * Op::OE == 256;
  // Waves per SIMD the kernel is compiled for: a 64x64 wave tile is small
  // enough for two (two workgroups per CU).
  static constexpr int WPE = TP * TQ * ACC <= 64 && NS == 2 ? 2 : 1;
};

template <class Op, bool PKM, int BP, int BQ, int NS, bool KT>
__device__ __forceinline__ void gemm_tn_body(const GemmArgs& a) {
  using Cfg = TnCfg<Op, PKM, BP, BQ, NS>;
  constexpr int NW = Cfg::NW, E = Cfg::E, FC = Cfg::FC, ROWB = Cfg::ROWB, BK = Cfg::BK, CPE = Cfg::CPE;
  constexpr int TP = Cfg::TP, TQ = Cfg::TQ, QSEG = Cfg::QSEG, NDMA = Cfg::NDMA;
  constexpr int NREAD = Cfg::NREAD, NMFMA = Cfg::NMFMA, NA = Cfg::NA, NB = Cfg::NB, NBSPAN = Cfg::NBSPAN;
  constexpr int NASPAN = Cfg::NASPAN;
  constexpr int MT = Cfg::MT, KI = Cfg::KI, CPK = Cfg::CPK;
  using Acc = typename Cfg::Acc;

  __shared__ __attribute__((aligned(1024))) char smem[Cfg::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int wp = wave_u / Cfg::WQ, wq = wave_u % Cfg::WQ;
  const int64_t K = a.K;
  const int nst = (int)((K + BK - 1) / BK);
  const uint32_t kbytes16 = (uint32_t)(((K * E) + 15) & ~(int64_t)15);
  const int64_t ntiles = a.tiles_p * a.tiles_q;

  // ---- copies ----
  // One copy instruction fills one 1 KiB LDS segment = 8 rows of 128 bytes:
  // lane l lands at byte 16*l, row 8*seg + l/8, physical chunk l%8, which
  // holds logical chunk (l%8) ^ key(row), key(row) = (row/2) mod 8 =
  // (4*(wave%2) + l/16) mod 8 for segment i*4 + wave.  Rows past the matrix
  // edge need no test: their offsets are at least rows*ld >= num_records.
  const int dkc = (lane & 7) ^ ((4 * (wave_u & 1) + (lane >> 4)) & 7);
  const int dk0 = dkc * CPE;
  uint32_t qvo[QSEG], pvo[Cfg::PSEG];
#pragma unroll
  for (int i = 0; i < QSEG; ++i) qvo[i] = (uint32_t)((8 * (i * NW + wave_u) + (lane >> 3)) * a.ldq + dkc * 16);
  if constexpr (!PKM) {
#pragma unroll
    for (int i = 0; i < Cfg::PSEG; ++i)
      pvo[i] = (uint32_t)((8 * (i * NW + wave_u) + (lane >> 3)) * a.ldp + dkc * 16);
  } else {
    // p-contiguous P (NN's B): a segment holds RPSG rows of k; lane l lands
    // at row l*16 / PROWB, byte (l*16) % PROWB, i.e. physical unit pu with
    // offset w, which holds logical unit pu ^ pkey(k).  Rows past K are past
    // num_records and read zero; columns past the tile edge read whatever
    // follows in B (those p are never stored).
#pragma unroll
    for (int i = 0; i < Cfg::PSEG; ++i) {
      const int kr = Cfg::RPSG * (i * NW + wave_u) + (lane * 16) / Cfg::PROWB;
      const int br = (lane * 16) % Cfg::PROWB;
      const int lu = (br / Cfg::UB) ^ Cfg::pkey(kr);
      pvo[i] = (uint32_t)(kr * a.ldp + lu * Cfg::UB + br % Cfg::UB);
    }
  }
  // Copy source of one tile: block base pointers and descriptor sizes.  A
  // tile index past the end gives zero records (its copies read zeros).
  struct Src {
    const char* q;
    const char* p;
    uint32_t qn, pn;
    const uint8_t* sq;   // MX: block scales of the tile's q and p rows
    const uint8_t* sp;
    uint32_t sqn, spn;
  };
  auto tile_src = [&](int64_t tile) {
    Src r;
    if (tile < ntiles) {
      int64_t tp, tq;
      tile_map(a.tiles_p, a.tiles_q, a.group, tile, &tp, &tq);
      const int64_t q0 = tq * Cfg::BQ, p0 = tp * Cfg::BP;
      const int64_t qrows = (a.Qn - q0) < Cfg::BQ ? (a.Qn - q0) : Cfg::BQ;
      const int64_t prows = (a.Pn - p0) < Cfg::BP ? (a.Pn - p0) : Cfg::BP;
      r.q = a.Q + q0 * a.ldq;
      r.qn = (uint32_t)((qrows - 1) * a.ldq) + kbytes16;
      if constexpr (Op::MX) {
        // The caller provides rows * ld scale bytes; with K == 0 none at all.
        r.sq = a.msq + q0 * a.ldsq;
        r.sqn = K > 0 ? (uint32_t)(qrows * a.ldsq) : 0u;
        r.sp = a.msp + p0 * a.ldsp;
        r.spn = K > 0 ? (uint32_t)(prows * a.ldsp) : 0u;
      }
      if constexpr (!PKM) {
        r.p = a.P + p0 * a.ldp;
        r.pn = (uint32_t)((prows - 1) * a.ldp) + kbytes16;
      } else {
        // (K == 0 has no rows of P at all: an empty descriptor, not one
        // whose (K - 1) * ldp term wraps around.)
        r.p = a.P + p0 * E;
        r.pn = K > 0 ? (uint32_t)((K - 1) * a.ldp) + (uint32_t)(((prows * E) + 15) & ~(int64_t)15) : 0u;
      }
    } else {
      r.q = a.Q;
      r.p = a.P;
      r.qn = 0;
      r.pn = 0;
      if constexpr (Op::MX) {
        r.sq = a.msq;
        r.sp = a.msp;
        r.sqn = 0;
        r.spn = 0;
      }
    }
    return r;
  };
  // With p-contiguous P the copies go through inline assembly (see
  // copy16_lds), which takes the descriptor as four dwords.
  using Rsrc = std::conditional_t<PKM, i32x4, __amdgpu_buffer_rsrc_t>;
  auto rsrc = [](const char* base, uint32_t nrec) -> Rsrc {
    if constexpr (PKM) return make_desc(base, nrec);
    else return make_rsrc(base, nrec);
  };
  // Chunks at or past K read zero: bit 31 puts the offset past num_records.
  // Only a stage that ends inside K has such chunks (KT).
  auto kill_at = [&](int t) -> uint32_t {
    if constexpr (!KT) {
      (void)t;
      return 0u;
    } else {
      const int64_t rem64 = K - (int64_t)t * BK;
      const int rem = (int)(rem64 < BK ? rem64 : BK);
      return dk0 >= rem ? kOobOffset : 0u;
    }
  };
  // Copy source of stream position t of a tile: descriptors advanced to
  // stage t (K-contiguous operands move along the row, p-contiguous P down
  // BK rows) and the tail mask.  An invalid position (a stage past the
  // tile's end, or of no tile) gets empty descriptors and reads zeros.  A
  // valid one keeps records left, as every stage of a tile starts inside
  // the descriptor's range; the count is a plain scalar select (a
  // saturating subtract would go through vector registers).
  struct Pos {
    Rsrc q, p;
    uint32_t kill;
  };
  auto pos_at = [&](const Src& src, int t, bool valid) -> Pos {
    const uint32_t aq = (uint32_t)t * ROWB;
    const uint32_t ap = PKM ? (uint32_t)((int64_t)t * BK * a.ldp) : aq;
    return Pos{rsrc(src.q + aq, valid ? src.qn - aq : 0u), rsrc(src.p + ap, valid ? src.pn - ap : 0u), kill_at(t)};
  };
  auto copy_d = [&](const Pos& ps, char* stage_lds, int d) {
    const Rsrc& rq = ps.q;
    const Rsrc& rp = ps.p;
    const uint32_t kill = ps.kill;
    if constexpr (PKM) {
      if (d < QSEG) copy16_lds(rq, qvo[d] | kill, stage_lds + Cfg::P_LDS + (d * NW + wave_u) * 1024);
      else copy16_lds(rp, pvo[d - QSEG], stage_lds + ((d - QSEG) * NW + wave_u) * 1024);
    } else if (d < QSEG) {
      char* dst = stage_lds + Cfg::P_LDS + (d * NW + wave_u) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (__attribute__((address_space(3))) void*)dst, 16, qvo[d] | kill, 0,
                                               0, 0);
    } else {
      char* dst = stage_lds + ((d - QSEG) * NW + wave_u) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (__attribute__((address_space(3))) void*)dst, 16,
                                               pvo[d - QSEG] | kill, 0, 0, 0);
    }
  };

  // ---- fragments and MFMAs ----
  // A lane holds row lr = lane % MT of its P and Q fragments; its lane group
  // lg = lane / MT selects the k it holds.
  const int lr = lane % MT, lg = lane / MT;
  const int sw_r = (lr >> 1) & 7;                // swizzle key of every fragment row of this lane
  const uint32_t pf_base = (uint32_t)((wp * Cfg::WTP + lr) * ROWB);
  const uint32_t qf_base = (uint32_t)(Cfg::P_LDS + (wq * Cfg::WTQ + lr) * ROWB);
  u32x4 fa[2][TP][FC], fb[2][TQ][FC];
  // Transposing reads of p-contiguous P (ds_read_b64_tr_b16 / _tr_b8): in
  // each 16-lane group, output lane i receives element i % 4 (bytes: i % 8)
  // of source lanes i/4 + 4j (i/8 + 2j).  So a source lane addresses 4 (8)
  // consecutive p of row k = kbase + s/4 (s/2), s = lane % 16, and output
  // lane i ends up with 4 (8) consecutive k of p = pbase + i.  Every row a
  // lane addresses has the same swizzle key, s/4 (s/2).
  const int tg = lane >> 4, ts = lane & 15;
  constexpr int TRK = 8 / E;                    // k per transposing read
  const int tkey = ts / (2 * E);                // k mod KEYM of every row this lane addresses
  auto read_one = [&](const char* sb, int kk, int set, int r) {
    const bool isb = r < TQ * FC;
    if (isb || !PKM) {
      const int rr = isb ? r : r - TQ * FC;
      const int tile = rr / FC, f = rr % FC;
      // 16-byte chunk kk*CPK + f*(CPK/FC) + lg of the stage row: 16-bit lane
      // group lg takes the lg-th 8 k of the step; FP8 lane group lg takes
      // chunks lg and lg + 4 (16 k each) of its 128-k step, which puts the
      // MFMA's scale block L on the L-th 32 k (see OpMX8).
      const uint32_t off = (uint32_t)(((kk * CPK + f * (CPK / FC) + lg) ^ sw_r) << 4);
      const char* base = sb + (isb ? qf_base : pf_base) + tile * MT * ROWB;
      const u32x4 v = *(const u32x4*)(base + off);
      if (isb) fb[set][tile][f] = v; else fa[set][tile][f] = v;
    } else {
      const int rr = r - TQ * FC;
      const int tile = rr / Cfg::PRD, q8 = rr % Cfg::PRD;   // which 8-byte piece of the fragment
      // k of this lane's row: the k-step, the lane group, the piece q8 (TRK
      // k each) and tkey, in the order of the K-contiguous reads of Q.
      // 16-bit: group tg holds k 8tg .. 8tg+7 of the step.  FP8: group tg
      // holds k 16tg .. 16tg+15 in pieces 0-1 and k 64+16tg .. in pieces 2-3.
      const int krow = E == 2 ? kk * KI + tg * 8 + q8 * TRK + tkey
                              : kk * KI + (q8 >> 1) * 64 + tg * 16 + (q8 & 1) * 8 + tkey;
      const int pbyte = (wp * Cfg::WTP + tile * MT) * E;
      const int unit = (pbyte / Cfg::UB) ^ Cfg::pkey(krow);
      const char* src = sb + krow * Cfg::PROWB + unit * Cfg::UB + pbyte % Cfg::UB + (ts % (2 * E)) * 8;
      typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
      u32x2 v;
      if constexpr (E == 2) {
        typedef __fp16 h16x4 __attribute__((ext_vector_type(4)));
        v = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                                          (__attribute__((address_space(3))) h16x4*)src));
      } else {
        typedef int i32x2v __attribute__((ext_vector_type(2)));
        v = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                          (__attribute__((address_space(3))) i32x2v*)src));
      }
      fa[set][tile][q8 >> 1][2 * (q8 & 1)] = v[0];
      fa[set][tile][q8 >> 1][2 * (q8 & 1) + 1] = v[1];
    }
  };
  Acc acc[TP][TQ];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < TP; ++i)
#pragma unroll
      for (int j = 0; j < TQ; ++j)
#pragma unroll
        for (int r = 0; r < Cfg::ACC; ++r) acc[i][j][r] = 0.0f;
  };
  // MX block scales: for the stage in use, lane l holds in scp[i] / scq[j]
  // the scale of its row of P tile i / Q tile j for block lg of the stage (a
  // stage is four blocks of 32 k), in byte 0.  Scale group G of a tile (stages 4G .. 4G+3) travels
  // as one 16-byte copy per row (64 rows per instruction, spread over the
  // waves) into ring buffer gam % 2, gam counting groups along the stream of
  // stages.  The last stage of a group picks (without branching) the group
  // two ahead; the next stage copies it first thing, into the buffer of the
  // group just finished, which every wave is done with since that stage's
  // barrier; its own barrier drains the copy before any stage reads it.  (A
  // branch among the MFMAs would let the compiler sink them past it.)  A
  // stage's dword is read in the second half of the stage before, and taken
  // at its start.
  char* const sring = smem + NS * Cfg::STAGE;
  [[maybe_unused]] uint32_t scp[TP], scq[TQ], nsp[TP], nsq[TQ];
  [[maybe_unused]] int gam = 0;
  [[maybe_unused]] bool gpend = false;   // a group copy for the next stage to issue
  [[maybe_unused]] int gpend_g = 0, gpend_buf = 0;
  [[maybe_unused]] Src gpend_src{};
  auto copy_group = [&](const Src& src, int G, int buf) {
    if constexpr (Op::MX) {
#pragma unroll
      for (int u0 = 0; u0 < Cfg::SC_INST; u0 += NW) {
        const int u = u0 + wave_u;
        if (u0 + NW > Cfg::SC_INST && u >= Cfg::SC_INST) break;
        const bool isp = 64 * u < Cfg::BP;
        const int row = isp ? 64 * u + lane : 64 * u - Cfg::BP + lane;
        const uint32_t voff = (uint32_t)(row * (isp ? a.ldsp : a.ldsq) + 16 * G);
        char* dst = sring + buf * Cfg::SG_BYTES + 1024 * u;
        if constexpr (PKM) {
          copy16_lds(isp ? make_desc(src.sp, src.spn) : make_desc(src.sq, src.sqn), voff, dst);
        } else {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(isp ? make_rsrc(src.sp, src.spn) : make_rsrc(src.sq, src.sqn),
                                                   (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, 0);
        }
      }
    }
  };
  auto read_scales = [&](int buf, int slot) {
    if constexpr (Op::MX) {
      const char* g0 = sring + buf * Cfg::SG_BYTES + 4 * slot;
#pragma unroll
      for (int i = 0; i < TP; ++i) nsp[i] = *(const uint32_t*)(g0 + 16 * (wp * Cfg::WTP + MT * i + lr));
#pragma unroll
      for (int j = 0; j < TQ; ++j) nsq[j] = *(const uint32_t*)(g0 + 16 * (Cfg::BP + wq * Cfg::WTQ + MT * j + lr));
    }
  };
  // Blocks at or past K/32 read as scale byte 0 (their data are zeros; a
  // stray 255 would be NaN).
  auto take_scales = [&](int t, const uint32_t(&sp)[TP], const uint32_t(&sq)[TQ]) {
    if constexpr (Op::MX) {
      const int64_t valid = K / 32 - 4 * (int64_t)t;
      const uint32_t m = valid >= 4 ? ~0u : (valid <= 0 ? 0u : ((1u << (8 * valid)) - 1u));
#pragma unroll
      for (int i = 0; i < TP; ++i) scp[i] = (sp[i] & m) >> (8 * lg);
#pragma unroll
      for (int j = 0; j < TQ; ++j) scq[j] = (sq[j] & m) >> (8 * lg);
    }
  };
  auto mfma_one = [&](int set, int t) {
    const int i = t / TQ, j = t % TQ;
    if constexpr (!Op::MX) acc[i][j] = Op::mma16(fa[set][i], fb[set][j], acc[i][j]);
  };
  // n operations spread over `span` MFMA slots: operation i goes out after
  // MFMA i * span / n, so slot t issues i in [first(n, span, t),
  // first(n, span, t + 1)).  (Ranges, not a test of every i in every slot:
  // the unroller would give up on the larger 16 x 16 schedules.)
  auto first = [](int n, int span, int t) { return (t * n + span - 1) / span; };
  constexpr int LAST = (Cfg::KSTEPS - 1) & 1;

  // MX: when stage s ends group gam, its buffer takes group gam + 2, the
  // group after the one the next stage opens, if the tile has it (else the
  // copy reads zeros from `none`).  Decided without branching; the next stage
  // issues the copy first thing.
  auto mx_next = [&](int s, int snext, bool opens, const Src& cu, const Src& none) {
    if constexpr (Op::MX) {
      const int Gn = snext / Cfg::SG_STAGES;
      const bool more = s + 1 < nst && (Gn + 1) * Cfg::SG_STAGES < nst;
      gpend = opens;
      gpend_buf = gam & 1;
      gpend_g = Gn + 1;
      gpend_src = more ? cu : none;
      gam += opens ? 1 : 0;
    }
  };

  // Stream position g + NS (the copies after the barrier of stage g).
  auto pos_far = [&](int s, const Src& cu) -> Pos { return pos_at(cu, s + NS, s + NS < nst); };

  // ---- one stage, rolling (one k-step per stage) ----
  // Phase 1, before the barrier: P tiles 0 .. HP-1 against every Q tile,
  // Q-major, while P tiles HP .. TP-1 of this stage are read (their
  // registers were freed by the previous stage's phase 2).  Phase 2: P tiles
  // HP .. TP-1, Q-major, so Q tile j is done after slot HP (j + 1) - 1 and
  // its next-stage fragment is read right then; P tiles 0 .. HP-1 of the
  // next stage are read over the first three quarters of the phase.  Every
  // read of buffer g % NS is issued before the barrier, so the copies after
  // it may overwrite that buffer; the next stage's reads come after it, once
  // its data is known to have landed.  Copies as in `stage`.
  auto stage_roll = [&](int g, int s, const Src& cu, const Src& none, Pos& p1) {
    constexpr int HP = TP / 2, NM1 = Cfg::SLOTS1;
    constexpr int RQ = TQ * FC;                 // reads of the Q fragments
    constexpr int RP = HP * Cfg::PRD;           // reads of half the P fragments
    const int b = g & (NS - 1);
    const char* sb = smem + b * Cfg::STAGE;
    char* ob = smem + ((g + 1) & (NS - 1)) * Cfg::STAGE;
    auto mma_ij = [&](int i, int j) {
      if constexpr (Op::MX) acc[i][j] = Op::mma16_mx(fa[0][i], fb[0][j], acc[i][j], scp[i], scq[j]);
      else acc[i][j] = Op::mma16(fa[0][i], fb[0][j], acc[i][j]);
    };
    if constexpr (Op::MX) {
      if (gpend) copy_group(gpend_src, gpend_g, gpend_buf);
      take_scales(s, nsp, nsq);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < NM1; ++t) {
      mma_ij(t % HP, t / HP);
#pragma unroll
      for (int x = first(RP, NM1 / 2, t); x < first(RP, NM1 / 2, t + 1) && x < RP; ++x)
        read_one(sb, 0, 0, RQ + RP + x);
      if constexpr (NB > 0) {
#pragma unroll
        for (int j = first(NB, NBSPAN, t); j < first(NB, NBSPAN, t + 1) && j < NB; ++j) copy_d(p1, ob, NA + j);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    [[maybe_unused]] const int snext = s + 1 >= nst ? 0 : s + 1;
    [[maybe_unused]] const bool opens = snext % Cfg::SG_STAGES == 0;
    if constexpr (NS == 2) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    else __builtin_amdgcn_s_waitcnt(kWaitVmcntBase | vmcnt_bits(Cfg::VM_MID));
    __syncthreads();
    // MX: the next stage's scales, first of the reads: it opens a group (its
    // tile's stage 0 or a multiple of four) or continues this one.
    if constexpr (Op::MX) read_scales((gam + (opens ? 1 : 0)) & 1, snext % Cfg::SG_STAGES);
    __builtin_amdgcn_sched_barrier(0);
    const Pos p2 = pos_far(s, cu);
    char* db = smem + b * Cfg::STAGE;
#pragma unroll
    for (int u = 0; u < NM1; ++u) {
      mma_ij(HP + u % HP, u / HP);
      if (u % HP == HP - 1) {
#pragma unroll
        for (int f = 0; f < FC; ++f) read_one(ob, 0, 0, (u / HP) * FC + f);
      }
#pragma unroll
      for (int x = first(RP, 3 * NM1 / 4, u); x < first(RP, 3 * NM1 / 4, u + 1) && x < RP; ++x)
        read_one(ob, 0, 0, RQ + x);
#pragma unroll
      for (int d = first(NA, NASPAN, u); d < first(NA, NASPAN, u + 1) && d < NA; ++d) copy_d(p2, db, d);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (Op::MX) mx_next(s, snext, opens, cu, none);
    p1 = p2;
  };

  // ---- one stage (FP16/BF16: two or more k-steps) ----
  // Global stage g (buffer g % NS) is stage s of the current tile.  Copies
  // issued here belong to the stream position g + NS (after the barrier; NA
  // of them) and g + 1 (before it; NB of them, two stages only); positions
  // past the tile read zeros.  `p1` holds position g + 1 on entry and g + NS
  // on return: with two stages that is the next stage's g + 1.
  auto stage = [&](int g, int s, const Src& cu, Pos& p1) {
    const int b = g & (NS - 1);
    const char* sb = smem + b * Cfg::STAGE;
    char* ob = smem + ((g + 1) & (NS - 1)) * Cfg::STAGE;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk + 1 < Cfg::KSTEPS; ++kk) {
      const int span = kk + 2 == Cfg::KSTEPS ? NMFMA / 2 : NMFMA;
#pragma unroll
      for (int t = 0; t < NMFMA; ++t) {
        mfma_one(kk & 1, t);
#pragma unroll
        for (int r = first(NREAD, span, t); r < first(NREAD, span, t + 1); ++r) read_one(sb, kk + 1, (kk + 1) & 1, r);
        if constexpr (NB > 0) {
          const int x = kk * NMFMA + t;
#pragma unroll
          for (int j = first(NB, NBSPAN, x); j < first(NB, NBSPAN, x + 1) && j < NB; ++j) copy_d(p1, ob, NA + j);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Stream position g + 1 has landed (later positions may still be in flight).
    if constexpr (NS == 2) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    else __builtin_amdgcn_s_waitcnt(kWaitVmcntBase | vmcnt_bits(Cfg::VM_MID));
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // stream position g + NS
    const Pos p2 = pos_far(s, cu);
    char* db = smem + b * Cfg::STAGE;
#pragma unroll
    for (int t = 0; t < NMFMA; ++t) {
      mfma_one(LAST, t);
#pragma unroll
      for (int r = first(NREAD, NMFMA, t); r < first(NREAD, NMFMA, t + 1); ++r) read_one(ob, 0, 0, r);
#pragma unroll
      for (int d = first(NA, NASPAN, t); d < first(NA, NASPAN, t + 1) && d < NA; ++d) copy_d(p2, db, d);
      __builtin_amdgcn_sched_barrier(0);
    }
    p1 = p2;
  };

  // ---- tiles ----
  const int64_t tile = blockIdx.x;
  if (tile >= ntiles) return;
  // Clock trace: the start stamps go out now, so that nothing of the trace
  // stays live across the stage loop.
  auto stamp = [&](int at) {
    if (a.trace != nullptr && wave_u == 0 && lane_id() == 0 && tile < a.trace_n) {
      unsigned long long* t = a.trace + 4 * tile + at;
      t[0] = __builtin_amdgcn_s_memtime();
      t[1] = __builtin_amdgcn_s_memrealtime();
    }
  };
  stamp(0);
  const Src cur = tile_src(tile);
  // A source with empty descriptors (its copies read zeros): MX scale
  // groups past the tile's last.
  [[maybe_unused]] const Src none = tile_src(ntiles);
  Pos p1;   // the stream position after the current stage's
  {
    // Prologue: stream positions 0 .. NS-1 (with nst < NS the later ones
    // read zeros that nothing uses), without the part-B copies of position 1,
    // which stage 0 issues.
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const Pos ps = pos_at(cur, t, t < nst);
      if (t == 1) p1 = ps;
#pragma unroll
      for (int d = 0; d < (t == NS - 1 ? NA : NDMA); ++d) copy_d(ps, smem + t * Cfg::STAGE, d);
      if (t == 0) {
        // MX: the first two scale groups of the stream, ahead of the copies
        // the wait below leaves open.
        copy_group(cur, 0, 0);
        if (Cfg::SG_STAGES < nst) copy_group(cur, 1, 1);
        else copy_group(none, 0, 1);
      }
    }
    // Position 0 has landed once at most the copies of positions 1 .. NS-1
    // are open.
    __builtin_amdgcn_s_waitcnt(kWaitVmcntBase | vmcnt_bits(Cfg::VM_MID + NA));
    __syncthreads();
    if constexpr (Op::MX) read_scales(0, 0);
    // Stage 0's first fragments: all of them, or (rolling) the Q tiles and
    // the first half of the P tiles.
    constexpr int NR0 = Cfg::ROLL ? TQ * FC + (TP / 2) * Cfg::PRD : NREAD;
#pragma unroll
    for (int r = 0; r < NR0; ++r) read_one(smem, 0, 0, r);
  }
  // Epilogue straight from the accumulators: four consecutive p of one q per
  // lane and group, one 8- or 16-byte store each (32 x 32 tiles: lane l
  // holds q = 32 j + l % 32, p = 32 i + 8 g + 4 (l / 32) for group g; 16 x 16
  // tiles: q = 16 j + l % 16, p = 16 i + 4 (l / 16)).
  constexpr int NG = MT * MT / 256;   // register groups of four per tile
  auto direct_epilogue = [&](int64_t t) {
    // (lane values recomputed here, not kept live across the stage loop)
    const int lr = lane_id() % MT, lg = lane_id() / MT;
    int64_t tp, tq;
    tile_map(a.tiles_p, a.tiles_q, a.group, t, &tp, &tq);
    const int64_t pb = tp * Cfg::BP + wp * Cfg::WTP, qb = tq * Cfg::BQ + wq * Cfg::WTQ;
    [[maybe_unused]] EpiScale<TQ, MT> sc;
    if constexpr (Op::SCALED) sc.init(a, lane_id(), qb);
    // Column by column: a lane's four stores into one column of C follow
    // each other, so each 128-byte line is written whole while it is open.
#pragma unroll
    for (int i = 0; i < TP; ++i) {
      [[maybe_unused]] f32x4 fp[NG];
      if constexpr (Op::SCALED) {
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) fp[gg] = EpiScale<TQ, MT>::p4(a, pb + MT * i + 8 * gg + 4 * lg);
      }
#pragma unroll
      for (int j = 0; j < TQ; ++j) {
        const int64_t q = qb + MT * j + lr;
        if (q >= a.Qn) continue;
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
          const int64_t p = pb + MT * i + 8 * gg + 4 * lg;
          float v0 = acc[i][j][4 * gg + 0], v1 = acc[i][j][4 * gg + 1], v2 = acc[i][j][4 * gg + 2],
                v3 = acc[i][j][4 * gg + 3];
          // 16 x 16: take the values through vector registers.  (Stored
          // straight from the accumulator registers, they led the register
          // allocator to give most MFMAs of the loop a separate destination
          // and copy every accumulator each stage.)
          asm("" : "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3));
          if constexpr (Op::SCALED) sc.apply(fp[gg], j, v0, v1, v2, v3);
          store4<Op>(a, q, p, v0, v1, v2, v3);
        }
      }
      // (Keeps the factor loads of later row tiles from being hoisted here,
      // where the next tile's fragments already hold most registers.)
      if constexpr (Op::SCALED) __builtin_amdgcn_sched_barrier(0);
    }
  };
  zero_acc();
  for (int s = 0; s < nst; ++s) {
    if constexpr (Cfg::ROLL) stage_roll(s, s, cur, none, p1);
    else stage(s, s, cur, p1);
  }
  // Copies issued past the tile read zeros; let them land before the LDS is
  // reused and before exit.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  // End stamp of the clock trace at the end of the stage loop (the clock
  // over the loop; nothing of the trace stays live into the epilogue).
  stamp(2);
  if constexpr (Cfg::STAGED_EPI) {
    // The stage buffers are free for an LDS-staged epilogue once every wave
    // is past its last read.
    __syncthreads();
    int64_t tp, tq;
    tile_map(a.tiles_p, a.tiles_q, a.group, tile, &tp, &tq);
    static_assert(!Cfg::STAGED_EPI || Cfg::WTQ * 256 * NW <= 2 * Cfg::STAGE, "staging fits in the stage buffers");
    staged_epilogue<Op, Cfg::WTP, Cfg::WTQ, TP, TQ, MT, Acc>(a, smem + wave_u * (Cfg::WTQ * 256), acc, lane_id(),
                                                             tp * Cfg::BP + wp * Cfg::WTP, tq * Cfg::BQ + wq * Cfg::WTQ);
  } else {
    direct_epilogue(tile);
  }
}

// KT: some stage ends inside K (K not a multiple of the stage depth), so
// the copies carry per-lane tail masks.
template <class Op, bool PKM, int BP, int BQ, int NS, bool KT>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(TnCfg<Op, PKM, BP, BQ, NS>::WPE, TnCfg<Op, PKM, BP, BQ, NS>::WPE)))
gemm_tn_kernel(const GemmArgs a) {
  gemm_tn_body<Op, PKM, BP, BQ, NS, KT>(a);
}

}  // namespace dg
