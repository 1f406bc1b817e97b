// libdgemm.so: the C ABI declared in include/dgemm.h.
//
// Host side of every call: validate the arguments, map (A, B, C, layout) onto
// the kernels' (P, Q, D) form, pick a tile configuration, and launch on the
// caller's stream.  No allocation, no synchronisation; the only state is a
// thread-local copy of the last HIP error code.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dgemm.h"
#include "common.hpp"
#include "gemm_f32.hpp"
#include "gemm_mfma.hpp"
#include "gemm_skinny.hpp"
#include "launch.hpp"

namespace dg {
namespace {

// hipError_t behind the calling thread's most recent DGEMM_ERR_HIP.
thread_local int g_last_hip_error = 0;

// Clock trace buffer of the calling thread (dgemm_trace_clock), passed to
// the four-wave kernels of its later calls.
thread_local unsigned long long* g_trace = nullptr;
thread_local int64_t g_trace_n = 0;

int hip_failed(hipError_t e) {
  g_last_hip_error = (int)e;
  return DGEMM_ERR_HIP;
}

// DT_FP8S: FP8 with scale factors (gemm_fp8_scaled); DT_MX8: MXFP8 with
// E8M0 block scales (gemm_mxfp8).
enum Dtype { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_FP8 = 3, DT_FP8S = 4, DT_MX8 = 5 };

bool is_fp8(int dt) { return dt == DT_FP8 || dt == DT_FP8S || dt == DT_MX8; }

constexpr int64_t kMaxDescBytes = (int64_t(1) << 31) - 64;

int in_elem(int dt) { return dt == DT_F32 ? 4 : (is_fp8(dt) ? 1 : 2); }
int out_elem(int dt) { return (dt == DT_F32 || is_fp8(dt)) ? 4 : 2; }

// ---- kernel table ------------------------------------------------------------
// 16-bit and FP8: 256 x 256 block tile, 8 waves as 2 (p) x 4 (q), wave tile
// 128 x 64 (4 x 2 MFMA tiles of 32 x 32), 128 bytes of K per stage, two LDS
// buffers (128 KiB).
// FP32: 128 x 128 block tile, 4 waves as 2 x 2, wave tile 64 x 64, K = 32 per
// stage, two buffers (64-68 KiB, so two workgroups fit one CU).

template <class Op, bool PT>
Launch mfma_launch(const char* name) {
  using Cfg = MfmaCfg<Op, 256, 256, 2, 4, PT>;
  return Launch{(const void*)&gemm_mfma_kernel<Op, 256, 256, 2, 4, PT>, name, 256, 256, Cfg::NT,
                2 * Cfg::STAGE, PT};
}

// Whether K ends inside a stage of the four-wave kernel (stages of 128 bytes
// of k).
bool k_tail(int dt, int64_t K) { return K % (128 / in_elem(dt)) != 0; }

// Block tiles of the four-wave kernel and their throughput relative to the
// 256 x 256 tile when every CU is busy, measured on MI355X at 8192^3 class
// sizes (bf16 and fp8 TN; 128 x 128 runs two workgroups per CU): smaller
// tiles re-read more of A and B per flop and give each wave fewer MFMAs per
// fragment read, but fill the CUs when the problem has few tiles. With these
// rates 128 x 128 never loses to 256 x 128, so the latter serves only FP8
// with p-contiguous P, whose transposing-read swizzle needs 256-byte rows.
// 128 x 128 comes twice: two workgroups per CU with two LDS stages, or one
// with four stages, whose copies run three stages ahead.  The four-stage
// tile is only taken when all its tiles fit one round (at most one per CU):
// there it beats the two-stage one (bf16 2048^3: 678 against 563 TF/s,
// 1536 x 1536 x 8192: 586 against 453), with more rounds it loses (bf16
// 4352 x 4352 x 1024: 550 against 649; 8192^3 forced: 926 against 1012).
// Its rate is the one measured at one round.
// 192 x 256 (TN: wave tile 96 x 128, direct epilogue) fills a round
// where 256 x 256 leaves CUs idle: bf16 3072 x 4096 x 8192 has 192 tiles of
// 256 x 256 and 256 of 192 x 256 (1152 -> 1256 TF/s; 1536 x 8192 x 8192
// 1274 -> 1383); over whole rounds it runs at 0.87 of 256 x 256 (bf16
// 6144 x 8192 x 8192: 1302 against 1495); 256 x 192 does the same along q
// (bf16 4096 x 3072 x 8192 1209 -> 1374, 8192 x 1536 x 8192 1278 -> 1436;
// fp8 2162 -> 2458, 2302 -> 2596).  Both are offered for one round only
// (over two or three rounds they gained or lost a few percent against the
// 256 x 256 grid or its split: bf16 3072 x 8192 x 8192 +4%, 1536 x 14336 x
// 8192 -4%, 2560 x 14336 x 8192 -7%) and from K = 4096 on:
// at short K its direct epilogue weighs more, and as the second launch of a
// split it lost (bf16 5120 x 5120 x 1024: 915 against 959; 4352 x 6144 x
// 1024: 933 against 989), while at K = 4096 and up it won (3072 x 4096:
// +10%, 1024 x 10240 x 4096: +10%, 3584 x 8192 x 8192 as a split: +1-2%).
// The choice minimises ceil(tiles / slots) * tile work / rate, i.e. the
// number of rounds of workgroups times the time of one round ("FP16 GEMM
// Optimization on AMD RDNA 3 and RDNA 4", Where That Leaves Us: no single
// tile is best on every shape).
struct TileChoice {
  int bp, bq, per_cu;   // tile, workgroups resident per CU
  double rate;          // CU throughput relative to 256 x 256
  int max_rounds;       // 0: any number of rounds
};
constexpr TileChoice kTiles[kNumTiles] = {{256, 256, 1, 1.00, 0},
                                          {256, 128, 1, 0.76, 0},
                                          {128, 128, 2, 0.78, 0},
                                          {128, 128, 1, 0.47, 1},
                                          {192, 256, 1, 0.87, 1},
                                          {256, 192, 1, 0.87, 1}};
constexpr int kPlanCus = 256;  // MI355X CUs, for the tile choice only

int pick_tile(int64_t Pn, int64_t Qn, unsigned allowed, double* cost = nullptr) {
  int best = -1;
  double best_t = 0.0;
  for (int i = 0; i < kNumTiles; ++i) {
    if (!(allowed >> i & 1u)) continue;
    const TileChoice& c = kTiles[i];
    const int64_t tiles = ((Pn + c.bp - 1) / c.bp) * ((Qn + c.bq - 1) / c.bq);
    const int64_t slots = (int64_t)kPlanCus * c.per_cu;
    const double rounds = (double)((tiles + slots - 1) / slots);
    if (c.max_rounds > 0 && rounds > c.max_rounds) continue;
    const double t = rounds * (double)c.bp * c.bq * c.per_cu / c.rate;
    if (best < 0 || t < best_t) { best = i; best_t = t; }
  }
  if (cost) *cost = best_t;
  return best;
}

// Tiles a four-wave variant allows: p-contiguous FP8 P keeps 256-wide rows
// (the transposing-read swizzle needs eight 32-byte units per row).
// MXFP8's scale ring needs two LDS stages, so it leaves out the four-stage
// tile.  192 x 256 and 256 x 192 are built for TN (where they were
// measured: fp8 3072 x 4096 x 8192 2155 -> 2423 TF/s, 1536 x 8192 x 8192
// 2307 -> 2573); NN, whose p-contiguous P keeps 256-wide rows, takes
// 256 x 192 only.
unsigned tile_mask(int dt, bool nn, int64_t K) {
  const unsigned t192 = K < 4096 ? 0u : (nn ? 0b100000u : 0b110000u);
  if (nn && is_fp8(dt)) return 0b0011u | t192;
  return (dt == DT_MX8 ? 0b0101u : 0b1101u) | t192;
}

template <bool PT, int BT>
Launch f32_launch(const char* name) {
  using Cfg = F32Cfg<BT, BT, 2, 2, PT>;
  return Launch{(const void*)&gemm_f32_kernel<BT, BT, 2, 2, PT>, name, BT, BT, Cfg::NT, 2 * Cfg::STAGE, PT};
}

// FP32 tile: 128 x 128 (four waves of 64 x 64) once the grid has at least
// half as many tiles as there are CUs; below that 64 x 64 (four waves of
// 32 x 32), four times the workgroups.  A 256^3 product is 4 workgroups at
// 128 x 128, each a full K loop on one CU, against 16 at 64 x 64.
Launch f32_tile(bool nn, bool small) {
  if (small) return nn ? f32_launch<true, 64>("f32_nn_64x64") : f32_launch<false, 64>("f32_tn_64x64");
  return nn ? f32_launch<true, 128>("f32_nn_128x128") : f32_launch<false, 128>("f32_tn_128x128");
}

template <class Op, int PF>
Launch skinny_launch(const char* name) {
  return Launch{(const void*)&gemm_skinny_kernel<Op, PF>, name, 16 * PF, SkinnyCfg<Op, PF>::BQ, SkinnyCfg<Op, PF>::NT,
                (int)SkinnyCfg<Op, PF>::LDS, false};
}

// Skinny TN problems (at most 32 rows of A) stream B once with a split-K
// kernel; everything else uses the block-tiled kernels.
bool use_skinny(int dt, int layout, int64_t M) {
  return layout == DGEMM_TN && (dt == DT_F16 || dt == DT_BF16) && M <= 32;
}

Launch select_skinny(int dt, int64_t M) {
  if (dt == DT_F16) return M <= 16 ? skinny_launch<OpF16, 1>("f16_tn_skinny16") : skinny_launch<OpF16, 2>("f16_tn_skinny32");
  return M <= 16 ? skinny_launch<OpBF16, 1>("bf16_tn_skinny16") : skinny_launch<OpBF16, 2>("bf16_tn_skinny32");
}

// The four-wave kernel (gemm_tn.hpp) for kTiles entry `idx` (one tile_mask
// allows); its instantiations live in four_wave.hip, one translation unit
// per format and layout.
Launch four_wave(int dt, bool nn, int idx, bool kt) {
  switch (dt) {
    case DT_F16: return nn ? four_wave_f16_nn(idx, kt) : four_wave_f16_tn(idx, kt);
    case DT_BF16: return nn ? four_wave_bf16_nn(idx, kt) : four_wave_bf16_tn(idx, kt);
    case DT_FP8S: return nn ? four_wave_fp8s_nn(idx, kt) : four_wave_fp8s_tn(idx, kt);
    case DT_MX8: return nn ? four_wave_mx8_nn(idx, kt) : four_wave_mx8_tn(idx, kt);
    default: return nn ? four_wave_fp8_nn(idx, kt) : four_wave_fp8_tn(idx, kt);
  }
}

// The kernel for kTiles entry `idx`: TN 256 x 256 tiles of FP16, BF16 and
// FP8 (with or without scale factors) run the eight-wave ping-pong kernel
// (gemm_pp.hpp; at 8192^3 on one box: FP8 2648 -> 2859 TF/s, BF16 1513 ->
// 1550, FP16 1437 -> 1473, against the four-wave kernel); everything else
// the four-wave kernel.
Launch main_tile(int dt, bool nn, int idx, bool kt) {
  if (idx == 0 && !nn && dt != DT_MX8)
    return ping_pong_tn(dt == DT_F16 ? 0 : dt == DT_BF16 ? 1 : dt == DT_FP8 ? 2 : 3, kt);
  return four_wave(dt, nn, idx, kt);
}

// The kernels of one call: a main launch, and optionally a second one over
// the rest of one axis, p >= at (split_p) or q >= at.
struct Choice {
  Launch L;
  bool split;
  bool split_p;
  int64_t at;
  Launch T;
};

// When the 256 x 256 grid ends in a partial round, the call can run the
// whole rounds with 256 x 256 tiles over the first part of the p or the q
// range and the rest as a second launch with the tile the table picks for
// it (e.g. bf16 6144^2 x 4096: 1032 -> 1157 TF/s, fp8 8192 x 5120 x 8192:
// 2287 -> 2540 TF/s).  Taken when the cost model (rounds x round time, as
// pick_tile) gains at least 5%.
// Sweeps and A/B timing: DGEMM_CONFIG=<kernel name>, as dgemm_kernel_config
// prints it, forces that kernel (one launch, no split) for every call it
// can serve: a four-wave tile of the call's format and layout, or the
// eight-wave ping-pong kernel for TN.  Other calls keep the table's choice.
// Read at every call; nothing is cached.
bool forced_choice(int dt, bool nn, int64_t K, Choice* c) {
  const char* want = getenv("DGEMM_CONFIG");
  if (want == nullptr || *want == 0) return false;
  if (dt == DT_F32) {
    for (int small = 0; small < 2; ++small) {
      const Launch L = f32_tile(nn, small != 0);
      if (strcmp(L.name, want) == 0) {
        c->L = L;
        return true;
      }
    }
    return false;
  }
  const int e = in_elem(dt);
  if (!(dt == DT_MX8 || (dt != DT_F32 && K % (16 / e) == 0 && K >= 2 * (128 / e)))) return false;
  const bool kt = k_tail(dt, K);
  for (int idx = 0; idx < kNumTiles; ++idx) {
    const Launch L = four_wave(dt, nn, idx, kt);
    if (strcmp(L.name, want) == 0) {
      c->L = L;
      return true;
    }
  }
  if (!nn && dt != DT_MX8) {
    const Launch L = ping_pong_tn(dt == DT_F16 ? 0 : dt == DT_BF16 ? 1 : dt == DT_FP8 ? 2 : 3, kt);
    if (strcmp(L.name, want) == 0) {
      c->L = L;
      return true;
    }
  }
  return false;
}

Choice choose(int dt, int layout, int64_t M, int64_t N, int64_t K) {
  const bool nn = layout == DGEMM_NN;
  const int64_t Pn = nn ? N : M, Qn = nn ? M : N;
  Choice c{};
  if (dt == DT_MX8) {
    // MXFP8 (K a multiple of 32) takes the four-wave kernel; below two
    // stages only the one-tile-per-workgroup tiles.  K == 0 (C = 0, no
    // scale is read) goes to the eight-wave kernel's zero fill.
    if (K == 0) {
      c.L = nn ? mfma_launch<OpFP8, true>("fp8_nn_256x256") : mfma_launch<OpFP8, false>("fp8_tn_256x256");
      return c;
    }
    if (K < 256) {
      c.L = four_wave(dt, nn, nn ? 1 : 2, k_tail(dt, K));
      return c;
    }
  }
  // K a whole number of 16-byte chunks and at least two stages: the
  // four-wave kernel (gemm_tn.hpp), tile chosen by shape; NN reads B with
  // transposing LDS reads.
  const int e = in_elem(dt);
  if (dt == DT_MX8 || (dt != DT_F32 && K % (16 / e) == 0 && K >= 2 * (128 / e))) {
    const unsigned mask = tile_mask(dt, nn, K);
    double whole = 0.0;
    const int idx = pick_tile(Pn, Qn, mask, &whole);
    c.L = main_tile(dt, nn, idx, k_tail(dt, K));
    const int64_t slots = kPlanCus;
    const int64_t tp = (Pn + 255) / 256, tq = (Qn + 255) / 256, tiles = tp * tq;
    double best = 0.95 * whole;
    // A last round of 256 x 256 tiles at least half full runs at a higher
    // clock than a full one (fewer CUs under the power limit) and costs
    // less than the round model says: measured, a single launch beat the
    // split or tied it at 1.5 and 3.5 rounds (bf16 5120^2 x 4096 1356 vs
    // 1308 TF/s, fp8 2362 vs 2211; 4096 x 14336 x 4096 1404 vs 1397, fp8
    // 2501 vs 2484; 8192 x 5120 x 4096 1400 vs 1384), while the split won
    // with a last round a quarter full or less (4352^2 x 4096 1205 vs 1007,
    // 6144^2 x 4096 1307 vs 1256, 7168^2 x 4096 1368 vs 1251).
    // (Measured with the eight-wave TN kernel as the main launch; with the
    // four-wave one (NN, MXFP8) the split also paid at 2.5 rounds: fp8
    // 8192 x 5120 x 8192 2287 -> 2455-2540.)
    const bool pp_main = !nn && dt != DT_MX8;
    const bool consider = tiles % slots != 0 && (!pp_main || 2 * (tiles % slots) < slots);
    for (int axis = 0; axis < 2 && consider; ++axis) {
      // axis 0 splits q, axis 1 splits p: n1 whole tiles of the split axis
      // fit the full rounds.
      const int64_t across = axis == 0 ? tp : tq, along = axis == 0 ? tq : tp;
      const int64_t n1 = (tiles / slots) * slots / across;
      if (n1 < 1 || n1 >= along) continue;
      double tail = 0.0;
      const int tidx = axis == 0 ? pick_tile(Pn, Qn - 256 * n1, mask, &tail)
                                 : pick_tile(Pn - 256 * n1, Qn, mask, &tail);
      const double cost = (double)((across * n1 + slots - 1) / slots) * 65536.0 + tail;
      if (cost < best) {
        best = cost;
        c.L = main_tile(dt, nn, 0, k_tail(dt, K));
        c.split = true;
        c.split_p = axis == 1;
        c.at = 256 * n1;
        c.T = four_wave(dt, nn, tidx, k_tail(dt, K));
      }
    }
    return c;
  }
  switch (dt) {
    case DT_F32:  c.L = f32_tile(nn, ((Pn + 127) / 128) * ((Qn + 127) / 128) < kPlanCus / 2); break;
    case DT_F16:  c.L = nn ? mfma_launch<OpF16, true>("f16_nn_256x256") : mfma_launch<OpF16, false>("f16_tn_256x256"); break;
    case DT_BF16: c.L = nn ? mfma_launch<OpBF16, true>("bf16_nn_256x256") : mfma_launch<OpBF16, false>("bf16_tn_256x256"); break;
    case DT_FP8S: c.L = nn ? mfma_launch<OpFP8S, true>("fp8s_nn_256x256") : mfma_launch<OpFP8S, false>("fp8s_tn_256x256"); break;
    default:      c.L = nn ? mfma_launch<OpFP8, true>("fp8_nn_256x256") : mfma_launch<OpFP8, false>("fp8_tn_256x256"); break;
  }
  return c;
}

struct Plan {
  Launch L;
  GemmArgs g;
  int64_t grid;
  bool split;      // a second launch over p or q >= the split point
  bool split_p;
  Launch L2;
  GemmArgs g2;
  int64_t grid2;
};

// Scale factors of gemm_fp8_scaled: na values at sa (1 or M), nb at sb (1 or N).
struct Scales {
  const float* sa;
  int64_t na;
  const float* sb;
  int64_t nb;
};

// E8M0 block scales of gemm_mxfp8: row i of A has K/32 bytes at sa + i*ldsa,
// column j of B K/32 bytes at sb + j*ldsb.
struct MxScales {
  const uint8_t* sa;
  int64_t ldsa;
  const uint8_t* sb;
  int64_t ldsb;
};

// p + n, leaving a null pointer null (the host-only planning helpers plan
// without operands).
template <class T>
T* advance(T* p, int64_t n) {
  return p ? p + n : p;
}

// Validation in the documented order, then the (P, Q, D) mapping.
int plan(int dt, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
         void* C, int64_t ldc, int layout, Plan* out, bool check_pointers, const Scales* sc = nullptr,
         const MxScales* mx = nullptr) {
  if (layout != DGEMM_NN && layout != DGEMM_TN) return DGEMM_ERR_INVALID_LAYOUT;
  if (M < 0 || N < 0 || K < 0) return DGEMM_ERR_INVALID_DIM;
  if (sc && ((sc->na != 1 && sc->na != M) || (sc->nb != 1 && sc->nb != N))) return DGEMM_ERR_INVALID_DIM;
  if (dt == DT_MX8 && K % 32 != 0) return DGEMM_ERR_INVALID_DIM;
  out->split = false;
  if (M == 0 || N == 0) { out->grid = 0; return DGEMM_OK; }
  if (check_pointers && ((K > 0 && (A == nullptr || B == nullptr)) || C == nullptr)) return DGEMM_ERR_NULL_POINTER;
  if (check_pointers && sc && (sc->sa == nullptr || sc->sb == nullptr)) return DGEMM_ERR_NULL_POINTER;
  if (check_pointers && mx && K > 0 && (mx->sa == nullptr || mx->sb == nullptr)) return DGEMM_ERR_NULL_POINTER;
  const bool nn = layout == DGEMM_NN;
  const int64_t min_lda = K > 0 ? K : 1;
  const int64_t min_ldb = nn ? N : (K > 0 ? K : 1);
  const int64_t min_ldc = nn ? N : M;
  if (lda < min_lda || ldb < min_ldb || ldc < min_ldc) return DGEMM_ERR_INVALID_LD;
  if (mx && (mx->ldsa < K / 32 || mx->ldsb < K / 32)) return DGEMM_ERR_INVALID_LD;
  const int e = in_elem(dt);
  if (check_pointers && K > 0 &&
      ((((uintptr_t)A) & 15) != 0 || (((uintptr_t)B) & 15) != 0 || ((lda * e) & 15) != 0 || ((ldb * e) & 15) != 0))
    return DGEMM_ERR_MISALIGNED;
  if (((uintptr_t)C) % (uintptr_t)out_elem(dt) != 0) return DGEMM_ERR_MISALIGNED;
  if (sc && ((((uintptr_t)sc->sa) & 3) != 0 || (((uintptr_t)sc->sb) & 3) != 0)) return DGEMM_ERR_MISALIGNED;
  if (mx && K > 0 &&
      ((((uintptr_t)mx->sa) & 15) != 0 || (((uintptr_t)mx->sb) & 15) != 0 || (mx->ldsa & 15) != 0 ||
       (mx->ldsb & 15) != 0))
    return DGEMM_ERR_MISALIGNED;

  Choice ch{};
  const bool forced = forced_choice(dt, layout == DGEMM_NN, K, &ch);
  const bool skinny = !forced && use_skinny(dt, layout, M);
  if (skinny) ch.L = select_skinny(dt, M);
  else if (!forced) ch = choose(dt, layout, M, N, K);
  const Launch L = ch.L;
  GemmArgs g{};
  if (!nn) {
    g.P = (const char*)A; g.ldp = lda * e; g.Pn = M;
    g.Q = (const char*)B; g.ldq = ldb * e; g.Qn = N;
  } else {
    g.P = (const char*)B; g.ldp = ldb * e; g.Pn = N;
    g.Q = (const char*)A; g.ldq = lda * e; g.Qn = M;
  }
  g.C = C; g.ldc = ldc; g.K = K;
  g.trace = g_trace;
  g.trace_n = g_trace_n;
  if (sc) {
    // Factor vectors are addressed through buffer descriptors in bytes.
    if (sc->na * 4 > kMaxDescBytes || sc->nb * 4 > kMaxDescBytes) return DGEMM_ERR_UNSUPPORTED;
    g.sp = nn ? sc->sb : sc->sa;
    g.sp_row = (nn ? sc->nb : sc->na) > 1 ? 1 : 0;
    g.sq = nn ? sc->sa : sc->sb;
    g.sq_row = (nn ? sc->na : sc->nb) > 1 ? 1 : 0;
  }
  if (mx) {
    // A tile's block scales are addressed through one descriptor in bytes.
    if (256 * mx->ldsa > kMaxDescBytes || 256 * mx->ldsb > kMaxDescBytes) return DGEMM_ERR_UNSUPPORTED;
    g.msp = nn ? mx->sb : mx->sa;
    g.ldsp = nn ? mx->ldsb : mx->ldsa;
    g.msq = nn ? mx->sa : mx->sb;
    g.ldsq = nn ? mx->ldsa : mx->ldsb;
  }
  // Descriptor ranges must stay below 2^31 bytes.
  for (const Launch* l : {&ch.L, &ch.T}) {
    if (l == &ch.T && !ch.split) break;
    if ((int64_t)l->bq * g.ldq > kMaxDescBytes) return DGEMM_ERR_UNSUPPORTED;
    if (!l->p_trans && (int64_t)l->bp * g.ldp > kMaxDescBytes) return DGEMM_ERR_UNSUPPORTED;
    if (l->p_trans && K * g.ldp > kMaxDescBytes) return DGEMM_ERR_UNSUPPORTED;
  }
  if (K * e > kMaxDescBytes) return DGEMM_ERR_UNSUPPORTED;
  g.group = 8;
  const int oe = out_elem(dt);
  g.vec_store = ((((uintptr_t)C) % (uintptr_t)(4 * oe)) == 0 && ((ldc * oe) % (4 * oe)) == 0) ? 1 : 0;
  g.vec16 = ((((uintptr_t)C) % 16) == 0 && ((ldc * oe) % 16) == 0) ? 1 : 0;
  if (ch.split) {
    // The second launch covers q >= at (rows of Q and of the factor / scale
    // arrays along q, columns of D) or p >= at (rows of P -- for
    // p-contiguous P its columns --, factors along p, rows of D).
    GemmArgs g2 = g;
    g2.trace = nullptr;   // the trace records the main launch
    const int64_t x0 = ch.at;
    if (!ch.split_p) {
      g2.Q = advance(g.Q, x0 * g.ldq);
      g2.C = advance((char*)C, x0 * ldc * oe);
      g2.Qn = g.Qn - x0;
      if (g.sq && g.sq_row) g2.sq = g.sq + x0;
      if (g.msq) g2.msq = g.msq + x0 * g.ldsq;
      g.Qn = x0;
    } else {
      g2.P = advance(g.P, ch.L.p_trans ? x0 * e : x0 * g.ldp);
      g2.C = advance((char*)C, x0 * oe);
      g2.Pn = g.Pn - x0;
      if (g.sp && g.sp_row) g2.sp = g.sp + x0;
      if (g.msp) g2.msp = g.msp + x0 * g.ldsp;
      g.Pn = x0;
    }
    g2.tiles_p = (g2.Pn + ch.T.bp - 1) / ch.T.bp;
    g2.tiles_q = (g2.Qn + ch.T.bq - 1) / ch.T.bq;
    out->split = true;
    out->split_p = ch.split_p;
    out->L2 = ch.T;
    out->g2 = g2;
    out->grid2 = g2.tiles_p * g2.tiles_q;
    if (out->grid2 > 0x7fffffff) return DGEMM_ERR_UNSUPPORTED;
  }
  g.tiles_p = skinny ? 1 : (g.Pn + L.bp - 1) / L.bp;
  g.tiles_q = (g.Qn + L.bq - 1) / L.bq;
  out->L = L;
  out->g = g;
  out->grid = g.tiles_p * g.tiles_q;
  if (out->grid > 0x7fffffff) return DGEMM_ERR_UNSUPPORTED;
  return DGEMM_OK;
}

// One launch on the caller's stream.
int launch(const Launch& L, const GemmArgs& g, int64_t grid, void* stream) {
  GemmArgs arg = g;
  void* args[] = {(void*)&arg};
  const hipError_t err = hipLaunchKernel(L.fn, dim3((unsigned)grid), dim3(L.threads), args, 0, (hipStream_t)stream);
  if (err != hipSuccess) return hip_failed(err);
  return DGEMM_OK;
}

int run(int dt, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
        void* C, int64_t ldc, int layout, void* stream, const Scales* sc = nullptr, const MxScales* mx = nullptr) {
  Plan pl;
  const int st = plan(dt, M, N, K, A, lda, B, ldb, C, ldc, layout, &pl, true, sc, mx);
  if (st != DGEMM_OK || pl.grid == 0) return st;
  const int r = launch(pl.L, pl.g, pl.grid, stream);
  if (r != DGEMM_OK || !pl.split) return r;
  return launch(pl.L2, pl.g2, pl.grid2, stream);
}

}  // namespace
}  // namespace dg

extern "C" {

int dgemm_trace_clock(unsigned long long* buf, int64_t n_workgroups) {
  if (buf != nullptr && n_workgroups < 0) return DGEMM_ERR_INVALID_DIM;
  dg::g_trace = buf;
  dg::g_trace_n = buf ? n_workgroups : 0;
  return DGEMM_OK;
}

int gemm_f32(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B, int64_t ldb, float* C,
             int64_t ldc, int layout, void* stream) {
  return dg::run(dg::DT_F32, M, N, K, A, lda, B, ldb, C, ldc, layout, stream);
}

int gemm_f16(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
             uint16_t* C, int64_t ldc, int layout, void* stream) {
  return dg::run(dg::DT_F16, M, N, K, A, lda, B, ldb, C, ldc, layout, stream);
}

int gemm_bf16(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
              uint16_t* C, int64_t ldc, int layout, void* stream) {
  return dg::run(dg::DT_BF16, M, N, K, A, lda, B, ldb, C, ldc, layout, stream);
}

int gemm_fp8(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
             float* C, int64_t ldc, int layout, void* stream) {
  return dg::run(dg::DT_FP8, M, N, K, A, lda, B, ldb, C, ldc, layout, stream);
}

int gemm_fp8_scaled(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                    float* C, int64_t ldc, const float* scale_a, int64_t n_scale_a, const float* scale_b,
                    int64_t n_scale_b, int layout, void* stream) {
  const dg::Scales sc{scale_a, n_scale_a, scale_b, n_scale_b};
  return dg::run(dg::DT_FP8S, M, N, K, A, lda, B, ldb, C, ldc, layout, stream, &sc);
}

int gemm_mxfp8(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
               float* C, int64_t ldc, const uint8_t* scale_a, int64_t ldsa, const uint8_t* scale_b, int64_t ldsb,
               int layout, void* stream) {
  const dg::MxScales mx{scale_a, ldsa, scale_b, ldsb};
  return dg::run(dg::DT_MX8, M, N, K, A, lda, B, ldb, C, ldc, layout, stream, nullptr, &mx);
}

const char* gemm_strerror(int status) {
  switch (status) {
    case DGEMM_OK: return "success";
    case DGEMM_ERR_INVALID_DIM: return "invalid dimension (M, N or K negative)";
    case DGEMM_ERR_NULL_POINTER: return "null operand pointer";
    case DGEMM_ERR_INVALID_LD: return "leading dimension below its minimum";
    case DGEMM_ERR_INVALID_LAYOUT: return "layout is neither DGEMM_NN nor DGEMM_TN";
    case DGEMM_ERR_MISALIGNED: return "operand base or pitch not 16-byte aligned";
    case DGEMM_ERR_UNSUPPORTED: return "problem exceeds the supported size limits";
    case DGEMM_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int dgemm_last_hip_error(void) { return dg::g_last_hip_error; }

const char* dgemm_hip_error_string(int code) { return hipGetErrorString((hipError_t)code); }

int dgemm_tile_map(int64_t tiles_p, int64_t tiles_q, int64_t group, int64_t pid, int64_t* tile_p, int64_t* tile_q) {
  if (tiles_p <= 0 || tiles_q <= 0 || group <= 0 || pid < 0 || pid >= tiles_p * tiles_q || !tile_p || !tile_q)
    return -1;
  dg::tile_map(tiles_p, tiles_q, group, pid, tile_p, tile_q);
  return 0;
}

int64_t dgemm_lds_bytes(int bm, int bn, int bk, int elem, int pad_bytes, int buffers) {
  if (bm < 0 || bn < 0 || bk < 0 || elem < 0 || pad_bytes < 0 || buffers < 0) return -1;
  return dg::lds_bytes(bm, bn, bk, elem, pad_bytes, buffers);
}

int dgemm_kernel_config(int dtype, int layout, int64_t M, int64_t N, int64_t K, char* buf, int64_t len) {
  if (dtype < 0 || dtype > 5) return DGEMM_ERR_UNSUPPORTED;
  const int e = dg::in_elem(dtype);
  const bool nn = layout == DGEMM_NN;
  // Minimal legal, aligned leading dimensions for the description.
  int64_t lda = K > 0 ? K : 1, ldb = nn ? N : (K > 0 ? K : 1);
  const int64_t al = 16 / e;
  lda = (lda + al - 1) / al * al;
  ldb = (ldb + al - 1) / al * al;
  dg::Plan pl;
  const int st = dg::plan(dtype, M, N, K, nullptr, lda, nullptr, ldb, nullptr, nn ? N : M, layout, &pl, false);
  if (st != DGEMM_OK) return st;
  if (buf && len > 0) {
    if (pl.grid == 0)
      snprintf(buf, (size_t)len, "none (empty output)");
    else if (!pl.split)
      snprintf(buf, (size_t)len, "%s tile=%dx%d threads=%d lds=%d grid=%lld tiles=%lldx%lld group=%lld",
               pl.L.name, pl.L.bp, pl.L.bq, pl.L.threads, pl.L.lds, (long long)pl.grid, (long long)pl.g.tiles_p,
               (long long)pl.g.tiles_q, (long long)pl.g.group);
    else
      snprintf(buf, (size_t)len,
               "%s tile=%dx%d threads=%d lds=%d grid=%lld tiles=%lldx%lld group=%lld"
               " + %s tile=%dx%d lds=%d grid=%lld tiles=%lldx%lld from %c=%lld",
               pl.L.name, pl.L.bp, pl.L.bq, pl.L.threads, pl.L.lds, (long long)pl.grid, (long long)pl.g.tiles_p,
               (long long)pl.g.tiles_q, (long long)pl.g.group, pl.L2.name, pl.L2.bp, pl.L2.bq, pl.L2.lds,
               (long long)pl.grid2, (long long)pl.g2.tiles_p, (long long)pl.g2.tiles_q, pl.split_p ? 'p' : 'q',
               (long long)(pl.split_p ? pl.g.Pn : pl.g.Qn));
  }
  return DGEMM_OK;
}

}  // extern "C"
