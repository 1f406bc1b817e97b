// Launch descriptors shared by the host dispatch (dgemm.hip) and the
// translation units that instantiate the four-wave kernels
// (four_wave.hip, compiled once per format and layout).
#pragma once

#include "common.hpp"

namespace dg {

// A launchable configuration: a kernel symbol plus its tile geometry.  Every
// kernel runs one workgroup per tile.
struct Launch {
  const void* fn;
  const char* name;
  int bp, bq, threads, lds;
  bool p_trans;
};

// Entries of the block-tile table of the four-wave kernel (dgemm.hip,
// kTiles): 0 256x256, 1 256x128, 2 128x128 (two workgroups per CU),
// 3 128x128 with four LDS stages, 4 192x256, 5 256x192.
constexpr int kNumTiles = 6;

// The four-wave launch of table entry `idx` for one input format and layout
// (`kt`: K ends inside a stage, so the copies need tail masks).  Entries a
// variant does not build fall back to 256 x 256 (the table masks them out).
Launch four_wave_f16_tn(int idx, bool kt);
Launch four_wave_f16_nn(int idx, bool kt);
Launch four_wave_bf16_tn(int idx, bool kt);
Launch four_wave_bf16_nn(int idx, bool kt);
Launch four_wave_fp8_tn(int idx, bool kt);
Launch four_wave_fp8_nn(int idx, bool kt);
Launch four_wave_fp8s_tn(int idx, bool kt);
Launch four_wave_fp8s_nn(int idx, bool kt);
Launch four_wave_mx8_tn(int idx, bool kt);
Launch four_wave_mx8_nn(int idx, bool kt);

// The eight-wave ping-pong kernel (gemm_pp.hpp), TN, 256 x 256: op 0 FP16,
// 1 BF16, 2 FP8, 3 FP8 with scale factors.
Launch ping_pong_tn(int op, bool kt);

}  // namespace dg
