// Instantiations of the eight-wave ping-pong kernel (gemm_pp.hpp): TN, 256 x
// 256 block tile, FP16, BF16, FP8 and FP8 with scale factors, with and
// without K-tail masks.
#include "gemm_pp.hpp"
#include "launch.hpp"

namespace dg {
namespace {

template <class Op>
Launch pp_launch(const char* name, bool kt) {
  using Cfg = PpCfg<Op>;
  const void* fn = kt ? (const void*)&gemm_pp_kernel<Op, true> : (const void*)&gemm_pp_kernel<Op, false>;
  return Launch{fn, name, Cfg::BP, Cfg::BQ, Cfg::NT, Cfg::LDS, false};
}

}  // namespace

Launch ping_pong_tn(int op, bool kt) {
  switch (op) {
    case 0: return pp_launch<OpF16>("f16_tn_256x256_pp", kt);
    case 1: return pp_launch<OpBF16>("bf16_tn_256x256_pp", kt);
    case 2: return pp_launch<OpFP8>("fp8_tn_256x256_pp", kt);
    default: return pp_launch<OpFP8S>("fp8s_tn_256x256_pp", kt);
  }
}

}  // namespace dg
