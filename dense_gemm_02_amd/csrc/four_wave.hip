// Instantiations of the four-wave kernel (gemm_tn.hpp) for one input format
// and layout, selected at compile time: DG_OP (OpF16, OpBF16, OpFP8, OpFP8S,
// OpMX8), DG_PKM (1: NN, B read through transposing LDS reads; 0: TN),
// DG_TAG (name prefix, e.g. bf16_tn) and DG_FN (the function launch.hpp
// declares for the pair).  One translation unit per pair lets the library
// build in parallel.
#include "gemm_tn.hpp"
#include "launch.hpp"

#ifndef DG_OP
#error "DG_OP, DG_PKM, DG_TAG and DG_FN select the instantiation"
#endif

#define DG_STR2(x) #x
#define DG_STR(x) DG_STR2(x)
#define DG_NAME(tile) DG_STR(DG_TAG) "_" tile

namespace dg {
namespace {

template <class Op, bool PKM, int BP, int BQ, int NS = 2>
Launch tn_launch(const char* name, bool kt) {
  using Cfg = TnCfg<Op, PKM, BP, BQ, NS>;
  const void* fn = kt ? (const void*)&gemm_tn_kernel<Op, PKM, BP, BQ, NS, true>
                      : (const void*)&gemm_tn_kernel<Op, PKM, BP, BQ, NS, false>;
  return Launch{fn, name, BP, BQ, Cfg::NT, Cfg::LDS, PKM};
}

}  // namespace

Launch DG_FN(int idx, bool kt) {
  using Op = DG_OP;
  constexpr bool PKM = DG_PKM != 0;
  if constexpr (PKM && Op::ELEM == 1) {
    // p-contiguous FP8 P keeps 256-wide rows (the transposing-read swizzle
    // needs eight 32-byte units per row).
    if (idx == 1) return tn_launch<Op, PKM, 256, 128>(DG_NAME("256x128_w4"), kt);
    if (idx == 5) return tn_launch<Op, PKM, 256, 192>(DG_NAME("256x192_w4"), kt);
    return tn_launch<Op, PKM, 256, 256>(DG_NAME("256x256_w4"), kt);
  } else {
    switch (idx) {
      case 4:
        if constexpr (!PKM) return tn_launch<Op, PKM, 192, 256>(DG_NAME("192x256_w4"), kt);
        [[fallthrough]];
      case 5: return tn_launch<Op, PKM, 256, 192>(DG_NAME("256x192_w4"), kt);
      case 2: return tn_launch<Op, PKM, 128, 128>(DG_NAME("128x128_w4"), kt);
      case 3:
        // The MX scale ring needs two LDS stages.
        if constexpr (!Op::MX) return tn_launch<Op, PKM, 128, 128, 4>(DG_NAME("128x128_w4_s4"), kt);
        [[fallthrough]];
      default: return tn_launch<Op, PKM, 256, 256>(DG_NAME("256x256_w4"), kt);
    }
  }
}

}  // namespace dg
