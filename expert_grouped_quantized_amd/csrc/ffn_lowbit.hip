// ffn_lowbit.hip -- launches of the expert-grouped SwiGLU GEMMs for routed
// experts coded at 2, 3, 5, 6, 7 or 8 bits with one fp16 scale per 32 weights
// along K (TandemLLM roadmap, "A mixture-of-experts model, and what is left":
// MoE kernels over several code widths).  Same kernels as int4; only the
// weight tile and its dequantization differ (WTileP).
#include "ffn_kernels.h"

namespace moe {

template <int RF>
static hipError_t launch_fmt(const FfnArgs& a, hipStream_t s) {
  const int sf = a.n_shared ? a.shared_fmt : MOE_BF16;
  if (sf == MOE_BF16) return launch_pair<RF, MOE_BF16>(a, s);
  if (sf == MOE_I8_ROW) return launch_pair<RF, MOE_I8_ROW>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_ffn_lowbit(const FfnArgs& a, hipStream_t s) {
  switch (a.routed_fmt) {
    case MOE_I2_G32: return launch_fmt<MOE_I2_G32>(a, s);
    case MOE_I3_G32: return launch_fmt<MOE_I3_G32>(a, s);
    case MOE_I5_G32: return launch_fmt<MOE_I5_G32>(a, s);
    case MOE_I6_G32: return launch_fmt<MOE_I6_G32>(a, s);
    case MOE_I7_G32: return launch_fmt<MOE_I7_G32>(a, s);
    case MOE_I8_G32: return launch_fmt<MOE_I8_G32>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
