// FAST dequant-GEMM without a prepass: the kernel converts the caller's bf16
// x to fp16 in LDS as it arrives (tile_accumulate3's ONLINE form in
// gemm3_core.h), and a second launch on the same grid recomputes with SPLIT
// numerics any tile with a row outside that conversion's range. Same grid,
// layouts and arguments as the FAST GEMM (x16 holds the bf16 x, rowscale is
// unused); no fused epilogue.
#include "gemm3_core.h"

namespace ql {

hipError_t launch_gemm3_online(int bits, const Gemm3Args &a, hipStream_t stream) {
  if (a.glu || a.gate) return hipErrorInvalidValue;
  switch (bits) {
    case 2: return g3::launch3_bits<2, false, true>(a, stream);
    case 3: return g3::launch3_bits<3, false, true>(a, stream);
    case 4: return g3::launch3_bits<4, false, true>(a, stream);
    case 8: return g3::launch3_bits<8, false, true>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ql
