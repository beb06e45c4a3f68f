// SPLIT numerics of the large-M dequant-GEMM: bf16 x straight from the caller,
// each weight dequantized in fp32 (s*q + b, one rounding) and fed to the bf16
// MFMA as two bf16 terms hi + lo (see gemm3_core.h). Needs no activation
// prepass and no scratch memory unless K is split.
#include "gemm3_core.h"

namespace ql {

hipError_t launch_gemm4(int bits, const Gemm3Args &a, hipStream_t stream) {
  if (a.glu || a.gate) return hipErrorInvalidValue;  // the fused epilogues run on FAST numerics
  if (bits == 4) return g3::launch3_bits<4, true>(a, stream);
  if (bits == 8) return g3::launch3_bits<8, true>(a, stream);
  if (bits == 2) return g3::launch3_bits<2, true>(a, stream);
  if (bits == 3) return g3::launch3_bits<3, true>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ql
