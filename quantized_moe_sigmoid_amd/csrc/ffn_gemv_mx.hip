// ffn_gemv_mx.hip — the expert GEMVs for MXFP4 weights (E2M1 codes, one E8M0 scale
// per 32 inputs), instantiated from ffn_gemv_impl.h.
#include "ffn_gemv_impl.h"

namespace coli {

hipError_t launch_gemv_mx(int mode, const FfnArgs &a, hipStream_t s) {
  if (mode == MODE_GATEUP) return launch_mode<W_MX, MODE_GATEUP, true>(a, s);
  return launch_mode<W_MX, MODE_DOWN, true>(a, s);
}

}  // namespace coli
