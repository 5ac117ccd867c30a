// ffn_gemv_w8.hip — the expert GEMVs for int8 weights (one scale per row, or
// group scales), instantiated from ffn_gemv_impl.h.
#include "ffn_gemv_impl.h"

namespace coli {

hipError_t launch_gemv_w8(int mode, bool gs, const FfnArgs &a, hipStream_t s) {
  if (mode == MODE_GATEUP)
    return gs ? launch_mode<8, MODE_GATEUP, true>(a, s) : launch_mode<8, MODE_GATEUP, false>(a, s);
  return gs ? launch_mode<8, MODE_DOWN, true>(a, s) : launch_mode<8, MODE_DOWN, false>(a, s);
}

}  // namespace coli
