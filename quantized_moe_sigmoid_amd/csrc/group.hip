// group.hip — standalone batch-union grouping kernel (one workgroup of 1024
// threads); the routine itself is group_body in group_impl.h.
#include "group_impl.h"

namespace coli {

constexpr int GROUP_THREADS = 1024;

template <int Q>
__global__ __launch_bounds__(GROUP_THREADS) void group_kernel(const int32_t *__restrict__ idx, int P, int E, int C,
                                                              GroupOut o) {
  extern __shared__ uint16_t hist[];
  __shared__ GroupLds<GROUP_THREADS> L;
  group_body<GROUP_THREADS, Q>(idx, P, E, C, o, hist, L);
}

bool group_supported(int P, int E) {
  int Q, C;
  return P <= 65535 && E <= 1024 && group_shape(P, E, Q, C);
}

hipError_t launch_group(const coli_moe_cfg &c, const int32_t *idx, int32_t T, int32_t *cnt, int32_t *off,
                        int32_t *perm, int32_t *active, int32_t *nact, hipStream_t s) {
  const int E = c.n_experts, P = T * c.top_k;
  int Q, C;
  if (!group_shape(P, E, Q, C)) return hipErrorInvalidValue;
  const size_t lds = (size_t)C * E * sizeof(uint16_t);
  const GroupOut o{cnt, off, perm, active, nact};
  switch (Q) {
    case 1: hipLaunchKernelGGL(group_kernel<1>, dim3(1), dim3(GROUP_THREADS), lds, s, idx, P, E, C, o); break;
    case 2: hipLaunchKernelGGL(group_kernel<2>, dim3(1), dim3(GROUP_THREADS), lds, s, idx, P, E, C, o); break;
    case 4: hipLaunchKernelGGL(group_kernel<4>, dim3(1), dim3(GROUP_THREADS), lds, s, idx, P, E, C, o); break;
    case 8: hipLaunchKernelGGL(group_kernel<8>, dim3(1), dim3(GROUP_THREADS), lds, s, idx, P, E, C, o); break;
    default: hipLaunchKernelGGL(group_kernel<16>, dim3(1), dim3(GROUP_THREADS), lds, s, idx, P, E, C, o); break;
  }
  return hipGetLastError();
}

}  // namespace coli
