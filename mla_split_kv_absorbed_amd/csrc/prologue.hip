// Rotary embedding of the query rope part and append of the new tokens'
// cache rows, as a kernel of its own (the fp32 prologue; bf16 / fp16 fuse
// the same code into the absorption kernel). Grid (H, 1, ceil(T / 32)),
// 256 threads: block (h, t-block) rotates head h's q_pe, block h = 0 also
// appends the token block's cache rows.
#include "prologue.h"

namespace mla {

template <typename T>
__global__ __launch_bounds__(256) void rope_append_kernel(PrologueParams pp) {
  rope_append_block<T>(pp, blockIdx.x, blockIdx.z * 32, true, blockIdx.x == 0);
}

hipError_t launch_rope_append(const PrologueParams& pp, int dt, hipStream_t st) {
  dim3 g(pp.H, 1, (pp.T + 31) / 32);
  if (dt == MLA_F32)
    hipLaunchKernelGGL(rope_append_kernel<float>, g, dim3(256), 0, st, pp);
  else if (dt == MLA_BF16)
    hipLaunchKernelGGL(rope_append_kernel<bf16>, g, dim3(256), 0, st, pp);
  else
    hipLaunchKernelGGL(rope_append_kernel<f16>, g, dim3(256), 0, st, pp);
  return hipGetLastError();
}

}  // namespace mla
