// Split-KV partial attention over ranges of a few keys: the MTP current
// chunk of the study page (the CURRENT call: q_len query tokens against the
// q_len keys of the chunk itself, under the causal window), where the cache
// is a contiguous [B][kv_seq_stride][576] tensor with kv_seq_stride <=
// kShortKeys, so no valid range holds more keys than that.
//
// One wave per (part, query token) and 4 heads (short.h). The keys of a
// sequence are shared by all its rows and stay in the L1/L2 caches, so the
// launch moves about one read of the queries and one write of the outputs;
// the matrix kernel would spend a workgroup's fixed cost (128 heads of
// queries in, 128 output rows out) on a single tile.
#include "short.h"

#include <algorithm>

namespace mla {

constexpr int kShortHeads = 4;  // heads per wave of the standalone kernel

template <typename T>
__global__ __launch_bounds__(256) void partial_short_kernel(PartialParams pp) {
  const int lane = threadIdx.x & 63;
  const long long tasks = short_tasks(pp, kShortHeads);
  const long long stride = (long long)gridDim.x * 4;
  const long long first =
      (long long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (long long task = first; task < tasks; task += stride)
    short_task<T, kShortHeads>(pp, task, lane);
}

hipError_t launch_partial_short(const PartialParams& pp, int dtype, hipStream_t st) {
  // four wave tasks per workgroup; very large calls loop over the tasks
  const unsigned grid =
      (unsigned)std::min<long long>((short_tasks(pp, kShortHeads) + 3) / 4, 1 << 20);
  if (dtype == MLA_BF16)
    hipLaunchKernelGGL(partial_short_kernel<bf16>, dim3(grid), dim3(256), 0, st, pp);
  else
    hipLaunchKernelGGL(partial_short_kernel<f16>, dim3(grid), dim3(256), 0, st, pp);
  return hipGetLastError();
}

}  // namespace mla
