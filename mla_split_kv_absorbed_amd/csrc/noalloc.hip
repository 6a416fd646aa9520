// mla_decode_partial_noalloc: the partial call with the library's own
// device scratch as its workspace, for callers that cannot allocate (code
// under HIP graph capture, serving loops, harnesses that forbid hipMalloc).
//
// The scratch is a file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends. In host
// code the array's name only stands in for the symbol, so its device address
// is looked up once per device (hipGetSymbolAddress with that device
// current) and kept; kernels and copies get that address, never the name.
//
// Nothing in the workspace has to start at zero: every call's kernels write
// the split-unit count and every descriptor they read later. Calls that
// overlap on one GPU (other streams, other host threads) share the array and
// race; order them on one stream.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = (size_t)96 << 20;
constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device (null: not looked up)

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// the current device's copy of `scratch` (looked up on its first use)
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

size_t mla_noalloc_scratch_bytes(void) { return kScratchBytes; }

int mla_decode_partial_noalloc(const mla_partial_args* a, void* stream) {
  if (!a) return MLA_ERR_NULL;
  const size_t need = mla::partial_workspace_need(a);
  if (need == (size_t)-1) return mla::partial_call(a, nullptr, 0, stream);  // the error code
  if (need > kScratchBytes) return MLA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const int st = scratch_address(&ws);
    if (st != MLA_OK) return st;
  }
  return mla::partial_call(a, ws, need > 0 ? kScratchBytes : 0, stream);
}

}  // extern "C"
