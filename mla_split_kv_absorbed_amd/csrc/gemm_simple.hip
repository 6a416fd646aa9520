// Plain VALU per-head GEMMs of the decode step (fp32 accumulate):
//   q absorption  q_lat[t][h][c] = sum_j W_UK[h][c][j] q_nope[t][h][j]
//   V-up          out[t][h][v]   = sum_c x[t][h][c]   W_UV[h][c][v]
// Used for fp32 and for shapes the MFMA kernels do not cover.
#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int kTT = 32;  // query tokens per workgroup

// grid (H, ceil(T/32), 2); 64 threads; thread owns one output column v.
template <typename T>
__global__ __launch_bounds__(64) void vup_simple_kernel(const T* __restrict__ x,
                                                        const T* __restrict__ w,
                                                        T* __restrict__ out, int Tn, int H) {
  __shared__ float xs[kTT][kDc];
  const int h = blockIdx.x, t0 = blockIdx.y * kTT;
  const int v = blockIdx.z * 64 + threadIdx.x;
  const int nt = min(kTT, Tn - t0);
  for (int i = threadIdx.x; i < kTT * kDc; i += 64) {
    const int tt = i / kDc, c = i % kDc;
    xs[tt][c] = tt < nt ? to_f(x[((size_t)(t0 + tt) * H + h) * kDc + c]) : 0.f;
  }
  __syncthreads();
  float acc[kTT];
#pragma unroll
  for (int i = 0; i < kTT; ++i) acc[i] = 0.f;
  const T* wh = w + (size_t)h * kDc * kDv + v;
  for (int c = 0; c < kDc; ++c) {
    const float wv = to_f(wh[(size_t)c * kDv]);
#pragma unroll
    for (int i = 0; i < kTT; ++i) acc[i] = fmaf(xs[i][c], wv, acc[i]);
  }
  for (int i = 0; i < nt; ++i) out[((size_t)(t0 + i) * H + h) * kDv + v] = from_f<T>(acc[i]);
}

// grid (H, ceil(T/32), 8); 64 threads; thread owns one latent column c.
template <typename T>
__global__ __launch_bounds__(64) void absorb_simple_kernel(const T* __restrict__ qn,
                                                           const T* __restrict__ w,
                                                           T* __restrict__ ql, int Tn, int H) {
  __shared__ float qs[kTT][kDn];
  const int h = blockIdx.x, t0 = blockIdx.y * kTT;
  const int c = blockIdx.z * 64 + threadIdx.x;
  const int nt = min(kTT, Tn - t0);
  for (int i = threadIdx.x; i < kTT * kDn; i += 64) {
    const int tt = i / kDn, j = i % kDn;
    qs[tt][j] = tt < nt ? to_f(qn[((size_t)(t0 + tt) * H + h) * kDn + j]) : 0.f;
  }
  __syncthreads();
  float acc[kTT];
#pragma unroll
  for (int i = 0; i < kTT; ++i) acc[i] = 0.f;
  const T* wr = w + ((size_t)h * kDc + c) * kDn;
  for (int j = 0; j < kDn; ++j) {
    const float wv = to_f(wr[j]);
#pragma unroll
    for (int i = 0; i < kTT; ++i) acc[i] = fmaf(qs[i][j], wv, acc[i]);
  }
  for (int i = 0; i < nt; ++i) ql[((size_t)(t0 + i) * H + h) * kDc + c] = from_f<T>(acc[i]);
}

hipError_t launch_vup_simple(const void* x, const void* w, void* out, int Tn, int H, int dt,
                             hipStream_t st) {
  dim3 g(H, (Tn + kTT - 1) / kTT, kDv / 64);
  if (dt == MLA_F32)
    hipLaunchKernelGGL(vup_simple_kernel<float>, g, dim3(64), 0, st, (const float*)x,
                       (const float*)w, (float*)out, Tn, H);
  else if (dt == MLA_BF16)
    hipLaunchKernelGGL(vup_simple_kernel<bf16>, g, dim3(64), 0, st, (const bf16*)x,
                       (const bf16*)w, (bf16*)out, Tn, H);
  else
    hipLaunchKernelGGL(vup_simple_kernel<f16>, g, dim3(64), 0, st, (const f16*)x,
                       (const f16*)w, (f16*)out, Tn, H);
  return hipGetLastError();
}

hipError_t launch_absorb_simple(const void* qn, const void* w, void* ql, int Tn, int H, int dt,
                                hipStream_t st) {
  dim3 g(H, (Tn + kTT - 1) / kTT, kDc / 64);
  if (dt == MLA_F32)
    hipLaunchKernelGGL(absorb_simple_kernel<float>, g, dim3(64), 0, st, (const float*)qn,
                       (const float*)w, (float*)ql, Tn, H);
  else if (dt == MLA_BF16)
    hipLaunchKernelGGL(absorb_simple_kernel<bf16>, g, dim3(64), 0, st, (const bf16*)qn,
                       (const bf16*)w, (bf16*)ql, Tn, H);
  else
    hipLaunchKernelGGL(absorb_simple_kernel<f16>, g, dim3(64), 0, st, (const f16*)qn,
                       (const f16*)w, (f16*)ql, Tn, H);
  return hipGetLastError();
}

}  // namespace mla
