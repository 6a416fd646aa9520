// LSE combine of P partial latent outputs (+ an optional local part).
// One wave per (token, head) row of 512 values: every lane owns 8
// consecutive values, so each part's row is read with one coalesced
// 1 KB (16-bit) / 2 KB (fp32) wave access. fp32 math in registers; parts are
// summed in index order with the local part last.
#include "common.h"
#include "kernels.h"

namespace mla {

template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
  typedef bf16 v __attribute__((ext_vector_type(8)));
};
template <> struct Vec8<f16> {
  typedef f16 v __attribute__((ext_vector_type(8)));
};
template <> struct Vec8<float> {
  typedef float v __attribute__((ext_vector_type(8)));
};

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* o) {
  typename Vec8<T>::v x = *(const typename Vec8<T>::v*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)x[i];
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float* o) {
  typename Vec8<T>::v x;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = from_f<T>(o[i]);
  *(typename Vec8<T>::v*)p = x;
}

// LSE of merged part i of a row (parts in index order, the local part last)
__device__ __forceinline__ float part_lse(const CombineParams& c, int i, size_t row,
                                          size_t rows) {
  return i < c.P ? load_any(c.parts_lse, (size_t)i * rows + row, c.lse_dtype)
                 : load_any(c.local_lse, row, c.lse_dtype);
}

template <typename TP, typename TO>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams c) {
  const int lane = threadIdx.x & 63;
  const size_t rows = (size_t)c.T * c.H;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int np = c.P + (c.local_out ? 1 : 0);

  // lane i holds the LSE of part i0 + i: the maximum and the weights take
  // one load round trip for up to 64 parts
  float m = -INFINITY;
  bool nan_seen = false;
  for (int i0 = 0; i0 < np; i0 += 64) {
    const float li = i0 + lane < np ? part_lse(c, i0 + lane, row, rows) : -INFINITY;
    nan_seen |= isnan(li);
    m = fmaxf(m, li);
  }
  m = wave_max(m);
  nan_seen = __builtin_amdgcn_ballot_w64(nan_seen) != 0;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float z = 0.f;
  if (m != -INFINITY && !nan_seen) {
    for (int i0 = 0; i0 < np; i0 += 64) {
      const int cnt = min(64, np - i0);
      const float li = lane < cnt ? part_lse(c, i0 + lane, row, rows) : -INFINITY;
      const float wl = li == -INFINITY ? 0.f : expf(li - m);
      // parts in ascending order, 4 rows in flight
      for (int i = 0; i < cnt; i += 4) {
        float v[4][8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int k = i0 + i + q;
          if (i + q < cnt) {
            const TP* src = k < c.P ? (const TP*)c.parts_out + ((size_t)k * rows + row) * kDc
                                    : (const TP*)c.local_out + row * kDc;
            load8<TP>(src + lane * 8, v[q]);
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float w = __shfl(wl, i + q, 64);
          if (i + q < cnt) {
            z += w;
            if (w != 0.f)
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, v[q][e], acc[e]);
          }
        }
      }
    }
  }
  float o[8];
  float lse;
  if (nan_seen) {
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = NAN;
    lse = NAN;
  } else if (z > 0.f) {
    const float inv = 1.f / z;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = acc[k] * inv;
    lse = m + logf(z);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = 0.f;
    lse = -INFINITY;
  }
  store8<TO>((TO*)c.out + row * kDc + lane * 8, o);
  if (c.lse_out && lane == 0) c.lse_out[row] = lse;
}

template <typename TP>
static void launch_combine_out(const CombineParams& c, dim3 g, hipStream_t st) {
  if (c.out_dtype == MLA_F32)
    hipLaunchKernelGGL((combine_kernel<TP, float>), g, dim3(256), 0, st, c);
  else if (c.out_dtype == MLA_BF16)
    hipLaunchKernelGGL((combine_kernel<TP, bf16>), g, dim3(256), 0, st, c);
  else
    hipLaunchKernelGGL((combine_kernel<TP, f16>), g, dim3(256), 0, st, c);
}

hipError_t launch_combine(const CombineParams& c, hipStream_t st) {
  const size_t rows = (size_t)c.T * c.H;
  dim3 g((unsigned)((rows + 3) / 4));
  if (c.part_dtype == MLA_F32) launch_combine_out<float>(c, g, st);
  else if (c.part_dtype == MLA_BF16) launch_combine_out<bf16>(c, g, st);
  else launch_combine_out<f16>(c, g, st);
  return hipGetLastError();
}

}  // namespace mla
