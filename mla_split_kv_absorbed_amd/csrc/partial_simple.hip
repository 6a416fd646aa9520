// Plain VALU split-KV partial attention: one workgroup per (part, query
// token, head). It is the fp32 path (fp32 arithmetic throughout) and the
// path for shapes the MFMA kernel does not cover. Online softmax over
// 256-key chunks, reductions in a fixed order.
#include "common.h"
#include "kernels.h"

namespace mla {

template <typename T>
__device__ __forceinline__ const T* row_ptr(const PartialParams& pp, int b, int j) {
  const T* kv = (const T*)pp.kv;
  if (pp.block_size > 0) {
    int id = pp.block_table[(size_t)b * pp.max_blocks + j / pp.block_size];
    return kv + ((size_t)id * pp.block_size + (j % pp.block_size)) * kRow;
  }
  return kv + ((size_t)b * pp.kv_seq_stride + j) * kRow;
}

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = is_max ? wave_max(v) : wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < 4; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  return r;
}

template <typename T>
__global__ __launch_bounds__(256) void partial_simple_kernel(PartialParams pp) {
  const int tid = threadIdx.x;
  const int unit = blockIdx.x;            // (p, b, s), s fastest
  const int s = unit % pp.S;
  const int b = (unit / pp.S) % pp.B;
  const int p = unit / (pp.S * pp.B);
  const int h = blockIdx.y;
  const int t = b * pp.S + s;
  const int Tq = pp.B * pp.S;

  __shared__ float qs[kRow];
  __shared__ float ps[256];
  __shared__ float red[4];

  const T* ql = (const T*)pp.q_lat + ((size_t)t * pp.H + h) * kDc;
  const T* qr = (const T*)pp.q_rope + ((size_t)t * pp.H + h) * kDr;
  for (int i = tid; i < kRow; i += 256) qs[i] = i < kDc ? to_f(ql[i]) : to_f(qr[i - kDc]);

  const int st = pp.range_start[(size_t)p * pp.B + b];
  const int en = pp.range_end[(size_t)p * pp.B + b];
  bool bad = st < 0 || en < st || (long long)en > pp.capacity;
  int vend = en;
  if (pp.mask == MLA_MASK_CAUSAL_WINDOW) vend = en - pp.S + s + 1;
  if (vend > en) vend = en;
  if (!bad && pp.block_size > 0 && vend > st) {
    int b0 = st / pp.block_size, b1 = (vend - 1) / pp.block_size;
    int f = 0;
    for (int i = b0 + tid; i <= b1; i += 256) {
      int id = pp.block_table[(size_t)b * pp.max_blocks + i];
      f |= (id < 0 || id >= pp.num_blocks);
    }
    bad = __syncthreads_or(f);
  }
  __syncthreads();

  float m = -INFINITY, l = 0.f, a0 = 0.f, a1 = 0.f;
  if (!bad) {
    for (int k0 = st; k0 < vend; k0 += 256) {
      const int j = k0 + tid;
      float sc = -INFINITY;
      if (j < vend) {
        const T* r = row_ptr<T>(pp, b, j);
        float d = 0.f;
        for (int i = 0; i < kRow; ++i) d = fmaf(qs[i], to_f(r[i]), d);
        sc = d * pp.scale;
      }
      const float mt = block_reduce(sc, red, true);
      const float mn = fmaxf(m, mt);
      const float pj = (j < vend) ? expf(sc - mn) : 0.f;
      ps[tid] = pj;
      const float alpha = (m == -INFINITY) ? 0.f : expf(m - mn);
      const float ls = block_reduce(pj, red, false);
      l = l * alpha + ls;
      a0 *= alpha;
      a1 *= alpha;
      m = mn;
      __syncthreads();
      const int nk = min(256, vend - k0);
      for (int jj = 0; jj < nk; ++jj) {
        const T* r = row_ptr<T>(pp, b, k0 + jj);
        const float w = ps[jj];
        a0 = fmaf(w, to_f(r[tid]), a0);
        a1 = fmaf(w, to_f(r[tid + 256]), a1);
      }
      __syncthreads();
    }
  }
  const size_t row = ((size_t)p * Tq + t) * pp.H + h;
  float o0, o1, lv;
  if (bad) {
    o0 = o1 = lv = NAN;
  } else if (l > 0.f) {
    const float inv = 1.f / l;
    o0 = a0 * inv;
    o1 = a1 * inv;
    lv = m + logf(l);
  } else {
    o0 = o1 = 0.f;
    lv = -INFINITY;
  }
  store_any(pp.out, row * kDc + tid, pp.out_dtype, o0);
  store_any(pp.out, row * kDc + tid + 256, pp.out_dtype, o1);
  if (tid == 0) store_any(pp.lse, row, pp.lse_dtype, lv);
}

hipError_t launch_partial_simple(const PartialParams& pp, int dtype, hipStream_t st) {
  dim3 grid(pp.P * pp.B * pp.S, pp.H);
  if (dtype == MLA_F32)
    hipLaunchKernelGGL(partial_simple_kernel<float>, grid, dim3(256), 0, st, pp);
  else if (dtype == MLA_BF16)
    hipLaunchKernelGGL(partial_simple_kernel<bf16>, grid, dim3(256), 0, st, pp);
  else
    hipLaunchKernelGGL(partial_simple_kernel<f16>, grid, dim3(256), 0, st, pp);
  return hipGetLastError();
}

}  // namespace mla
