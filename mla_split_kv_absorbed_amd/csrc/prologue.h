// Rotary embedding and cache append of the decode prologue (device code
// shared by the fused matrix-core kernel and the stand-alone kernel).
//
// rope rotates each consecutive pair (x[2i], x[2i+1]) of the 64 rope values
// by pos * theta^(-2i/64); the angle is formed and reduced in double
// precision (positions reach tens of thousands of radians), the rotation
// itself is fp32.
#pragma once

#include "common.h"
#include "kernels.h"

namespace mla {

__device__ __forceinline__ void rope_cs(int pos, int i, double log2_theta, float& c, float& s) {
  const double inv = exp2(-(double)(2 * i) / (double)kDr * log2_theta);
  double sn, cs;
  sincos((double)pos * inv, &sn, &cs);
  c = (float)cs;
  s = (float)sn;
}

// cache row of new token t, or -1 when its slot is invalid
__device__ __forceinline__ long long prologue_row(const PrologueParams& pp, int t) {
  const int b = t / pp.S;
  const int pos = pp.positions[t];
  if (pos < 0) return -1;
  if (pp.block_size > 0) {
    const int blk = pos / pp.block_size;
    if (blk >= pp.max_blocks) return -1;
    const int id = pp.block_table[(size_t)b * pp.max_blocks + blk];
    if (id < 0 || id >= pp.num_blocks) return -1;
    return (long long)id * pp.block_size + pos % pp.block_size;
  }
  if (pos >= pp.kv_seq_stride) return -1;
  return (long long)b * pp.kv_seq_stride + pos;
}

// With rot_q: q_rope of head h for tokens [t0, t0 + 32). With append: the
// cache rows of those tokens. 256 threads.
template <typename T>
__device__ __forceinline__ void rope_append_block(const PrologueParams& pp, int h, int t0,
                                                  bool rot_q, bool append) {
  const int tid = threadIdx.x;
  if (rot_q) {
    for (int idx = tid; idx < 32 * (kDr / 2); idx += 256) {
      const int t = t0 + idx / (kDr / 2), i = idx % (kDr / 2);
      if (t >= pp.T) continue;
      float c, s;
      rope_cs(pp.positions[t], i, pp.log2_theta, c, s);
      const size_t o = ((size_t)t * pp.H + h) * kDr + 2 * i;
      const float x0 = (float)((const T*)pp.q_pe)[o], x1 = (float)((const T*)pp.q_pe)[o + 1];
      ((T*)pp.q_rope)[o] = from_f<T>(x0 * c - x1 * s);
      ((T*)pp.q_rope)[o + 1] = from_f<T>(x0 * s + x1 * c);
    }
  }
  if (append) {
    for (int tt = 0; tt < 32; ++tt) {
      const int t = t0 + tt;
      if (t >= pp.T) break;
      const long long row = prologue_row(pp, t);
      if (row < 0) continue;
      const T* src = (const T*)pp.kv_new + (size_t)t * kRow;
      T* dst = (T*)pp.kv + (size_t)row * kRow;
      for (int e = tid; e < kDc; e += 256) dst[e] = src[e];
      if (tid < kDr / 2) {
        float c, s;
        rope_cs(pp.positions[t], tid, pp.log2_theta, c, s);
        const float x0 = (float)src[kDc + 2 * tid], x1 = (float)src[kDc + 2 * tid + 1];
        dst[kDc + 2 * tid] = from_f<T>(x0 * c - x1 * s);
        dst[kDc + 2 * tid + 1] = from_f<T>(x0 * s + x1 * c);
      }
    }
  }
}

}  // namespace mla
