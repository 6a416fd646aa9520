// The short-range partial attention (ranges of at most kShortKeys keys over
// a contiguous cache: the current chunk), as device functions shared by its
// own kernel (partial_short.hip) and by the matrix kernel's combined launch
// of a history call and a current-chunk call (partial_mfma.hip).
//
// One wave per (part, query token) and kHeads heads, vector units only:
// lane l holds latent values 8 l .. 8 l + 7 and rotary value l of the queries
// and of each key, a key's score is a wave sum, and the softmax runs in fp32.
#pragma once

#include "common.h"
#include "kernels.h"

namespace mla {

// Sum over the 64 lanes with data-parallel-primitive moves inside the
// vector unit (no LDS round trip per step): quad swaps, half-row and row
// mirrors, then row 0's and rows 0-1's sums broadcast into rows 1 and 3;
// lane 63 ends with the total, returned to every lane. Needs every lane of
// the wave active.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(
                 __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xF, false));
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_add<0x140, 0xF>(v);  // row_mirror
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

template <typename T>
__device__ __forceinline__ void store_row8(void* out, size_t row, int lane, int dt,
                                           const float* v) {
  if (dt == MLA_F32) {
    float4* o = (float4*)((float*)out + row * kDc) + 2 * lane;
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else if (dt == MLA_BF16) {
    typedef bf16 v8b __attribute__((ext_vector_type(8)));
    v8b x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (bf16)v[e];
    *((v8b*)((bf16*)out + row * kDc) + lane) = x;
  } else {
    typedef f16 v8h __attribute__((ext_vector_type(8)));
    v8h x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (f16)v[e];
    *((v8h*)((f16*)out + row * kDc) + lane) = x;
  }
}

// Wave task w: part p, query token t, heads h0 = kHeads j .. (rows of the
// output, consecutive). The queries are requested with the range; the
// visible keys (at most kShortKeys) follow in groups of 4 shared by the
// wave's heads, under an online softmax in fp32 (a key past the last repeats
// it and gets weight 0, so a group's loads issue together). The heads'
// score sums are independent, so their reductions overlap.
template <typename T, int kHeads>
__device__ __forceinline__ void short_task(const PartialParams& pp, long long task, int lane) {
  // every multiply and add exactly as written (no fusing by the compiler),
  // so that any kHeads and any kernel this is inlined into give the same bits
#pragma clang fp contract(off)
  typedef T v8 __attribute__((ext_vector_type(8)));
  const int Tq = pp.B * pp.S;
  const int hg = (pp.H + kHeads - 1) / kHeads;
  const int h0 = (int)(task % hg) * kHeads;
  const int t = (int)((task / hg) % Tq);
  const int p = (int)(task / ((long long)hg * Tq));
  const int b = t / pp.S, s = t % pp.S;
  v8 q[kHeads];
  float qr[kHeads];
#pragma unroll
  for (int i = 0; i < kHeads; ++i) {
    const size_t qrow = (size_t)t * pp.H + min(h0 + i, pp.H - 1);
    q[i] = *((const v8*)((const T*)pp.q_lat + qrow * kDc) + lane);
    qr[i] = to_f(((const T*)pp.q_rope)[qrow * kDr + lane]);
  }
  const int st = pp.range_start[(size_t)p * pp.B + b];
  const int en = pp.range_end[(size_t)p * pp.B + b];
  const bool bad = range_bad(st, en, pp.capacity);
  // visible keys: the whole range, or under the window offsets
  // 0 .. (en - st) - S + s; at most capacity <= kShortKeys
  int n = 0;
  if (!bad) {
    const int vend = pp.mask == MLA_MASK_CAUSAL_WINDOW ? min(en, en - pp.S + s + 1) : en;
    n = min(max(0, vend - st), kShortKeys);
  }
  float m[kHeads], l[kHeads], acc[kHeads][8];
#pragma unroll
  for (int i = 0; i < kHeads; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  }
  const T* kb = (const T*)pp.kv + ((size_t)b * pp.kv_seq_stride + (bad ? 0 : st)) * kRow;
  for (int g = 0; g < n; g += 4) {
    v8 c[4];
    float kr[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const size_t j = (size_t)min(g + k, n - 1);
      c[k] = *((const v8*)(kb + j * kRow) + lane);
      kr[k] = to_f(kb[j * kRow + kDc + lane]);
    }
#pragma unroll
    for (int i = 0; i < kHeads; ++i) {
      float sc[4];
      float mg = -INFINITY;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float d = qr[i] * kr[k];
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(to_f(q[i][e]), to_f(c[k][e]), d);
        d = wave_sum_dpp(d) * pp.scale;
        sc[k] = g + k < n ? d : -INFINITY;
        mg = fmaxf(mg, sc[k]);
      }
      const float mn = fmaxf(m[i], mg);
      const float alpha = m[i] == -INFINITY ? 0.f : expf(m[i] - mn);
      l[i] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] *= alpha;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float w = g + k < n ? expf(sc[k] - mn) : 0.f;
        l[i] += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(w, to_f(c[k][e]), acc[i][e]);
      }
      m[i] = mn;
    }
  }
  const size_t orow0 = ((size_t)p * Tq + t) * pp.H + h0;
#pragma unroll
  for (int i = 0; i < kHeads; ++i) {
    if (h0 + i >= pp.H) break;
    float lse;
    if (bad) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] = NAN;
      lse = NAN;
    } else if (n == 0) {
      lse = -INFINITY;  // acc stays 0
    } else {
      const float inv = 1.f / l[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] *= inv;
      lse = m[i] + logf(l[i]);
    }
    store_row8<T>(pp.out, orow0 + i, lane, pp.out_dtype, acc[i]);
    if (lane == 0) store_any(pp.lse, orow0 + i, pp.lse_dtype, lse);
  }
}

// wave tasks of a call at kHeads heads per wave
__host__ __device__ inline long long short_tasks(const PartialParams& pp, int heads) {
  return (long long)pp.P * pp.B * pp.S * ((pp.H + heads - 1) / heads);
}

}  // namespace mla
