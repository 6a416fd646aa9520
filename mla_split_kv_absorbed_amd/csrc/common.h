// Shared device/host helpers of the MLA decode library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "mla_decode.h"
#include "plan.h"

namespace mla {

constexpr int kDc = MLA_D_C;
constexpr int kDr = MLA_D_R;
constexpr int kRow = MLA_D_ROW;
constexpr int kDn = MLA_D_NOPE;
constexpr int kDv = MLA_D_V;
constexpr int kWave = 64;

typedef __bf16 bf16;
typedef _Float16 f16;

// ---- scalar conversions (round-to-nearest-even on the way down) ----------
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(f16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ f16 from_f<f16>(float x) { return (f16)x; }

// runtime-dtype load/store of one element (outputs whose dtype is an argument)
__device__ __forceinline__ float load_any(const void* p, size_t i, int dt) {
  if (dt == MLA_F32) return ((const float*)p)[i];
  if (dt == MLA_BF16) return (float)((const bf16*)p)[i];
  return (float)((const f16*)p)[i];
}
__device__ __forceinline__ void store_any(void* p, size_t i, int dt, float v) {
  if (dt == MLA_F32) ((float*)p)[i] = v;
  else if (dt == MLA_BF16) ((bf16*)p)[i] = (bf16)v;
  else ((f16*)p)[i] = (f16)v;
}

__host__ __device__ inline int elem_bytes(int dt) { return dt == MLA_F32 ? 4 : 2; }

// ---- wave / block reductions in a fixed order ------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

struct PartialParams {
  const void* q_lat;
  const void* q_rope;
  const void* kv;
  const int32_t* block_table;
  const int32_t* range_start;
  const int32_t* range_end;
  void* out;
  void* lse;
  void* ws_out;     // split partials [slot][S][H][512] in out_dtype
  float* ws_lse;    // split partials [slot][S][H] fp32
  int B, S, H, P;
  int block_size, max_blocks, num_blocks, kv_seq_stride;
  int mask;
  int out_dtype, lse_dtype;
  int num_splits;   // 0 = automatic
  int max_chunks;   // grid bound of the main kernel (in chunks)
  const int32_t* plan;  // a plan built on the host (plan.h layout), or NULL
  int plan_chunks, plan_split_units;  // its chunk and cut-range counts
  float scale;
  long long capacity;  // tokens addressable per sequence
};

}  // namespace mla
