// Per-head GEMMs of the decode step on CDNA4 matrix cores (bf16 / fp16 in,
// fp32 accumulate, one rounding to the output type):
//
//   q absorption  q_lat^T[c][t] = sum_j W_UK[h][c][j] q_nope[t][h][j]
//     Both operands are contiguous along the contraction index j, so they
//     are read straight from global memory into MFMA operand registers.
//   V-up          out^T[v][t]   = sum_c W_UV[h][c][v] x[t][h][c]
//     W_UV[h] is stored [c][v] (v contiguous) but the matrix instruction wants
//     8 consecutive c per lane: the head's 64-column slice is staged in LDS
//     and read with the transposed LDS read. x is read directly; the result
//     is written in its batch-major [T][H][128] layout without any transpose
//     pass (the fused, transpose-free V-up).
//
// Computing the transposed products puts 4 consecutive output columns in
// each lane, so every store is one 8-byte write.
#include "common.h"
#include "kernels.h"
#include "prologue.h"

namespace mla {

#define LDS_AS __attribute__((address_space(3)))

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

template <typename T> struct GT;
template <> struct GT<bf16> {
  typedef bf16x8 v8;
  typedef bf16x4 v4;
  static __device__ __forceinline__ floatx16 mfma(v8 a, v8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct GT<f16> {
  typedef f16x8 v8;
  typedef f16x4 v4;
  static __device__ __forceinline__ floatx16 mfma(v8 a, v8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// q absorption of one 32-token block (the fused prologue's grid: (H, 2
// halves of c, ceil(T/32))), 4 waves, each wave two 32-row c tiles.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void absorb_block(const T* __restrict__ qn, const T* __restrict__ wuk,
                                             T* __restrict__ ql, int Tn, int H) {
  typedef typename GT<T>::v8 v8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.x;
  const int c0 = blockIdx.y * 256 + wave * 64;
  const int t0 = blockIdx.z * 32;
  const int r = lane & 31, hi = lane >> 5;
  const int t = t0 + r;
  // B = q_nope^T: column t, 8 consecutive j per k step; A = W_UK rows of the
  // wave's two 32-row c tiles. Every operand is loaded before the first
  // matrix instruction, so the wave pays one memory round trip.
  // rows past Tn load the last valid row (no branch per load) and are zeroed
  const int tl = min(t, Tn - 1);
  v8 b[kDn / 16];
#pragma unroll
  for (int k = 0; k < kDn / 16; ++k)
    b[k] = *(const v8*)(qn + ((size_t)tl * H + h) * kDn + k * 16 + hi * 8);
  if (t >= Tn)
#pragma unroll
    for (int k = 0; k < kDn / 16; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) b[k][i] = (T)0.f;
  v8 a[2][kDn / 16];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const T* wr = wuk + ((size_t)h * kDc + c0 + ct * 32 + r) * kDn + hi * 8;
#pragma unroll
    for (int k = 0; k < kDn / 16; ++k) a[ct][k] = *(const v8*)(wr + k * 16);
  }
  __builtin_amdgcn_sched_barrier(0);  // all loads issued before the first product
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int c = c0 + ct * 32;
    floatx16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int k = 0; k < kDn / 16; ++k) acc = GT<T>::mfma(a[ct][k], b[k], acc);
    if (t < Tn) {
      T* dst = ql + ((size_t)t * H + h) * kDc + c + 4 * hi;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        typename GT<T>::v4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (T)acc[4 * g + i];
        *(typename GT<T>::v4*)(dst + 8 * g) = v;
      }
    }
  }
}

// q absorption over many token blocks: grid (H, 2 halves of c, ceil(blocks /
// kAbsorbBlocks)); each wave keeps its two W_UK tiles in registers and walks
// up to kAbsorbBlocks 32-token blocks, loading the next block's q_nope while
// the current one is multiplied, so W_UK[h] is read once per kAbsorbBlocks
// blocks instead of once per block.
constexpr int kAbsorbBlocks = 4;

template <typename T>
__global__ __launch_bounds__(256) void absorb_mfma_kernel(const T* __restrict__ qn,
                                                          const T* __restrict__ wuk,
                                                          T* __restrict__ ql, int Tn, int H) {
  typedef typename GT<T>::v8 v8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.x;
  const int c0 = blockIdx.y * 256 + wave * 64;
  const int r = lane & 31, hi = lane >> 5;
  const int nblk = (Tn + 31) / 32;
  const int b0 = blockIdx.z * kAbsorbBlocks, b1 = min(nblk, b0 + kAbsorbBlocks);
  // B = q_nope^T of block tb: column t, 8 consecutive j per k step (rows past
  // Tn load the last valid row and are never stored)
  auto load_b = [&](int tb, v8* b) __attribute__((always_inline)) {
    const int tl = min(tb * 32 + r, Tn - 1);
#pragma unroll
    for (int k = 0; k < kDn / 16; ++k)
      b[k] = *(const v8*)(qn + ((size_t)tl * H + h) * kDn + k * 16 + hi * 8);
  };
  v8 a[2][kDn / 16];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const T* wr = wuk + ((size_t)h * kDc + c0 + ct * 32 + r) * kDn + hi * 8;
#pragma unroll
    for (int k = 0; k < kDn / 16; ++k) a[ct][k] = *(const v8*)(wr + k * 16);
  }
  v8 b[2][kDn / 16];
  load_b(b0, b[0]);
#pragma unroll
  for (int i = 0; i < kAbsorbBlocks; ++i) {
    const int tb = b0 + i;
    if (tb >= b1) break;
    if (tb + 1 < b1) load_b(tb + 1, b[(i + 1) & 1]);
    const int t = tb * 32 + r;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      floatx16 acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
      for (int k = 0; k < kDn / 16; ++k) acc = GT<T>::mfma(a[ct][k], b[i & 1][k], acc);
      if (t < Tn) {
        T* dst = ql + ((size_t)t * H + h) * kDc + c0 + ct * 32 + 4 * hi;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          typename GT<T>::v4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (T)acc[4 * g + e];
          *(typename GT<T>::v4*)(dst + 8 * g) = v;
        }
      }
    }
  }
}

// The fused decode prologue: the absorption blocks (head, c half, token
// block) also rotate head h's q_pe (c half 0) and, for head 0 / c half 1,
// append the token block's cache rows.
template <typename T>
__global__ __launch_bounds__(256) void prologue_mfma_kernel(PrologueParams pp) {
  absorb_block<T>((const T*)pp.q_nope, (const T*)pp.w_uk, (T*)pp.q_lat, pp.T, pp.H);
  rope_append_block<T>(pp, blockIdx.x, blockIdx.z * 32, blockIdx.y == 0,
                       blockIdx.x == 0 && blockIdx.y == 1);
}

// ---------------------------------------------------------------------------
// V-up: grid (H, 2 halves of v, ceil(T/32)), 4 waves. All 4 waves stage
// W_UV[h][:, 64-column half] in LDS (every load issued before the first LDS
// write, so the block pays one memory round trip); waves 0 and 1 then each
// compute one 32-column v tile of one 32-token block with their x operands
// (all 32 k steps) already in registers.
// ---------------------------------------------------------------------------
constexpr int kVupCols = 64;
constexpr int kVupRow = kVupCols * 2 + 32;  // bytes per LDS row (padded)
constexpr int kVupThreads = 256;
constexpr int kVupChunks = kDc * kVupCols * 2 / 16 / kVupThreads;  // 16-byte chunks per thread

template <typename T>
__global__ __launch_bounds__(kVupThreads) void vup_mfma_kernel(const T* __restrict__ x,
                                                               const T* __restrict__ wuv,
                                                               T* __restrict__ out, int Tn, int H) {
  typedef typename GT<T>::v8 v8;
  __shared__ __attribute__((aligned(16))) char ws[kDc * kVupRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, vh = blockIdx.y * kVupCols;
  const int t0 = blockIdx.z * 32;
  const int r = lane & 31, hi = lane >> 5;
  const int t = t0 + r;
  // W_UV[h][c][vh : vh+64]: 512 rows x 128 B = 4096 chunks of 16 B
  const T* wsrc = wuv + (size_t)h * kDc * kDv + vh;
  v8 st[kVupChunks];
#pragma unroll
  for (int i = 0; i < kVupChunks; ++i) {
    const int idx = tid + i * kVupThreads, c = idx >> 3, q = idx & 7;
    st[i] = *(const v8*)(wsrc + (size_t)c * kDv + q * 8);
  }
  // x operand of waves 0 and 1: column t, 8 consecutive c per k step
  // (rows past Tn load the last valid row, no branch per load; their
  // results are never stored)
  v8 b[kDc / 16];
  if (wave < 2) {
    const T* xr = x + ((size_t)min(t, Tn - 1) * H + h) * kDc + hi * 8;
#pragma unroll
    for (int k = 0; k < kDc / 16; ++k) b[k] = *(const v8*)(xr + k * 16);
  }
#pragma unroll
  for (int i = 0; i < kVupChunks; ++i) {
    const int idx = tid + i * kVupThreads, c = idx >> 3, q = idx & 7;
    *(v8*)(ws + c * kVupRow + q * 16) = st[i];
  }
  __syncthreads();
  if (wave >= 2) return;
  // A = W^T (rows v, k = c) by transposed reads: 16-lane block g16 covers
  // v 16(g16&1)..+15 and c rows 8(g16>>1).. of each 16-wide k step
  const int j16 = lane & 15, g16 = lane >> 4;
  const int a_off = ((8 * (g16 >> 1) + (j16 >> 2)) * kVupRow) +
                    (wave * 32 + 16 * (g16 & 1) + 4 * (j16 & 3)) * 2;
  floatx16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int k = 0; k < kDc / 16; ++k) {
    const char* a0 = ws + a_off + k * 16 * kVupRow;
    const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)a0);
    const shortx4 h4 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)(a0 + 4 * kVupRow));
    const v8 a = __builtin_bit_cast(v8, __builtin_shufflevector(lo, h4, 0, 1, 2, 3, 4, 5, 6, 7));
    acc = GT<T>::mfma(a, b[k], acc);
  }
  if (t < Tn) {
    T* dst = out + ((size_t)t * H + h) * kDv + vh + wave * 32 + 4 * hi;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      typename GT<T>::v4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (T)acc[4 * g + i];
      *(typename GT<T>::v4*)(dst + 8 * g) = v;
    }
  }
}

static_assert(kVupChunks * kVupThreads * 16 == kDc * kVupCols * 2, "V-up staging split");

hipError_t launch_absorb_mfma(const void* qn, const void* w, void* ql, int Tn, int H, int dt,
                              hipStream_t st) {
  dim3 g(H, kDc / 256, ((Tn + 31) / 32 + kAbsorbBlocks - 1) / kAbsorbBlocks);
  if (dt == MLA_BF16)
    hipLaunchKernelGGL(absorb_mfma_kernel<bf16>, g, dim3(256), 0, st, (const bf16*)qn,
                       (const bf16*)w, (bf16*)ql, Tn, H);
  else
    hipLaunchKernelGGL(absorb_mfma_kernel<f16>, g, dim3(256), 0, st, (const f16*)qn,
                       (const f16*)w, (f16*)ql, Tn, H);
  return hipGetLastError();
}

hipError_t launch_prologue_mfma(const PrologueParams& pp, int dt, hipStream_t st) {
  dim3 g(pp.H, kDc / 256, (pp.T + 31) / 32);
  if (dt == MLA_BF16)
    hipLaunchKernelGGL(prologue_mfma_kernel<bf16>, g, dim3(256), 0, st, pp);
  else
    hipLaunchKernelGGL(prologue_mfma_kernel<f16>, g, dim3(256), 0, st, pp);
  return hipGetLastError();
}

hipError_t launch_vup_mfma(const void* x, const void* w, void* out, int Tn, int H, int dt,
                           hipStream_t st) {
  dim3 g(H, kDv / kVupCols, (Tn + 31) / 32);
  if (dt == MLA_BF16)
    hipLaunchKernelGGL(vup_mfma_kernel<bf16>, g, dim3(kVupThreads), 0, st, (const bf16*)x,
                       (const bf16*)w, (bf16*)out, Tn, H);
  else
    hipLaunchKernelGGL(vup_mfma_kernel<f16>, g, dim3(kVupThreads), 0, st, (const f16*)x,
                       (const f16*)w, (f16*)out, Tn, H);
  return hipGetLastError();
}

}  // namespace mla
