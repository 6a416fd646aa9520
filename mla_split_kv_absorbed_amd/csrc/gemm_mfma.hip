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

// q absorption of the decode step: grid (H, 4 quarters of c, ceil(T / 128)
// token groups), 4 waves. The workgroup's 128 rows of W_UK[h] (32 KB) and
// its tokens' q_nope[t][h] rows (256 B each) are staged in LDS by direct
// loads, every instruction covering whole 256-byte rows (four per
// instruction), so each cache line is fetched once; the operands are then
// read from LDS in the matrix layout. Wave w computes c rows 32 w .. of the
// quarter for every 32-token block of the group; each block's results go out
// through LDS (the W rows, once every wave holds its own in registers), one
// 256-byte row per token, as soon as the block is done. LDS rows are 16 chunks of
// 16 B with chunk c of row r at position c ^ (r & 15), which keeps the
// operand reads (16 rows per read) free of bank conflicts.
constexpr int kAbsRows = 128;  // c rows per workgroup
constexpr int kAbsTok = 128;   // tokens per workgroup
constexpr int kAbsRowB = kDn * 2;  // 256 bytes per LDS row

__device__ __forceinline__ int abs_pos(int chunk, int row) { return (chunk ^ (row & 15)) << 4; }

template <typename T>
__global__ __launch_bounds__(256) void absorb_mfma_kernel(const T* __restrict__ qn,
                                                          const T* __restrict__ wuk,
                                                          T* __restrict__ ql, int Tn, int H) {
  typedef typename GT<T>::v8 v8;
  __shared__ __attribute__((aligned(1024))) char wl[kAbsRows * kAbsRowB];  // W rows, then the results
  __shared__ __attribute__((aligned(1024))) char qs[kAbsTok * kAbsRowB];   // q_nope rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, c0 = blockIdx.y * kAbsRows, t0 = blockIdx.z * kAbsTok;
  const int nt = min(kAbsTok, Tn - t0);
  // W_UK[h][c0 + r][:]: 128 contiguous rows. Load i of wave w fills rows
  // 4 (8 w + i) .. + 3: lane l takes row 4 (8 w + i) + l / 16, LDS position
  // l % 16, i.e. the row's chunk (l % 16) ^ (row % 16).
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(wuk + ((size_t)h * kDc + c0) * kDn), (short)0, kAbsRows * kAbsRowB, 0x00020000);
  // q_nope[t0 + j][h][:]: rows H * 256 bytes apart; tokens past Tn fall
  // outside the records and load zeros
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(qn + ((size_t)t0 * H + h) * kDn), (short)0, ((nt - 1) * H + 1) * kAbsRowB,
      0x00020000);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 4 * (8 * wave + i) + (lane >> 4);
    const int pos = abs_pos(lane & 15, row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (LDS_AS void*)(wl + (8 * wave + i) * 1024), 16,
                                             row * kAbsRowB + pos, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (LDS_AS void*)(qs + (8 * wave + i) * 1024), 16,
                                             row * H * kAbsRowB + pos, 0, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's rows landed
  __syncthreads();

  const int r = lane & 31, hi = lane >> 5;
  // A = W rows 32 wave + r, 8 consecutive j per k step
  v8 a[kDn / 16];
#pragma unroll
  for (int k = 0; k < kDn / 16; ++k)
    a[k] = *(const v8*)(wl + (32 * wave + r) * kAbsRowB + abs_pos(2 * k + hi, r));
  const int nblk = (nt + 31) / 32;
  __syncthreads();  // every wave holds its W rows: their LDS takes the results
  // Token block bk: its products, then its results (token 32 bk + r, c rows
  // 32 wave + 8 g + 4 hi .. + 3: 8 bytes at chunk 4 wave + g, half hi of LDS
  // row 32 bk + r), then one 256-byte row per token to q_lat[t0 + row][h]
  // [c0 .. c0 + 127]; the stores of a block drain while the next block's
  // products run.
#pragma unroll
  for (int bk = 0; bk < kAbsTok / 32; ++bk) {
    if (bk < nblk) {
      floatx16 acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
      for (int k = 0; k < kDn / 16; ++k) {
        const v8 b = *(const v8*)(qs + (32 * bk + r) * kAbsRowB + abs_pos(2 * k + hi, r));
        acc = GT<T>::mfma(a[k], b, acc);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        typename GT<T>::v4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (T)acc[4 * g + e];
        *(typename GT<T>::v4*)(wl + (32 * bk + r) * kAbsRowB + abs_pos(4 * wave + g, r) + 8 * hi) = v;
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 32 * 16 / 256; ++i) {
        const int idx = tid + i * 256, row = 32 * bk + (idx >> 4), ch = idx & 15;
        if (row < nt)
          *(uint4*)(ql + ((size_t)(t0 + row) * H + h) * kDc + c0 + ch * 8) =
              *(const uint4*)(wl + row * kAbsRowB + abs_pos(ch, row));
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
  dim3 g(H, kDc / kAbsRows, (Tn + kAbsTok - 1) / kAbsTok);
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
