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

// Merge of one (token, head) row by one wave: lane l returns the merged
// values 8 l .. 8 l + 7 in o[] and the row's LSE.
template <typename TP>
__device__ __forceinline__ float merge_row(const CombineParams& c, size_t row, size_t rows,
                                           int lane, float* o) {
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
  return lse;
}

// Merge of R rows by one wave with every load issued before the first use:
// lane i < np loads part i's LSE of each row, every lane loads its 8 values
// of every part of every row, then the rows are merged with exactly the
// arithmetic of merge_row (same order of the sums), so one memory round
// trip serves all R rows. Up to kFastParts parts (the local part included);
// more parts take merge_row, one row at a time. valid[r] false: row r is
// neither loaded nor merged.
constexpr int kFastParts = 8;

template <typename TP, int R>
__device__ __forceinline__ void merge_rows(const CombineParams& c, const size_t* row,
                                           const bool* valid, size_t rows, int lane,
                                           float (*o)[8], float* lse) {
  const int np = c.P + (c.local_out ? 1 : 0);
  if (np > kFastParts) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (valid[r]) lse[r] = merge_row<TP>(c, row[r], rows, lane, o[r]);
    return;
  }
  typedef typename Vec8<TP>::v v8p;
  float li[R];
  v8p raw[R][kFastParts];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    li[r] = -INFINITY;
    if (valid[r] && lane < np) li[r] = part_lse(c, lane, row[r], rows);
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int k = 0; k < kFastParts; ++k)
      if (valid[r] && k < np) {
        const TP* src = k < c.P ? (const TP*)c.parts_out + ((size_t)k * rows + row[r]) * kDc
                                : (const TP*)c.local_out + row[r] * kDc;
        raw[r][k] = *(const v8p*)(src + lane * 8);
      }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (!valid[r]) continue;
    const bool nan_seen = __builtin_amdgcn_ballot_w64(isnan(li[r])) != 0;
    const float m = wave_max(li[r]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float z = 0.f;
    if (m != -INFINITY && !nan_seen) {
      const float wl = li[r] == -INFINITY ? 0.f : expf(li[r] - m);
#pragma unroll
      for (int k = 0; k < kFastParts; ++k) {
        if (k < np) {
          const float w = __shfl(wl, k, 64);
          z += w;
          if (w != 0.f)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, (float)raw[r][k][e], acc[e]);
        }
      }
    }
    if (nan_seen) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][e] = NAN;
      lse[r] = NAN;
    } else if (z > 0.f) {
      const float inv = 1.f / z;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][e] = acc[e] * inv;
      lse[r] = m + logf(z);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][e] = 0.f;
      lse[r] = -INFINITY;
    }
  }
}

template <typename TP, typename TO>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams c) {
  const int lane = threadIdx.x & 63;
  const size_t rows = (size_t)c.T * c.H;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  float o[1][8], lse[1];
  const bool valid[1] = {true};
  merge_rows<TP, 1>(c, &row, valid, rows, lane, o, lse);
  store8<TO>((TO*)c.out + row * kDc + lane * 8, o[0]);
  if (c.lse_out && lane == 0) c.lse_out[row] = lse[0];
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

// ---------------------------------------------------------------------------
// LSE combine fused with V-up. One workgroup per (head h, block of tb <= 32
// tokens): its 4 waves merge the block's latent rows of head h (one row per
// wave at a time, as combine_kernel), round them to the compute type into
// LDS, then run out^T[v][t] = sum_c W_UV[h][c][v] x[t][c] on the matrix
// cores in two 64-column passes; W_UV[h] is loaded into registers before the
// merge, so its memory round trip overlaps the part reads. The merged latent
// never goes to HBM (unless lat_out asks for it).
// ---------------------------------------------------------------------------
#define LDS_AS __attribute__((address_space(3)))
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short shortx4 __attribute__((ext_vector_type(4)));

template <typename T> struct CvT;
template <> struct CvT<bf16> {
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  typedef __bf16 v4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ floatx16 mfma(v8 a, v8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct CvT<f16> {
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  typedef _Float16 v4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ floatx16 mfma(v8 a, v8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

constexpr int kCvCols = 64;                           // W_UV columns per pass
constexpr int kCvWRow = kCvCols * 2 + 32;             // LDS bytes per W row (padded)
constexpr int kCvXRow = kDc * 2 + 16;                 // LDS bytes per latent row (padded)
constexpr int kCvWaves = 16;                         // rows merged concurrently
constexpr int kCvThreads = kCvWaves * 64;
constexpr int kCvPieces = kDc * kCvCols * 2 / 16 / kCvThreads;  // 16-byte W pieces per thread per pass
static_assert(kCvPieces * kCvThreads * 16 == kDc * kCvCols * 2, "W pass split");

// kTb: tokens per workgroup (16 or 32), cv.tb
template <typename TP, typename T, int kTb>
__global__ __launch_bounds__(kCvThreads) void combine_vup_kernel(CombineVupParams cv) {
  typedef typename CvT<T>::v8 v8;
  __shared__ __attribute__((aligned(16))) char wl[kDc * kCvWRow];
  __shared__ __attribute__((aligned(16))) char xl[32 * kCvXRow];
  const CombineParams& c = cv.c;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x;
  const int t0 = blockIdx.y * kTb;
  const int nt = min(kTb, c.T - t0);
  const size_t rows = (size_t)c.T * c.H;

  // W_UV[h][:, 64 p .. 64 p + 63] for both passes p: 512 rows x 128 B each
  const T* wsrc = (const T*)cv.w_uv + (size_t)h * kDc * kDv;
  v8 st[2][kCvPieces];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int i = 0; i < kCvPieces; ++i) {
      const int idx = tid + i * kCvThreads, cc = idx >> 3, q = idx & 7;
      st[p][i] = *(const v8*)(wsrc + (size_t)cc * kDv + p * kCvCols + q * 8);
    }

  // merged latent rows of the block (wave w: rows w and, with 32 tokens,
  // w + 16, both in flight together for 16-bit parts, one after the other
  // for fp32 parts), rounded to T as a stored latent would be; the rows of
  // a 16-token block past 16 are zero
  constexpr int kRows = kTb / kCvWaves;                   // rows per wave
  constexpr int kR = sizeof(TP) == 4 ? 1 : kRows;         // rows in flight
  if (kTb < 32) {
    v8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (T)0.f;
#pragma unroll
    for (int r = kTb + wave; r < 32; r += kCvWaves) *(v8*)(xl + r * kCvXRow + lane * 16) = z;
  }
#pragma unroll
  for (int i0 = 0; i0 < kRows; i0 += kR) {
    size_t row[kR];
    bool valid[kR];
    float o[kR][8], lse[kR];
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const int r = wave + (i0 + i) * kCvWaves;
      valid[i] = r < nt;
      row[i] = (size_t)(t0 + (valid[i] ? r : 0)) * c.H + h;
    }
    merge_rows<TP, kR>(c, row, valid, rows, lane, o, lse);
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const int r = wave + (i0 + i) * kCvWaves;
      v8 xv;
      if (valid[i]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[e] = from_f<T>(o[i][e]);
        if (cv.lat_out) *(v8*)((T*)cv.lat_out + row[i] * kDc + lane * 8) = xv;
        if (c.lse_out && lane == 0) c.lse_out[row[i]] = lse[i];
      } else {
        // columns past the block: their products are never stored
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[e] = (T)0.f;
      }
      *(v8*)(xl + r * kCvXRow + lane * 16) = xv;
    }
  }

  const int r32 = lane & 31, hi = lane >> 5;
  const int j16 = lane & 15, g16 = lane >> 4;
  // A = W^T (rows v, k = c) by transposed reads: 16-lane block g16 covers
  // v 16 (g16 & 1) .. + 15 and c rows 8 (g16 >> 1) .. of each 16-wide k step
  const int a_off = ((8 * (g16 >> 1) + (j16 >> 2)) * kCvWRow) +
                    ((wave & 1) * 32 + 16 * (g16 & 1) + 4 * (j16 & 3)) * 2;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    if (p) __syncthreads();  // every wave is done reading the previous pass
#pragma unroll
    for (int i = 0; i < kCvPieces; ++i) {
      const int idx = tid + i * kCvThreads, cc = idx >> 3, q = idx & 7;
      *(v8*)(wl + cc * kCvWRow + q * 16) = st[p][i];
    }
    __syncthreads();
    // waves 0 and 1 take the pass's two 32-column tiles, B = x^T column t
    if (wave < 2) {
      floatx16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int k = 0; k < kDc / 16; ++k) {
        const char* a0 = wl + a_off + k * 16 * kCvWRow;
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)a0);
        const shortx4 h4 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)(a0 + 4 * kCvWRow));
        const v8 a = __builtin_bit_cast(v8, __builtin_shufflevector(lo, h4, 0, 1, 2, 3, 4, 5, 6, 7));
        const v8 b = *(const v8*)(xl + r32 * kCvXRow + (16 * k + 8 * hi) * 2);
        acc = CvT<T>::mfma(a, b, acc);
      }
      if (r32 < nt) {
        T* dst = (T*)cv.out + ((size_t)(t0 + r32) * c.H + h) * kDv + p * kCvCols + wave * 32 + 4 * hi;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          typename CvT<T>::v4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = from_f<T>(acc[4 * g + i]);
          *(typename CvT<T>::v4*)(dst + 8 * g) = v;
        }
      }
    }
  }
}

template <typename TP, typename T>
static void launch_combine_vup_tb(const CombineVupParams& cv, dim3 g, hipStream_t st) {
  if (cv.tb == 16)
    hipLaunchKernelGGL((combine_vup_kernel<TP, T, 16>), g, dim3(kCvThreads), 0, st, cv);
  else
    hipLaunchKernelGGL((combine_vup_kernel<TP, T, 32>), g, dim3(kCvThreads), 0, st, cv);
}

template <typename TP>
static void launch_combine_vup_t(const CombineVupParams& cv, dim3 g, hipStream_t st) {
  if (cv.c.out_dtype == MLA_BF16)
    launch_combine_vup_tb<TP, bf16>(cv, g, st);
  else
    launch_combine_vup_tb<TP, f16>(cv, g, st);
}

hipError_t launch_combine_vup(const CombineVupParams& cv, hipStream_t st) {
  dim3 g((unsigned)cv.c.H, (unsigned)((cv.c.T + cv.tb - 1) / cv.tb));
  if (cv.c.part_dtype == MLA_F32) launch_combine_vup_t<float>(cv, g, st);
  else if (cv.c.part_dtype == MLA_BF16) launch_combine_vup_t<bf16>(cv, g, st);
  else launch_combine_vup_t<f16>(cv, g, st);
  return hipGetLastError();
}

}  // namespace mla
