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
// trip serves all R rows. The loads (merge_issue) and the arithmetic
// (merge_finish) are separate steps, so a caller can have other work between
// them. Up to kMP parts (the local part included) are loaded ahead; more
// parts take merge_row, one row at a time. valid[r] false: row r is neither
// loaded nor merged. Rows must be the same for every lane of the wave.
constexpr int kFastParts = 8;

template <typename TP, int R, int kMP = kFastParts>
struct MergeLoads {
  float li[R];
  typename Vec8<TP>::v raw[R][kMP];
};

// the loads: LSE of part `lane` and every part's 8 values of each valid row
// (nothing when there are more than kMP parts)
template <typename TP, int R, int kMP>
__device__ __forceinline__ void merge_issue(const CombineParams& c, const size_t* row,
                                            const bool* valid, size_t rows, int lane,
                                            MergeLoads<TP, R, kMP>& ml) {
  typedef typename Vec8<TP>::v v8p;
  const int np = c.P + (c.local_out ? 1 : 0);
  if (np > kMP) return;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    ml.li[r] = -INFINITY;
    if (valid[r] && lane < np) ml.li[r] = part_lse(c, lane, row[r], rows);
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int k = 0; k < kMP; ++k)
      if (valid[r] && k < np) {
        const TP* src = k < c.P ? (const TP*)c.parts_out + ((size_t)k * rows + row[r]) * kDc
                                : (const TP*)c.local_out + row[r] * kDc;
        // the row's address is uniform: kept a scalar base, so only the lane
        // offset is a vector register (no per-part vector pointers); the load
        // is a global one (a flat load would also count against the LDS
        // counter and hold up the waits for LDS reads)
        asm volatile("" : "+s"(src));
        ml.raw[r][k] = *(const __attribute__((address_space(1))) v8p*)(src + lane * 8);
      }
}

// the arithmetic on the values merge_issue loaded (merge_row itself when
// there are more than kMP parts)
template <typename TP, int R, int kMP>
__device__ __forceinline__ void merge_finish(const CombineParams& c, const size_t* row,
                                             const bool* valid, size_t rows, int lane,
                                             const MergeLoads<TP, R, kMP>& ml, float (*o)[8],
                                             float* lse) {
  const int np = c.P + (c.local_out ? 1 : 0);
  if (np > kMP) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (valid[r]) lse[r] = merge_row<TP>(c, row[r], rows, lane, o[r]);
    return;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (!valid[r]) continue;
    const bool nan_seen = __builtin_amdgcn_ballot_w64(isnan(ml.li[r])) != 0;
    const float m = wave_max(ml.li[r]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float z = 0.f;
    if (m != -INFINITY && !nan_seen) {
      const float wl = ml.li[r] == -INFINITY ? 0.f : expf(ml.li[r] - m);
#pragma unroll
      for (int k = 0; k < kMP; ++k) {
        if (k < np) {
          const float w = __shfl(wl, k, 64);
          z += w;
          if (w != 0.f)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, (float)ml.raw[r][k][e], acc[e]);
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

// both steps at once
template <typename TP, int R>
__device__ __forceinline__ void merge_rows(const CombineParams& c, const size_t* row,
                                           const bool* valid, size_t rows, int lane,
                                           float (*o)[8], float* lse) {
  MergeLoads<TP, R, kFastParts> ml;
  merge_issue<TP, R, kFastParts>(c, row, valid, rows, lane, ml);
  merge_finish<TP, R, kFastParts>(c, row, valid, rows, lane, ml, o, lse);
}

template <typename TP, typename TO>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams c) {
  const int lane = threadIdx.x & 63;
  const size_t rows = (size_t)c.T * c.H;
  const size_t row = (size_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
// LSE combine fused with V-up. One workgroup of 16 waves per (head h, group
// of nbw consecutive blocks of kTb = 16 or 32 tokens). The groups of one head
// are consecutive workgroups of one XCD (workgroup i runs on XCD i mod 8),
// so they run together and read W_UV[h] from HBM once, through that XCD's L2.
// W_UV[h] (128 KB) goes to LDS by direct loads that waves 0-3, the matrix
// waves, issue at the start; the other waves never wait for it. Per block:
// every wave merges its rows of head h (the arithmetic of combine_kernel) and
// issues the loads of its rows of the next block at once, so they are in
// flight through the matrix phase; the merged rows, rounded to the compute
// type, go to LDS, and waves 0-3 each compute one 32-column v tile of
// out^T = W_UV[h]^T x^T on the matrix cores (W by transposed LDS reads, the
// k steps in order: the V-up kernel's products bit for bit). The merged
// latent never goes to HBM (unless lat_out asks for it).
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

constexpr int kCvWaves = 16;                 // rows merged concurrently
constexpr int kCvThreads = kCvWaves * 64;
constexpr int kCvWRow = kDv * 2;             // 256-byte W_UV rows in LDS
constexpr int kCvXRow = kDc * 2;             // 1 KB latent rows in LDS

// LDS chunk positions (16-byte chunks). W_UV row c: chunk k at k ^ 4 (c & 3),
// so the 4 rows x 4 chunks of a 32-lane transposed read cover the 64 banks
// once. Latent row t: chunk k at k ^ (t & 15), so the 16 rows of a 16-lane
// operand read do.
__device__ __forceinline__ int cvw_pos(int chunk, int row) {
  return (chunk ^ ((row & 3) << 2)) << 4;
}
__device__ __forceinline__ int cvx_pos(int chunk, int row) { return (chunk ^ (row & 15)) << 4; }

template <typename TP, typename T, int kTb, int kMP>
__global__ __launch_bounds__(kCvThreads) void combine_vup_kernel(CombineVupParams cv) {
  typedef typename CvT<T>::v8 v8;
  __shared__ __attribute__((aligned(1024))) char wl[kDc * kCvWRow];  // W_UV[h]
  __shared__ __attribute__((aligned(1024))) char xl[kTb * kCvXRow];  // the block's merged rows
  const CombineParams& c = cv.c;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int nb = (c.T + kTb - 1) / kTb;
  const int ng = (nb + cv.nbw - 1) / cv.nbw;
  const int n = c.H * ng;
  const int per = (n + 7) >> 3;
  const int u = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (u >= n) return;
  const int h = u / ng;
  const int b0 = (u - h * ng) * cv.nbw, b1 = min(nb, b0 + cv.nbw);
  const size_t rows = (size_t)c.T * c.H;

  // rows wave + 16 i of a block; 16-bit parts: all of them in flight together
  // (and the next block's during the matrix phase), fp32 parts one at a time
  constexpr int kR = kTb / kCvWaves;
  constexpr bool kAhead = sizeof(TP) == 2;
  size_t row[kR];
  bool valid[kR];
  MergeLoads<TP, kAhead ? kR : 1, kMP> ml;
  auto set_rows = [&](int b) {
    // (opaque to the loop optimiser: per-block addresses stay scalar bases
    // instead of becoming loop-carried vector pointers)
    const int t0 = __builtin_amdgcn_readfirstlane(b * kTb), nt = min(kTb, c.T - t0);
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const int r = wave + i * kCvWaves;
      valid[i] = r < nt;
      row[i] = (size_t)(t0 + (valid[i] ? r : 0)) * c.H + h;
    }
  };
  set_rows(b0);
  if constexpr (kAhead) merge_issue<TP, kR, kMP>(c, row, valid, rows, lane, ml);

  // W_UV[h]: 512 rows of 256 B, loaded by the matrix waves 0-3 (the other
  // waves then never wait for it). Load i of wave w fills LDS rows
  // 4 (32 w + i) .. + 3: lane l takes row 4 (32 w + i) + l / 16, position
  // l % 16, i.e. the row's chunk (l % 16) ^ 4 (row & 3).
  if (wave < 4) {
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const T*)cv.w_uv + (size_t)h * kDc * kDv), (short)0, kDc * kCvWRow,
        0x00020000);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int wrow = 4 * (32 * wave + i) + (lane >> 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (LDS_AS void*)(wl + (32 * wave + i) * 1024),
                                               16, wrow * kCvWRow + cvw_pos(lane & 15, wrow),
                                               0, 0, 0);
    }
  }

  const int r32 = lane & 31, hi = lane >> 5;
  const int j16 = lane & 15, g16 = lane >> 4;
  // A = W^T (rows v, k = c) by transposed reads: 16-lane group g16 covers
  // v 32 wave + 16 (g16 & 1) .. + 15 and c rows 8 (g16 >> 1) + 0..3 (then
  // + 4..7) of each 16-wide k step; a row's index mod 4 is j16 / 4
  const int a_off = (8 * (g16 >> 1) + (j16 >> 2)) * kCvWRow +
                    cvw_pos(4 * wave + 2 * (g16 & 1) + ((j16 & 3) >> 1), j16 >> 2) +
                    ((j16 & 1) << 3);
  // B = x^T column r32 (a 16-token block: columns 16..31 repeat rows 0..15;
  // their results are never stored)
  const int xrow = kTb == 32 ? r32 : (r32 & 15);

  for (int b = b0; b < b1; ++b) {
    // merge the block's rows (their loads are in flight), rounded to T as a
    // stored latent would be
    typename CvT<T>::v8 xr[kR];
    {
      float o[kR][8], lse[kR];
      if constexpr (kAhead) {
        merge_finish<TP, kR, kMP>(c, row, valid, rows, lane, ml, o, lse);
      } else {
#pragma unroll
        for (int i = 0; i < kR; ++i) {
          merge_issue<TP, 1, kMP>(c, &row[i], &valid[i], rows, lane, ml);
          merge_finish<TP, 1, kMP>(c, &row[i], &valid[i], rows, lane, ml, &o[i], &lse[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < kR; ++i) {
        if (!valid[i]) continue;
#pragma unroll
        for (int e = 0; e < 8; ++e) xr[i][e] = from_f<T>(o[i][e]);
        if (cv.lat_out) *(v8*)((T*)cv.lat_out + row[i] * kDc + lane * 8) = xr[i];
        if (c.lse_out && lane == 0) c.lse_out[row[i]] = lse[i];
      }
    }
    // the matrix waves wait for their W_UV rows before anything younger is issued
    if (b == b0 && wave < 4) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    // the next block's loads go out now, in flight through the matrix phase
    const int t0 = b * kTb, nt = min(kTb, c.T - t0);
    bool cur_valid[kR];
#pragma unroll
    for (int i = 0; i < kR; ++i) cur_valid[i] = valid[i];
    if (b + 1 < b1) {
      set_rows(b + 1);
      if constexpr (kAhead) merge_issue<TP, kR, kMP>(c, row, valid, rows, lane, ml);
    }
    if (b > b0) __syncthreads();  // every wave is done reading the previous block
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const int r = wave + i * kCvWaves;
      if (cur_valid[i]) *(v8*)(xl + r * kCvXRow + cvx_pos(lane, r)) = xr[i];
    }
    __syncthreads();
    if (wave < 4) {
      // the operand offsets are recomputed in every block (kept out of the
      // block loop, they would hold registers through the merge)
      int xb = xrow * kCvXRow, ab = a_off;
      asm volatile("" : "+v"(xb), "+v"(ab));
      floatx16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll 4
      for (int k = 0; k < kDc / 16; ++k) {
        const char* a0 = wl + ab + k * 16 * kCvWRow;
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)a0);
        const shortx4 h4 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)(a0 + 4 * kCvWRow));
        const v8 a = __builtin_bit_cast(v8, __builtin_shufflevector(lo, h4, 0, 1, 2, 3, 4, 5, 6, 7));
        const v8 bv = *(const v8*)(xl + xb + cvx_pos(2 * k + hi, xrow));
        acc = CvT<T>::mfma(a, bv, acc);
      }
      if (r32 < nt) {
        T* dst = (T*)cv.out + ((size_t)(t0 + r32) * c.H + h) * kDv + wave * 32 + 4 * hi;
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

template <typename TP, typename T, int kTb>
static void launch_combine_vup_mp(const CombineVupParams& cv, dim3 g, hipStream_t st) {
  // registers for the parts in flight: the smallest of 2, 4, 8 that holds
  // them (32-token blocks hold two rows per wave and stop at 4; the host
  // picks them only for up to 4 parts, more would merge row by row)
  const int np = cv.c.P + (cv.c.local_out ? 1 : 0);
  if (np <= 2)
    hipLaunchKernelGGL((combine_vup_kernel<TP, T, kTb, 2>), g, dim3(kCvThreads), 0, st, cv);
  else if (kTb == 32 || np <= 4)
    hipLaunchKernelGGL((combine_vup_kernel<TP, T, kTb, 4>), g, dim3(kCvThreads), 0, st, cv);
  else
    hipLaunchKernelGGL((combine_vup_kernel<TP, T, kTb, kTb == 32 ? 4 : 8>), g, dim3(kCvThreads),
                       0, st, cv);
}

template <typename TP, typename T>
static void launch_combine_vup_tb(const CombineVupParams& cv, dim3 g, hipStream_t st) {
  if (cv.tb == 16)
    launch_combine_vup_mp<TP, T, 16>(cv, g, st);
  else
    launch_combine_vup_mp<TP, T, 32>(cv, g, st);
}

template <typename TP>
static void launch_combine_vup_t(const CombineVupParams& cv, dim3 g, hipStream_t st) {
  if (cv.c.out_dtype == MLA_BF16)
    launch_combine_vup_tb<TP, bf16>(cv, g, st);
  else
    launch_combine_vup_tb<TP, f16>(cv, g, st);
}

hipError_t launch_combine_vup(const CombineVupParams& cv, hipStream_t st) {
  const long long nb = (cv.c.T + cv.tb - 1) / cv.tb;
  const long long n = (long long)cv.c.H * ((nb + cv.nbw - 1) / cv.nbw);
  dim3 g((unsigned)(8 * ((n + 7) / 8)));
  if (cv.c.part_dtype == MLA_F32) launch_combine_vup_t<float>(cv, g, st);
  else if (cv.c.part_dtype == MLA_BF16) launch_combine_vup_t<bf16>(cv, g, st);
  else launch_combine_vup_t<f16>(cv, g, st);
  return hipGetLastError();
}

}  // namespace mla
