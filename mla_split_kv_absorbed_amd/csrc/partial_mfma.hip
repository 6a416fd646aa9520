// Split-KV partial attention on CDNA4 matrix cores (bf16 / fp16 in, fp32
// accumulate), the hot kernel of the decode step.
//
// Work decomposition. One workgroup owns one query token of one (part,
// sequence) range -- or one sub-range ("chunk") of it -- for 128 heads. All
// 128 heads share the latent cache, so each 576-wide key row is read from HBM
// once and used by every head: the head-batched products S^T = K . Q^T and
// O^T += C^T . P^T are real dense contractions (M = 32 tokens or 32 latent
// columns, N = 32 heads per wave, K = 576 dims or 32 tokens).
//
// Data flow per 32-token tile (one LDS stage of 32 x 576 x 2 B = 36 KB):
//   HBM --buffer_load_dwordx4 ... lds--> LDS ring (4 stages, no VGPRs used)
//   LDS --ds_read_b128--> key operand of S^T = K Q^T (32x32x16 MFMA, Q in VGPRs)
//   softmax in registers (each lane holds 16 tokens of one head; exponent
//   reference from the chunk's first tile, below) --> weights P to LDS
//   LDS --ds_read_b64_tr_b16--> transposed value operand of O^T += C^T P^T
// LDS layout of a stage is row-major, 1152 bytes per key row, with the 16-byte
// chunks of row r permuted within each 128-byte group: chunk c sits at
// position c ^ swz(r). Every LDS-direct load instruction then reads 1 KB of
// contiguous HBM (whole cache lines) and both operand read patterns are free
// of bank conflicts (see swz).
//
// Each wave owns 32 heads for the score product: Q^T for them stays in 144
// VGPRs. The softmax weights of all heads then go through an 8 KB LDS buffer
// and each wave runs the value product for all 128 heads over its own 128
// latent columns, so every transposed value operand feeds 4 matrix
// instructions; the fp32 output O^T (128 x 128 per wave) stays in 256
// accumulation registers (AGPRs).
//
// Softmax without rescaling the accumulators. Weights are 2^(score - ref)
// in log2 units with a fixed exponent reference per head and chunk.
// Floating-point results are invariant under a common scale (the output is
// divided by the same sum, the LSE adds the reference back), so this equals
// the rescaled online softmax as long as the weights neither overflow nor
// lose the dominant term, which depends on the weight type:
//  - bf16 weights share fp32's exponent range: the reference is 0 and every
//    head's maximum may lie anywhere in [-64, 64] (weights <= 2^64, the
//    largest >= 2^-64);
//  - fp16 weights overflow above 65504 and lose precision below 2^-14: the
//    reference is each head's maximum over the chunk's first tile (kept in
//    LDS, so the loop holds no extra register), and later scores may exceed
//    it by at most 15 (weights <= 2^15; the dominant weight is >= 1).
// A chunk where some head's maximum leaves its window is replayed once with
// each head's exact maximum as the reference (weights <= 1). The hot loop
// therefore never touches the output accumulators outside the matrix
// instructions and needs no cross-lane maximum per tile.
//
// Heads come in groups of 128 (blockIdx.y): a group with fewer than 128
// real heads (H not a multiple of 128) runs with zero queries in the missing
// rows, whose results are never stored. The keys are read once per group.
//
// Step j of the tile loop: wait for tile j's loads and barrier; the score
// product of tile j (one accumulation chain, key operands read 8 instructions
// ahead), behind the value-product group carried over from the previous step;
// the value product of tile j - 1 with tile j's softmax interleaved; barrier;
// tile j's weights go to LDS between the instructions of one more value
// group, and the last group is carried across the next barrier so the matrix
// unit has work while the first key operands load. The loads of tile j + 2
// are spread over the score product.
//
// Ranges that need splitting (few sequences, long ranges) are cut into
// chunks; chunk results go to a workspace (outputs in the output type, LSEs
// in fp32) and a second kernel merges them by LSE in a fixed order. The
// chunks come from an in-kernel plan, or, with an explicit split count, from
// a closed form that needs no plan.
#include "common.h"
#include "short.h"
#include "kernels.h"

#include <algorithm>
#include <cstring>
#include <type_traits>

namespace mla {

#define LDS_AS __attribute__((address_space(3)))

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;                      // 4 x 32 heads = 128 heads per group
constexpr int kHeadsWave = 32;
constexpr int kHeadsGroup = kWaves * kHeadsWave;
constexpr int kStages = 4;
constexpr int kAheadTiles = kStages - 2;       // tiles in flight (one stage computes, one
                                               // holds the previous tile for its value product)
constexpr int kRowBytes = kRow * 2;            // 1152
constexpr int kChunksRow = kRowBytes / 16;     // 72
constexpr int kStageBytes = kTile * kRowBytes; // 36864
constexpr int kLoadsWave = kStageBytes / 16 / 64 / kWaves;  // 9
constexpr int kKSteps = kRow / 16;             // 36
constexpr int kDTiles = kDc / 32;              // 16
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kIdCache = 256;                  // block ids staged in LDS per refill

// chunk permutation inside a row: position = chunk ^ swz(row). The LDS has
// 64 four-byte banks; a 16-byte read serves 16 lanes per cycle and the 8-byte
// transposed read 32 lanes. swz gives the 8 even (and the 8 odd) rows of any
// 16 consecutive rows distinct positions, so the 16 rows of a key-operand
// read cover all 64 banks once, and it makes rows 4m and 4m+2 differ in
// position bit 2, so the 4 rows x 2 chunks of a transposed read do too
// (both measured conflict-free with the SQ_LDS_BANK_CONFLICT counter).
__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// Weight buffer: one 64-byte row of 32 tokens per head; chunk c (tokens
// 8c .. 8c + 7) of head h sits at position c ^ ((h >> 2) & 3). The 16 lanes
// of a 16-byte read (16 consecutive heads, one chunk) then cover all 64
// banks.
constexpr int kPRow = kTile * 2;  // 64 bytes
__device__ __forceinline__ int pchunk(int c, int h) { return c ^ ((h >> 2) & 3); }

static_assert(kLoadsWave * 64 * 16 * kWaves == kStageBytes, "stage load split");
static_assert(2 * kLoadsWave < 64, "vmcnt range");


// s_waitcnt vmcnt(n) with expcnt / lgkmcnt unconstrained (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14)
#define MLA_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | 0x0F70)

// Wait until the LDS-direct loads of the current tile have landed. Per tile a
// wave issues kLoadsWave loads; n_after = number of tiles issued after the
// current one (loads complete in issue order).
__device__ __forceinline__ void wait_vm(int n_after) {
  if (n_after >= 2) __builtin_amdgcn_s_waitcnt(MLA_VMCNT(2 * kLoadsWave));
  else if (n_after == 1) __builtin_amdgcn_s_waitcnt(MLA_VMCNT(kLoadsWave));
  else __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
}
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0)); }

// The key-score product S^T = K Q^T is issued as inline assembly with its
// accumulator pinned to VGPRs, so that the 256 fp32 output accumulators of
// the value product (compiler-issued, AGPR form) and the 144 registers of
// Q^T fit the register file together. The compiler does not model the
// latency of these instructions: reading the scores with vector ALU
// instructions is preceded by qk_drain(), which covers the result latency
// of the last ones and carries the accumulators as operands.
template <typename T> struct MT;
template <> struct MT<bf16> {
  typedef bf16x8 v8;
  // first pass: reference 0, head maxima within [-kWindow, kWindow]
  static constexpr bool kTileRef = false;
  static constexpr float kWindow = 64.0f;
  static __device__ __forceinline__ floatx16 mfma(v8 a, v8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ void qk_first(floatx16& acc, v8 a, v8 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  }
  // c + a.x + a.y in one dot instruction
  static __device__ __forceinline__ float sum2(bf16x2 a, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, (bf16x2){(bf16)1.f, (bf16)1.f}, c, false);
  }
  static __device__ __forceinline__ void qk_next(floatx16& acc, v8 a, v8 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
  }
};
template <> struct MT<f16> {
  typedef f16x8 v8;
  // first pass: the first tile's maxima, later maxima at most kWindow above
  static constexpr bool kTileRef = true;
  static constexpr float kWindow = 15.0f;  // 2^15 < 65504
  static __device__ __forceinline__ floatx16 mfma(v8 a, v8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ void qk_first(floatx16& acc, v8 a, v8 b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ float sum2(f16x2 a, float c) {
    return __builtin_amdgcn_fdot2(a, (f16x2){(f16)1.f, (f16)1.f}, c, false);
  }
  static __device__ __forceinline__ void qk_next(floatx16& acc, v8 a, v8 b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
  }
};

// Wait states after the last score products before any other instruction
// reads their results (more than the 8-pass result latency rule requires).
// The accumulators are in/out operands, so no reader can be scheduled above.
__device__ __forceinline__ void qk_drain(floatx16& a) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a)::"memory");
}

// ---------------------------------------------------------------------------
// the plan: tiles, chunks and split slots of one call, computed in-kernel
// ---------------------------------------------------------------------------

struct Unit {
  int st, en;
  bool bad;
  int nt;
};

__device__ __forceinline__ Unit load_unit(const PartialParams& pp, int u) {
  Unit x;
  x.st = pp.range_start[u];
  x.en = pp.range_end[u];
  x.bad = range_bad(x.st, x.en, pp.capacity);
  x.nt = x.bad ? 0 : range_tiles(x.st, x.en);
  return x;
}

// Block-wide exclusive scans over the 256 threads: prefix sums within each
// wave by shuffles, then one LDS exchange of the 4 wave totals (2 barriers
// per call). `sh` holds at least 4 * N ints.
template <int N>
__device__ __forceinline__ void block_excl_scan(const int (&v)[N], int* sh, int (&base)[N],
                                                int (&total)[N]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc[N];
#pragma unroll
  for (int k = 0; k < N; ++k) inc[k] = v[k];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const int x = __shfl_up(inc[k], o, 64);
      if (lane >= o) inc[k] += x;
    }
  }
  if (lane == 63)
#pragma unroll
    for (int k = 0; k < N; ++k) sh[wave * N + k] = inc[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < N; ++k) {
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int t = sh[w * N + k];
      before += w < wave ? t : 0;
      all += t;
    }
    base[k] = before + inc[k] - v[k];
    total[k] = all;
  }
  __syncthreads();
}

struct Plan {
  int chunk_tiles;   // c
  int nchunks;       // total chunks
  int nsplit_units;  // units cut into more than one chunk
};

// Computes the plan; if `want` >= 0, also finds chunk `want`:
// found = {unit, first tile, end tile, slot (-1 = direct), chunk count of
// the unit, split index, the unit's range}
struct Found {
  int u, tb, te, slot, nsplit, split_idx, st, en;
};

// units per thread whose ranges stay in registers through the plan
constexpr int kPlanCache = 4;

// The automatic plan on the device, by the whole workgroup (block scans over
// the ranges; chunk ids longest first by the buckets of plan.h, range order
// within a bucket; slots and split indices in range order).
__device__ __forceinline__ Plan make_plan(const PartialParams& pp, int want, Found* found, int* sh) {
  const int tid = threadIdx.x;
  const int U = pp.P * pp.B;
  const int per = (U + 255) / 256;
  const int u0 = min(U, tid * per), u1 = min(U, u0 + per);
  // this thread's units: the first kPlanCache are loaded once
  Unit uc[kPlanCache];
#pragma unroll
  for (int i = 0; i < kPlanCache; ++i) {
    uc[i].nt = 0;
    if (u0 + i < u1) uc[i] = load_unit(pp, u0 + i);
  }
  auto unit_at = [&](int i) __attribute__((always_inline)) -> Unit {
    if (i < kPlanCache) {
      Unit x = uc[0];
#pragma unroll
      for (int k = 1; k < kPlanCache; ++k)
        if (i == k) x = uc[k];
      return x;
    }
    return load_unit(pp, u0 + i);
  };
  long long my_tiles = 0;
  for (int i = 0; i < u1 - u0; ++i) my_tiles += unit_at(i).nt;
  // total tiles (fits in int for any addressable cache)
  int tv[1] = {(int)my_tiles}, tb_[1], tt[1];
  block_excl_scan<1>(tv, sh, tb_, tt);
  const int total = tt[0];
  Plan pl;
  // the chunk size of the split rule (plan.h): c0, or the two-round c1
  int c = chunk_tiles_one_round(total, pp.S);
  {
    const int c1 = chunk_tiles_two_round(total, pp.S, U);
    if (c1 > 0 && c1 < c) {
      int nv[2] = {0, 0}, nb[2], ntot[2];
      for (int i = 0; i < u1 - u0; ++i) {
        const int nt = unit_at(i).nt;
        nv[0] += unit_chunks(nt, c, 0);
        nv[1] += unit_chunks(nt, c1, 0);
      }
      block_excl_scan<2>(nv, sh, nb, ntot);
      if (take_two_round(c, c1, ntot[0], ntot[1], pp.S)) c = c1;
    }
  }
  pl.chunk_tiles = c;
  // per bucket chunk counts of this thread, plus all chunks, split slots and
  // split units
  int mv[kBuckets + 3];
#pragma unroll
  for (int k = 0; k < kBuckets + 3; ++k) mv[k] = 0;
  for (int i = 0; i < u1 - u0; ++i) {
    const Unit x = unit_at(i);
    const int n = unit_chunks(x.nt, c, pp.num_splits);
    const int bk = len_bucket((x.nt + n - 1) / n, c);
#pragma unroll
    for (int k = 0; k < kBuckets; ++k)
      if (bk == k) mv[k] += n;
    mv[kBuckets] += n;
    if (n > 1) {
      mv[kBuckets + 1] += n;
      mv[kBuckets + 2] += 1;
    }
  }
  int mb[kBuckets + 3], mt[kBuckets + 3];
  block_excl_scan<kBuckets + 3>(mv, sh, mb, mt);
  pl.nchunks = mt[kBuckets];
  pl.nsplit_units = mt[kBuckets + 2];
  if (want < 0 || want >= pl.nchunks) return pl;  // grid slack: nothing to find
  // first chunk id of a bucket: the chunks of all longer buckets come first
  int run[kBuckets];
#pragma unroll
  for (int k = 0; k < kBuckets; ++k) {
    int above = 0;
#pragma unroll
    for (int k2 = k + 1; k2 < kBuckets; ++k2) above += mt[k2];
    run[k] = above + mb[k];
  }
  {
    int soff = mb[kBuckets + 1], poff = mb[kBuckets + 2];
    for (int i = 0; i < u1 - u0; ++i) {
      const Unit x = unit_at(i);
      const int n = unit_chunks(x.nt, c, pp.num_splits);
      const int bk = len_bucket((x.nt + n - 1) / n, c);
      int off = run[0];
#pragma unroll
      for (int k = 1; k < kBuckets; ++k)
        if (bk == k) off = run[k];
#pragma unroll
      for (int k = 0; k < kBuckets; ++k)
        if (bk == k) run[k] += n;
      if (want >= off && want < off + n) {
        const int k = want - off;
        found->u = u0 + i;
        found->tb = piece_tile(k, x.nt, n);
        found->te = piece_tile(k + 1, x.nt, n);
        found->slot = n > 1 ? soff + k : -1;
        found->nsplit = n;
        found->split_idx = n > 1 ? poff : -1;
        found->st = x.st;
        found->en = x.en;
        break;
      }
      if (n > 1) {
        soff += n;
        poff += 1;
      }
    }
  }
  return pl;
}

// workspace layout: [count | pad 256][split descriptors U x int4][lse fp32][out,
// in the output type]
struct WsLayout {
  size_t desc_off, lse_off, out_off, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline size_t slots_bound(int B, int S, int P, int hint) {
  return (size_t)plan_max_split_slots((long long)P * B, S, hint);
}

__host__ __device__ inline WsLayout ws_layout(int B, int S, int H, int P, int hint, int out_dtype) {
  WsLayout w;
  const size_t U = (size_t)P * B;
  const size_t rows = slots_bound(B, S, P, hint) * S * H;
  w.desc_off = 256;
  w.lse_off = align256(w.desc_off + U * 16);
  w.out_off = align256(w.lse_off + rows * 4);
  w.total = align256(w.out_off + rows * kDc * (out_dtype == MLA_F32 ? 4 : 2));
  return w;
}

// ---------------------------------------------------------------------------
// the main kernel
// ---------------------------------------------------------------------------

struct MfmaParams {
  PartialParams pp;
  int* ws_count;
  intx4* ws_desc;
  // a combined launch (mla_decode_partial_pair): workgroups from cur_x0 on
  // (head group 0 only) run the short-range call `cur`, kPairHeads heads per
  // wave task; cur_x0 = 0 when there is none
  PartialParams cur;
  int cur_x0;
  long long cur_tasks;
};

// heads per wave task of the current-chunk call in a combined launch: small
// workgroups pack into the history's ragged end (4 and 8 measured alike, 16
// and 1 slower)
constexpr int kPairHeads = 4;

// One LDS-direct load: 64 lanes x 16 bytes from the buffer `rs` at
// voffset + soffset into LDS [m0, m0 + 1024) (lane i lands at m0 + 16 i).
// Issued as assembly so that the compiler adds no waits of its own for these
// loads; the tile pipeline waits for them explicitly (wait_vm + barrier).
// M0 is written here and nothing else in the kernel uses it.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rs, unsigned m0, int voffset,
                                           int soffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voffset), "s"(rs), "s"(soffset)
               : "memory");
}

// kOneGroup: H == 128, one group of real heads (no head bound checks);
// kPair: a combined launch with a current-chunk call (MfmaParams::cur)
template <typename T, bool kOneGroup, bool kPair>
__global__ __launch_bounds__(256, 1) void partial_mfma_kernel(MfmaParams mp) {
  const PartialParams& pp = mp.pp;
  typedef typename MT<T>::v8 v8;
  // the LDS ring: kStages stages of one 32-token tile each
  __shared__ __attribute__((aligned(1024))) char lds[kStages * kStageBytes];
  __shared__ int sh_scan[256];
  __shared__ Found sh_found;
  __shared__ int sh_redo;
  __shared__ int sh_ids[kIdCache];  // first cache row of tiles [id_base, id_base + 256)
  // softmax weights of the current tile, all heads: [head][32 tokens] bf16 /
  // fp16, 16-byte chunks permuted by pchunk
  __shared__ __attribute__((aligned(16))) char sh_p[kHeadsGroup * kPRow];
  __shared__ float sh_inv[kHeadsGroup];
  __shared__ float sh_mref[kHeadsGroup];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = pp.S;

  // A combined launch: the workgroups past the history chunks run the
  // current-chunk call. They come last in dispatch order, so they fill the
  // compute units that the history's longest-first schedule frees at its end.
  if constexpr (kPair) {
    if ((int)blockIdx.x >= mp.cur_x0) {
      if (blockIdx.y == 0) {
        const long long task = (long long)(blockIdx.x - mp.cur_x0) * 4 +
                               __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        if (task < mp.cur_tasks) short_task<T, kPairHeads>(mp.cur, task, threadIdx.x & 63);
      }
      return;
    }
  }

  // blockIdx -> (chunk, query): the S queries of one chunk sit 8 ids apart,
  // i.e. on the same XCD, so their shared key tiles meet in one L2
  int chunk, s;
  if (S == 1) {
    chunk = blockIdx.x;
    s = 0;
  } else {
    const int grp = blockIdx.x / (8 * S), r = blockIdx.x % (8 * S);
    chunk = grp * 8 + (r & 7);
    s = r >> 3;
  }
  if (tid == 0) {
    sh_found.u = -1;
    sh_redo = 0;
  }
  // ---- Q^T for this wave's 32 heads, in registers -------------------------
  // requested as soon as the range index is known, ahead of the range's own
  // round trip (lane quantities read afresh here: the per-lane constants
  // below keep their own definitions for the tile loop's address arithmetic)
  v8 q[kKSteps];
  auto load_q = [&](int u) __attribute__((always_inline)) {
    const int ql_lane = threadIdx.x & 63;
    const int qhi = ql_lane >> 5;
    const int qhead =
        __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * kHeadsWave + (ql_lane & 31);
    const int qhead0 = kOneGroup ? 0 : blockIdx.y * kHeadsGroup;
    const bool qok = kOneGroup || qhead0 + qhead < pp.H;
    // a missing head (beyond H) loads a real row and zeroes it: every lane
    // issues the same loads
    const int tq = (u % pp.B) * S + s;
    const int hq = qok ? qhead0 + qhead : pp.H - 1;
    const T* ql = (const T*)pp.q_lat + ((size_t)tq * pp.H + hq) * kDc;
    const T* qr = (const T*)pp.q_rope + ((size_t)tq * pp.H + hq) * kDr;
#pragma unroll
    for (int k = 0; k < kKSteps; ++k) {
      const int d = k * 16 + qhi * 8;
      q[k] = d < kDc ? *(const v8*)(ql + d) : *(const v8*)(qr + (d - kDc));
    }
    if (!qok)
#pragma unroll
      for (int k = 0; k < kKSteps; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) q[k][i] = (T)0.f;
  };
  Found fd;
  bool first;  // this piece is the first of its range
  if (pp.plan) {
    // A plan built on the host: this chunk's entry. Every field is checked
    // against the arguments (the range is read from the range arrays, the
    // tiles clamped to it, the slot to the workspace), so a table that does
    // not belong to them gives wrong results but no access out of bounds.
    if (chunk >= pp.plan_chunks) return;  // grid slack
    const int* e = pp.plan + kPlanHeader + (size_t)chunk * kPlanEntry;
    const int u = __builtin_amdgcn_readfirstlane(e[0]);
    if (u < 0 || u >= pp.P * pp.B) return;
    load_q(u);
    const Unit x = load_unit(pp, u);
    const int tb = min(max(__builtin_amdgcn_readfirstlane(e[1]), 0), x.nt);
    const int te = min(max(__builtin_amdgcn_readfirstlane(e[2]), tb), x.nt);
    int slot = __builtin_amdgcn_readfirstlane(e[3]);
    if (slot < 0 || slot >= plan_max_split_slots((long long)pp.P * pp.B, S, pp.num_splits))
      slot = -1;
    fd.u = u;
    fd.tb = tb;
    fd.te = te;
    fd.slot = slot;
    fd.nsplit = 0;
    fd.split_idx = -1;  // the cut ranges' descriptors are in the plan
    fd.st = x.st;
    fd.en = x.en;
    first = false;
    __syncthreads();
  } else if (pp.num_splits > 0) {
    // An explicit count k: every range is cut into exactly k chunks (some
    // may be empty), so the plan has a closed form and its scans are
    // skipped. Chunk i of range u covers tiles [i nt / k, (i + 1) nt / k) of
    // that range, its result goes to slot u k + i, and range u is split
    // unit u. (The host passes k for ranges of equal length, where
    // longest-first ordering changes nothing.) Chunk c runs on XCD c mod 8;
    // when the range count is a multiple of 8, the k chunks of a range all
    // get the same residue (c = x + 8 (k (u div 8) + i), x = u mod 8), so the
    // rows of Q they share are fetched into one L2. Otherwise chunks follow
    // range order (c = u k + i). With k = 1 both orders are the identity.
    const int k = pp.num_splits;
    const int nunits = pp.P * pp.B;
    if (chunk >= nunits * k) return;  // grid slack
    int u, i;
    if ((nunits & 7) == 0) {
      const int pos = chunk >> 3;  // position among the chunks of XCD chunk & 7
      u = (chunk & 7) + 8 * (pos / k);
      i = pos % k;
    } else {
      u = chunk / k;
      i = chunk % k;
    }
    load_q(u);
    const Unit x = load_unit(pp, u);
    fd.u = u;
    fd.tb = piece_tile(i, x.nt, k);
    fd.te = piece_tile(i + 1, x.nt, k);
    fd.slot = k > 1 ? u * k + i : -1;
    fd.nsplit = k;
    fd.split_idx = k > 1 ? u : -1;
    fd.st = x.st;
    fd.en = x.en;
    // a range shorter than k tiles has several pieces that start at tile 0:
    // piece 0 alone is the first
    first = i == 0;
    if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) *mp.ws_count = k > 1 ? pp.P * pp.B : 0;
    __syncthreads();
  } else {
    __syncthreads();
    const Plan pl = make_plan(pp, chunk, &sh_found, sh_scan);
    __syncthreads();
    if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) *mp.ws_count = pl.nsplit_units;
    fd.u = __builtin_amdgcn_readfirstlane(sh_found.u);
    if (fd.u < 0) return;  // grid slack beyond the plan's chunks
    load_q(fd.u);
    fd.tb = __builtin_amdgcn_readfirstlane(sh_found.tb);
    fd.te = __builtin_amdgcn_readfirstlane(sh_found.te);
    fd.slot = __builtin_amdgcn_readfirstlane(sh_found.slot);
    fd.nsplit = __builtin_amdgcn_readfirstlane(sh_found.nsplit);
    fd.split_idx = __builtin_amdgcn_readfirstlane(sh_found.split_idx);
    fd.st = __builtin_amdgcn_readfirstlane(sh_found.st);
    fd.en = __builtin_amdgcn_readfirstlane(sh_found.en);
    // the plan gives every chunk at least one tile: only chunk 0 starts at 0
    first = fd.tb == 0;
  }

  const int p = fd.u / pp.B, b = fd.u % pp.B;
  const int t = b * S + s;
  const int Tq = pp.B * S;
  const int st = fd.st;
  const int en = fd.en;
  const bool unit_bad = range_bad(st, en, pp.capacity);
  int vend = en;
  if (pp.mask == MLA_MASK_CAUSAL_WINDOW) vend = min(en, en - S + s + 1);
  // the first piece of a split range records where its pieces' results live
  if (fd.split_idx >= 0 && first && s == 0 && blockIdx.y == 0 && tid == 0)
    mp.ws_desc[fd.split_idx] = intx4{fd.u, fd.slot, fd.nsplit, 0};

  // ---- per-lane constants -------------------------------------------------
  const int hi = lane >> 5;          // 0/1: which half of a 16-wide k step
  const int r32 = lane & 31;         // key row (QK) / head column
  const int head = wave * kHeadsWave + r32;  // head within the group
  const int head0 = kOneGroup ? 0 : blockIdx.y * kHeadsGroup;  // the group's first head
  const bool head_ok = kOneGroup || head0 + head < pp.H;
  // key operand of k step k: row r32, chunk 2k + hi, at
  // qk_off[k & 3] + (k >> 2) * 128
  int qk_off[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) qk_off[m] = r32 * kRowBytes + (((2 * m + hi) ^ swz(r32)) << 4);
  // value operand (transposed read) of latent tile dt (this wave's columns
  // 128 wave + 32 dt ..) and token half kk: 16-lane group g16 reads rows
  // 16 kk + 8 hi + 4 f + q4 (f = 0, 1: the two reads, k = 8 hi + 4 f + e is
  // token 16 kk + k) and chunk 16 wave + 4 dt + 2 (g16 & 1) + (j16 & 3) / 2,
  // at pv_off[dt & 1][f] + (dt >> 1) * 128 + 16 kk * 1152
  const int j16 = lane & 15, g16 = lane >> 4, q4 = j16 >> 2;
  int pv_off[2][2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int row = 8 * hi + 4 * f + q4;
      const int c = 16 * wave + 4 * e + 2 * (g16 & 1) + ((j16 & 3) >> 1);
      pv_off[e][f] = row * kRowBytes + ((c ^ swz(row)) << 4) + ((j16 & 1) << 3);
    }
  // weight operand P^T of head group g, token half kk: head 32 g + r32,
  // tokens 16 kk + 8 hi .. + 7, at pw_off[kk] + g * 32 * kPRow
  int pw_off[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) pw_off[kk] = r32 * kPRow + (pchunk(2 * kk + hi, r32) << 4);
  // this wave's softmax weights of head `head`, tokens 8 j + 4 hi .. + 3, go
  // to pst_off + (pchunk(j, r32) << 4)
  const int pst_off = head * kPRow + 8 * hi;
  // LDS-direct loads: load i of this wave fills slots (9 wave + i) * 64 + lane,
  // slot = row * 72 + position; the source is that row's chunk position ^ swz(row)
  int ld_off[kLoadsWave];
#pragma unroll
  for (int i = 0; i < kLoadsWave; ++i) {
    const int slot = (wave * kLoadsWave + i) * 64 + lane;
    const int r = slot / kChunksRow, pos = slot % kChunksRow;
    ld_off[i] = r * kRowBytes + ((pos ^ swz(r)) << 4);
  }
  const unsigned lds_base =
      __builtin_amdgcn_readfirstlane((unsigned)(size_t)(LDS_AS char*)lds);

  // The Q loads complete at the row table's wait (fill_rows), before the
  // first tile load: with nothing pending at loop entry the compiler places
  // no vmcnt waits of its own inside the tile loop (it cannot see the
  // LDS-direct loads, and a wait for an early Q load would otherwise drain
  // every tile in flight).

  floatx16 o[kDTiles];
#pragma unroll
  for (int i = 0; i < kDTiles; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[i][j] = 0.f;
  // The head's exponent reference (log2 units): bf16 keeps it in m_ref (0
  // on the first pass), fp16 in sh_mref (the maximum over the chunk's first
  // tile); on a replay, the head's exact maximum. m_seen: the running
  // maximum of the raw scores, for the replay decision.
  float m_ref = 0.f, m_seen = -INFINITY, l_part = 0.f, l_round = 0.f;
  auto ref = [&]() __attribute__((always_inline)) -> float {
    if constexpr (MT<T>::kTileRef)
      return sh_mref[head];
    else
      return m_ref;
  };
  bool bad = unit_bad;
  const float sl2 = pp.scale * kLog2e;

  const int tb = fd.tb, te = unit_bad ? fd.tb : fd.te;
  const int st_tile = st / kTile;
  const char* kvb = (const char*)pp.kv;
  // scalars used inside the tile lambdas (keeps the argument block out of
  // private memory)
  const int block_size = pp.block_size, max_blocks = pp.max_blocks;
  const int num_blocks = pp.num_blocks, kv_seq_stride = pp.kv_seq_stride;

  // tile j of the range: first token, and the LDS-direct loads of its rows
  auto tile_tok0 = [&](int j) __attribute__((always_inline)) {
    return j == 0 ? st : (st_tile + j) * kTile;
  };
  // The first cache row (block id * block size + slot, or the contiguous row)
  // of each of the chunk's tiles is staged in LDS by vector code, kIdCache
  // tiles per refill, so the tile loop does no division and no scalar loads
  // (whose out-of-order return would stall every LDS wait behind them).
  // -1 marks a tile past the range or a bad block id.
  int id_base = tb;
  auto fill_rows = [&](int from) __attribute__((always_inline)) {
    __syncthreads();
    for (int i = tid; i < kIdCache; i += 256) {
      const int j = from + i;
      int row = -1;
      if (j < te) {
        const int tok0 = tile_tok0(j);
        if (block_size > 0) {
          const int id = pp.block_table[(size_t)b * max_blocks + tok0 / block_size];
          if (id >= 0 && id < num_blocks) row = id * block_size + tok0 % block_size;
        } else {
          row = b * kv_seq_stride + tok0;
        }
      }
      sh_ids[i] = row;
    }
    wait_vm_all();
    __syncthreads();
  };
  int seg_end = te;  // end of the current segment (pipeline bound)
  auto tile_row = [&](int j) __attribute__((always_inline)) -> int {
    if (j >= seg_end) return -1;
    return __builtin_amdgcn_readfirstlane(sh_ids[j - id_base]);
  };
  // buffer resource over the rows of tile j starting at cache row `row`
  // (zero rows past the range or for a bad block id: those loads return zeros
  // without touching memory)
  auto tile_rsrc = [&](int j, int row) __attribute__((always_inline)) {
    const char* base = kvb;
    int nrows = 0;
    if (j < te) {
      if (row < 0) {
        bad = true;
      } else {
        base = kvb + (size_t)(unsigned)row * kRowBytes;
        nrows = min(en, (st_tile + j + 1) * kTile) - tile_tok0(j);
      }
    }
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nrows * kRowBytes,
                                             0x00020000);
  };
  // LDS-direct loads of tile j into `stage` (prologue)
  auto issue = [&](int j, int stage, int id) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(j, id);
    const unsigned m0 = lds_base + stage * kStageBytes + wave * kLoadsWave * 1024;
#pragma unroll
    for (int i = 0; i < kLoadsWave; ++i) lds_load16(rs, m0 + i * 1024, ld_off[i], 0);
  };
  // the first row of the next tile to issue is known one step ahead; the
  // row after it is read from LDS one more step ahead (pend_row), so the
  // read's latency never stalls a step
  int next_id = -1;
  int pend_row = -1;

  typedef T t2 __attribute__((ext_vector_type(2)));
  typedef T t4 __attribute__((ext_vector_type(4)));

  // O^T += C^T . P^T for this wave's 128 latent columns and all 128 heads,
  // C from the stage at `pb`, P^T from sh_p: per token half, 4 value
  // operands (transposed reads) times 4 weight operands, each value operand
  // feeding 4 instructions into different accumulators. With `soft`, the
  // softmax weights of the next tile (raw sums `sacc`) are computed in
  // between, so their vector work runs in the shadow of the matrix
  // instructions; they are returned packed in `pk`.
  // operands of the value product: C^T (transposed reads of the stage at
  // `pb`) and P^T (from sh_p)
  auto vload = [&](const char* pb, int dt, int kk) __attribute__((always_inline)) {
    const char* a0 = pb + (dt >> 1) * 128 + 16 * kk * kRowBytes;
    const shortx4 lo =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)(a0 + pv_off[dt & 1][0]));
    const shortx4 h4 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)(a0 + pv_off[dt & 1][1]));
    return __builtin_bit_cast(v8, __builtin_shufflevector(lo, h4, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto wload = [&](int g, int kk) __attribute__((always_inline)) {
    return *(const v8*)(sh_p + pw_off[kk] + g * kHeadsWave * kPRow);
  };

  // O^T += C^T . P^T for this wave's 128 latent columns and all 128 heads,
  // C from the stage at `pb`, P^T from sh_p: per token half, 4 value
  // operands (transposed reads) times 4 weight operands, each value operand
  // feeding 4 instructions into different accumulators. The first operands
  // (weights of token half 0, value operands 0 and 1) arrive in `wb0` /
  // `va01`, loaded during the preceding score product. With `soft`, the
  // softmax weights of the next tile (raw scores `sa`) are computed in
  // between, so their vector work runs in the shadow of the
  // matrix instructions; they are returned packed in `pk`.
  auto pv = [&](const char* pb, auto soft, const floatx16& sa, t2* pk, const v8* wb0,
                const v8* va01, v8* wb1_out, v8* va67_out) __attribute__((always_inline)) {
    constexpr bool kSoft = decltype(soft)::value;
    // weight of score i: 2^(s * sl2 - m_ref) with s = sa[i]; pairs
    // are packed to the matrix input type. The output is normalised by the
    // sum of the rounded weights the matrix product uses, the LSE comes from
    // the unrounded ones. The running maximum of the raw scores is checked
    // after the pass.
    float pf_even = 0.f;
    float mr = 0.f;
    if constexpr (kSoft) mr = ref();
    auto weight = [&](int i) __attribute__((always_inline)) {
      const float sc = sa[i];
      m_seen = fmaxf(m_seen, sc);
      const float pf = __builtin_amdgcn_exp2f(fmaf(sc, sl2, -mr));
      l_part += pf;
      if (i & 1) {
        pk[i >> 1] = t2{(T)pf_even, (T)pf};
        l_round = MT<T>::sum2(pk[i >> 1], l_round);
      } else {
        pf_even = pf;
      }
    };
    v8 wb[2][kWaves];
    v8 va[4];
#pragma unroll
    for (int g = 0; g < kWaves; ++g) wb[0][g] = wb0[g];
    va[0] = va01[0];
    va[1] = va01[1];
    // with soft, groups 6 and 7 are left to the caller (their operands are
    // returned): they fill the matrix unit across the step boundary
    constexpr int kGroups = kSoft ? 6 : 8;
#pragma unroll
    for (int n = 0; n < kGroups; ++n) {
      const int dt = n & 3, kk = n >> 2;
      if (n + 2 < 8) va[(n + 2) & 3] = vload(pb, (n + 2) & 3, (n + 2) >> 2);
      if (n == 1)
#pragma unroll
        for (int g = 0; g < kWaves; ++g) wb[1][g] = wload(g, 1);
#pragma unroll
      for (int g = 0; g < kWaves; ++g) {
        o[dt * 4 + g] = MT<T>::mfma(va[n & 3], wb[kk][g], o[dt * 4 + g]);
        // the 16 weights spread over instructions 4..23 (4 of every 5
        // slots): the first 4 cover the score product's result latency
        if constexpr (kSoft) {
          const int m = 4 * n + g - 4;
          if (m >= 0 && m % 5 != 4) weight(m - m / 5);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (!kSoft) __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kSoft) {
#pragma unroll
      for (int g = 0; g < kWaves; ++g) wb1_out[g] = wb[1][g];
      va67_out[0] = va[6 & 3];
      va67_out[1] = va[7 & 3];
    }
  };
  // one group (latent tile 2 or 3 of token half 1) of a value product whose
  // operands are already in registers
  auto pv_group = [&](int dt, const v8& va, const v8* wb1, int gfrom, int gto)
      __attribute__((always_inline)) {
#pragma unroll
    for (int g = gfrom; g < gto; ++g) o[dt * 4 + g] = MT<T>::mfma(va, wb1[g], o[dt * 4 + g]);
  };

  // One step of the tile pipeline: tile j's score product, then the value
  // product of tile j - 1 (if `has_prev`) with tile j's softmax in between,
  // then tile j's weights go to sh_p once every wave is done reading it.
  // group 7 of the previous step's value product, carried into this step
  // (zero operands when there is none: the instructions then add zero)
  v8 cw[kWaves], cv;
  auto zero_carry = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < kWaves; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) cw[g][i] = (T)0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) cv[i] = (T)0.f;
  };
  // take_ref: this is the chunk's first tile on the first pass (the
  // exponent reference is taken from it)
  auto step = [&](int j, int stage, bool has_prev, bool take_ref) __attribute__((always_inline)) {
    wait_vm(min(kAheadTiles - 1, seg_end - 1 - j));
    __syncthreads();
    // the loads of tile j + kAheadTiles go into the stage of tile j - 2,
    // which every wave finished reading before this barrier; they are
    // spread over the score product so the CU's address unit drains them
    // while the matrix unit works
    const bool do_issue = j + kAheadTiles < seg_end;
    __amdgpu_buffer_rsrc_t nrs = tile_rsrc(do_issue ? j + kAheadTiles : te, next_id);
    const unsigned nm0 =
        lds_base + ((stage + kAheadTiles) & (kStages - 1)) * kStageBytes + wave * kLoadsWave * 1024;
    if (do_issue) {
      next_id = __builtin_amdgcn_readfirstlane(pend_row);
      const int jn = j + kAheadTiles + 2;
      pend_row = jn < seg_end ? sh_ids[jn - id_base] : -1;
    }
    // issued on every step: past the segment the resource has no records,
    // so the loads touch no memory and only zero the stage of tile j - 2
    // (consumed); every step therefore adds the same count to vmcnt
    auto issue_part = [&](int i) __attribute__((always_inline)) {
      lds_load16(nrs, nm0 + i * 1024, ld_off[i], 0);
    };
    // the previous tile's stage, for the value product after the scores
    const char* pb = lds + ((stage + kStages - 1) & (kStages - 1)) * kStageBytes;
    v8 wb0[kWaves], va01[2];
    const char* sb = lds + stage * kStageBytes;

    // S^T = K . Q^T over 576 dims as one accumulation chain (a matrix
    // instruction whose accumulator is its predecessor's result issues back
    // to back). Key operands rotate through a kRing-entry ring, loaded kAhead
    // instructions ahead: a register is refilled only after the instruction
    // two slots back has issued, so an LDS return can never overwrite an
    // operand of a queued instruction (the compiler does not track these
    // assembly instructions' operands).
    constexpr int kAhead = 8, kRing = kAhead + 2;
    auto kaddr = [&](int k) __attribute__((always_inline)) {
      return (const v8*)(sb + qk_off[k & 3] + (k >> 2) * 128);
    };
    floatx16 sacc;
    v8 kb[kRing];
#pragma unroll
    for (int n = 0; n < kAhead; ++n) kb[n] = *kaddr(n);
    // the carried group runs while the first key operands are in flight
    pv_group(3, cv, cw, 0, kWaves);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int n = 0; n < kKSteps; ++n) {
      if (n == 0)
        MT<T>::qk_first(sacc, kb[0], q[0]);
      else
        MT<T>::qk_next(sacc, kb[n % kRing], q[n]);
      if (n + kAhead < kKSteps) kb[(n + kAhead) % kRing] = *kaddr(n + kAhead);
      if ((n & 3) == 2) issue_part(n >> 2);  // n = 2, 6, ..., 34: loads 0..8
      // first operands of the value product, in the last three slots
      // (harmless reads of stale data when there is no previous tile)
      if (n == kKSteps - 3)
#pragma unroll
        for (int g = 0; g < kWaves; ++g) wb0[g] = wload(g, 0);
      if (n == kKSteps - 2) va01[0] = vload(pb, 0, 0);
      if (n == kKSteps - 1) va01[1] = vload(pb, 1, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // The scores are read by vector instructions only after the result
    // latency of the last score product: behind qk_drain(), or, in the value
    // product, behind its first 4 matrix instructions (>= 128 cycles).
    // mask (a range's last tile, and the tiles the current-window mask
    // reaches back over; exp2(-inf) = 0)
    const int tok0 = tile_tok0(j);
    const int nvis = min(vend, min(en, (st_tile + j + 1) * kTile)) - tok0;
    if (nvis < kTile) {
      qk_drain(sacc);
      // row 8 (i >> 2) + 4 hi + (i & 3) is visible when below nvis: the
      // per-i part is a constant, so no row index stays live in the loop
      const int lim = nvis - 4 * hi;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 8 * (i >> 2) + (i & 3) < lim ? sacc[i] : -INFINITY;
    }
    __builtin_amdgcn_sched_barrier(0);

    t2 pk[8];
    v8 va67[2];
    if (has_prev) {
      pv(pb, std::integral_constant<bool, true>(), sacc, pk, wb0, va01, cw, va67);
    } else {
      // first tile of a segment: the weights alone (same arithmetic)
      qk_drain(sacc);
      if (MT<T>::kTileRef && take_ref) {
        // the chunk's first tile: the head's maximum over its 32 keys (16
        // in each lane of the pair that holds the head) becomes the
        // reference; a fully masked tile (the rest of the chunk is masked
        // too) keeps 0
        float mx = sacc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        if (hi == 0) sh_mref[head] = mx == -INFINITY ? 0.f : mx * sl2;
      }
      const float mr = ref();
      float pf_even = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float sc = sacc[i];
        m_seen = fmaxf(m_seen, sc);
        const float pf = __builtin_amdgcn_exp2f(fmaf(sc, sl2, -mr));
        l_part += pf;
        if (i & 1) {
          pk[i >> 1] = t2{(T)pf_even, (T)pf};
          l_round = MT<T>::sum2(pk[i >> 1], l_round);
        } else {
          pf_even = pf;
        }
      }
    }
    __syncthreads();  // every wave is done reading the previous weights
    // the new weights go out between the instructions of group 6
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      *(t4*)(sh_p + pst_off + (pchunk(j4, r32) << 4)) =
          __builtin_shufflevector(pk[2 * j4], pk[2 * j4 + 1], 0, 1, 2, 3);
      if (has_prev) pv_group(2, va67[0], cw, j4, j4 + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (has_prev)
      cv = va67[1];
    else
      zero_carry();
  };

  // Tiles run in segments of up to kIdCache: the row table is refilled and
  // the load pipeline restarted between segments (outside the tile loop).
  auto run_tiles = [&](bool first_pass) __attribute__((always_inline)) {
#pragma clang loop unroll(disable)
    for (int seg = tb; seg < te; seg += kIdCache) {
      id_base = seg;
      seg_end = min(te, seg + kIdCache);
      fill_rows(seg);
#pragma unroll
      for (int i = 0; i < kAheadTiles; ++i)
        if (seg + i < seg_end) issue(seg + i, i, tile_row(seg + i));
      next_id = tile_row(seg + kAheadTiles);
      pend_row = tile_row(seg + kAheadTiles + 1);
      zero_carry();
      step(seg, 0, false, first_pass && seg == tb);
#pragma clang loop unroll(disable)
      for (int j = seg + 1; j < seg_end; ++j) step(j, (j - seg) & (kStages - 1), true, false);
      // the last tile's value product
      __syncthreads();
      const char* pl = lds + ((seg_end - 1 - seg) & (kStages - 1)) * kStageBytes;
      v8 wb0[kWaves], va01[2];
#pragma unroll
      for (int g = 0; g < kWaves; ++g) wb0[g] = wload(g, 0);
      va01[0] = vload(pl, 0, 0);
      va01[1] = vload(pl, 1, 0);
      const floatx16 none = {};  // no softmax in this call: never read
      pv_group(3, cv, cw, 0, kWaves);
      pv(pl, std::integral_constant<bool, false>(), none, nullptr, wb0, va01, nullptr, nullptr);
    }
    // the last steps' loads (no records: they only zero consumed stages)
    // land before the workgroup moves on or ends
    wait_vm_all();
  };
  run_tiles(true);

  // replay the chunk with exact maxima if any head's maximum left its
  // window (fp16: above the first-tile reference by more than kWindow; the
  // maximum includes the first tile, so it never lies below it. bf16:
  // outside [-kWindow, kWindow])
  const float m_head = fmaxf(m_seen, __shfl_xor(m_seen, 32, 64)) * sl2;
  bool over;
  if constexpr (MT<T>::kTileRef)
    over = m_head > sh_mref[head] + MT<T>::kWindow;
  else
    over = m_head > MT<T>::kWindow || (m_head < -MT<T>::kWindow && m_head != -INFINITY);
  if (__builtin_amdgcn_ballot_w64(over) && lane == 0) atomicOr(&sh_redo, 1 << wave);
  __syncthreads();
  const int redo = __builtin_amdgcn_readfirstlane(sh_redo);
  if (redo) {
    const float exact = m_head == -INFINITY ? 0.f : m_head;
    if constexpr (MT<T>::kTileRef) {
      if (hi == 0) sh_mref[head] = exact;
    } else {
      m_ref = exact;
    }
    l_part = l_round = 0.f;
#pragma unroll
    for (int d = 0; d < kDTiles; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
    __syncthreads();
    run_tiles(false);
  }

  // ---- epilogue -------------------------------------------------------------
  const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
  const float l_rnd = l_round + __shfl_xor(l_round, 32, 64);
  float inv, lse;
  if (bad) {
    inv = NAN;
    lse = NAN;
  } else if (l_tot > 0.f) {
    inv = 1.f / l_rnd;
    lse = (ref() + log2f(l_tot)) * 0.6931471805599453f;
  } else {
    inv = 0.f;
    lse = -INFINITY;
  }
  // the normaliser of each head comes from the wave that ran its softmax
  if (hi == 0) sh_inv[head] = inv;
  // first row of this group's heads in the part output (or the workspace)
  const size_t row0 =
      (fd.slot < 0 ? ((size_t)p * Tq + t) * pp.H : ((size_t)fd.slot * S + s) * pp.H) + head0;
  if (hi == 0 && head_ok) {
    if (fd.slot < 0)
      store_any(pp.lse, row0 + head, pp.lse_dtype, lse);
    else
      pp.ws_lse[row0 + head] = lse;
  }
  __syncthreads();
  // The normalised rows go out through the (now idle) stage buffers, 64
  // heads at a time: each lane writes its values (head 32 g + r32, columns
  // 128 wave + 32 dt + 8 j + 4 hi + 0..3, held in o[4 dt + g][4 j + 0..3])
  // into a padded [64][512] block, then every store instruction writes 1 KB
  // of one head's contiguous 512-value row.
  auto store_out = [&](auto* dst) __attribute__((always_inline)) {
    typedef std::remove_pointer_t<decltype(dst)> TO;
    typedef TO v4 __attribute__((ext_vector_type(4)));
    constexpr int kSz = (int)sizeof(TO);
    constexpr int kPitch = kDc * kSz + 16;        // padded row: spreads the banks
    constexpr int kRowPieces = kDc * kSz / 16;    // 16-byte pieces per row
    static_assert(64 * kPitch <= kStages * kStageBytes, "output staging fits the stages");
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int g = 2 * half + gg;
        const float ig = sh_inv[g * kHeadsWave + r32];
        char* row = lds + (gg * kHeadsWave + r32) * kPitch;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              v[i] = from_f<TO>(bad ? NAN : o[4 * dt + g][4 * j + i] * ig);
            *(v4*)(row + (kDc / kWaves * wave + 32 * dt + 8 * j + 4 * hi) * kSz) = v;
          }
      }
      __syncthreads();
      char* out = (char*)(dst + (size_t)half * 64 * kDc);
      // rows of missing heads (beyond H) are not stored
      const int nrows = kOneGroup ? 64 : min(64, pp.H - head0 - half * 64);
#pragma unroll
      for (int i = 0; i < 64 * kRowPieces / 256; ++i) {
        const int idx = tid + i * 256, r = idx / kRowPieces, c = idx % kRowPieces;
        if (r < nrows)
          *(uint4*)(out + (size_t)r * kDc * kSz + c * 16) = *(const uint4*)(lds + r * kPitch + c * 16);
      }
      __syncthreads();
    }
  };
  // a chunk of a cut range goes to the workspace, in the output type
  void* dst = fd.slot >= 0 ? pp.ws_out : pp.out;
  if (pp.out_dtype == MLA_F32)
    store_out((float*)dst + row0 * kDc);
  else if (pp.out_dtype == MLA_BF16)
    store_out((bf16*)dst + row0 * kDc);
  else
    store_out((f16*)dst + row0 * kDc);
}

// ---------------------------------------------------------------------------
// merge of split chunks (fixed order), one wave per (unit, query, head) row
// ---------------------------------------------------------------------------

template <typename TO>
__device__ __forceinline__ void store8(TO* dst, const float* v) {
  typedef TO v8o __attribute__((ext_vector_type(8)));
  v8o x;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = from_f<TO>(v[i]);
  *(v8o*)dst = x;
}

// Lane i holds the LSE of chunk i0 + i; the chunks' partial rows (in the
// output type TO) are then accumulated in ascending order, 4 rows in flight.
// The first 64 LSEs and the first 4 rows are requested together, so a range
// of up to 4 pieces costs one round trip before its store.
template <typename TO>
__global__ __launch_bounds__(256) void split_merge_kernel(MfmaParams mp) {
  typedef TO v8o __attribute__((ext_vector_type(8)));
  const PartialParams& pp = mp.pp;
  const int lane = threadIdx.x & 63;
  // (a plan built on the host supplies the count and the descriptors: both
  // are checked, so a table that does not belong to the arguments stays in
  // bounds)
  const int U = pp.P * pp.B;
  const int n_units = min(max(*mp.ws_count, 0), U);
  const long long slots = plan_max_split_slots(U, pp.S, pp.num_splits);
  const long long rows = (long long)n_units * pp.S * pp.H;
  const int Tq = pp.B * pp.S;
  const long long waves = (long long)gridDim.x * 4;
  for (long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); r < rows; r += waves) {
    const int h = (int)(r % pp.H);
    const int s = (int)((r / pp.H) % pp.S);
    const int k = (int)(r / ((long long)pp.H * pp.S));
    const intx4 dsc = mp.ws_desc[k];
    const int u = dsc[0], slot0 = dsc[1], n = dsc[2];
    if (u < 0 || u >= U || slot0 < 0 || n < 1 || (long long)slot0 + n > slots) continue;
    auto wrow = [&](int i) { return ((size_t)(slot0 + i) * pp.S + s) * pp.H + h; };
    auto row_ptr = [&](int i) { return (const v8o*)((const TO*)pp.ws_out + wrow(i) * kDc) + lane; };
    const float l0 = lane < n ? pp.ws_lse[wrow(lane)] : -INFINITY;
    v8o raw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q < n) raw[q] = *row_ptr(q);
    bool nan_seen = isnan(l0);
    float m = l0;
    for (int i0 = 64; i0 < n; i0 += 64) {
      const float li = i0 + lane < n ? pp.ws_lse[wrow(i0 + lane)] : -INFINITY;
      nan_seen |= isnan(li);
      m = fmaxf(m, li);
    }
    m = wave_max(m);
    nan_seen = __builtin_amdgcn_ballot_w64(nan_seen) != 0;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float z = 0.f;
    if (m != -INFINITY && !nan_seen) {
      for (int i0 = 0; i0 < n; i0 += 64) {
        const int cnt = min(64, n - i0);
        const float li =
            i0 == 0 ? l0 : (lane < cnt ? pp.ws_lse[wrow(i0 + lane)] : -INFINITY);
        const float wl = li == -INFINITY ? 0.f : expf(li - m);
        z += wave_sum(wl);
        for (int i = 0; i < cnt; i += 4) {
          if (i0 + i > 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (i + q < cnt) raw[q] = *row_ptr(i0 + i + q);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float w = __shfl(wl, i + q, 64);
            if (i + q < cnt && w != 0.f)
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, (float)raw[q][e], acc[e]);
          }
        }
      }
    }
    const int p = u / pp.B, b = u % pp.B;
    const size_t orow = ((size_t)p * Tq + b * pp.S + s) * pp.H + h;
    float lse;
    if (nan_seen) {
      for (int i = 0; i < 8; ++i) acc[i] = NAN;
      lse = NAN;
    } else if (z > 0.f) {
      const float inv = 1.f / z;
      for (int i = 0; i < 8; ++i) acc[i] *= inv;
      lse = m + logf(z);
    } else {
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
      lse = -INFINITY;
    }
    store8<TO>((TO*)pp.out + orow * kDc + lane * 8, acc);
    if (lane == 0) store_any(pp.lse, orow, pp.lse_dtype, lse);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

bool mfma_path_supported(int dtype, int H, int block_size) {
  return (dtype == MLA_BF16 || dtype == MLA_F16) && H >= 1 &&
         (block_size == 0 || block_size % kTile == 0);
}

size_t mfma_max_chunks(int B, int S, int P, int hint) {
  return (size_t)plan_max_chunks((long long)P * B, S, hint);
}

size_t mfma_workspace_bytes(int B, int S, int H, int P, int hint, int out_dtype) {
  return ws_layout(B, S, H, P, hint, out_dtype).total;
}

long long pair_blocks(const PartialParams& cur) {
  return (short_tasks(cur, kPairHeads) + 3) / 4;
}

hipError_t launch_partial_mfma(const PartialParams& pp_in, int dtype, hipStream_t st,
                               const PartialParams* cur) {
  MfmaParams mp;
  memset(&mp, 0, sizeof(mp));
  mp.pp = pp_in;
  const WsLayout w = ws_layout(pp_in.B, pp_in.S, pp_in.H, pp_in.P, pp_in.num_splits, pp_in.out_dtype);
  char* ws = (char*)pp_in.ws_out;  // base of the workspace
  mp.ws_count = (int*)ws;
  mp.ws_desc = (intx4*)(ws + w.desc_off);
  mp.pp.ws_lse = (float*)(ws + w.lse_off);
  mp.pp.ws_out = ws + w.out_off;
  const long long U = (long long)pp_in.P * pp_in.B;
  if (pp_in.plan) {
    // the plan's cut-range count and descriptors (read-only to the merge)
    mp.ws_count = const_cast<int*>(pp_in.plan + 2);
    mp.ws_desc = (intx4*)const_cast<int*>(
        pp_in.plan + plan_desc_offset(U, pp_in.S, pp_in.num_splits));
  }
  const size_t chunks = pp_in.plan ? (size_t)pp_in.plan_chunks
                                   : mfma_max_chunks(pp_in.B, pp_in.S, pp_in.P, pp_in.num_splits);
  size_t groups = chunks * pp_in.S;
  if (pp_in.S > 1) groups = (groups + 8 * pp_in.S - 1) / (8 * pp_in.S) * (8 * pp_in.S);
  // blockIdx.y: the group of 128 heads; a current-chunk call rides behind
  // the history's chunks in x
  long long gx = (long long)groups;
  if (cur) {
    mp.cur = *cur;
    mp.cur_x0 = (int)groups;
    mp.cur_tasks = short_tasks(*cur, kPairHeads);
    gx += pair_blocks(*cur);
  }
  dim3 grid((unsigned)gx, (unsigned)((pp_in.H + kHeadsGroup - 1) / kHeadsGroup));
  const bool one = pp_in.H == kHeadsGroup;
  auto launch = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, mp); };
  if (dtype == MLA_BF16) {
    if (cur)
      one ? launch(partial_mfma_kernel<bf16, true, true>)
          : launch(partial_mfma_kernel<bf16, false, true>);
    else
      one ? launch(partial_mfma_kernel<bf16, true, false>)
          : launch(partial_mfma_kernel<bf16, false, false>);
  } else {
    if (cur)
      one ? launch(partial_mfma_kernel<f16, true, true>)
          : launch(partial_mfma_kernel<f16, false, true>);
    else
      one ? launch(partial_mfma_kernel<f16, true, false>)
          : launch(partial_mfma_kernel<f16, false, false>);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // no sub-splits requested (or none in the host's plan): every range is
  // written directly, nothing to merge
  if (pp_in.num_splits == 1 || (pp_in.plan && pp_in.plan_split_units == 0)) return hipSuccess;
  // one wave per merged row: at most min(U, groups) split units (a split
  // unit has more tiles than a chunk), capped; the kernel strides beyond
  const size_t split_units = pp_in.plan            ? (size_t)pp_in.plan_split_units
                             : pp_in.num_splits > 1 ? (size_t)U
                                                    : std::min((size_t)U, (size_t)kTargetGroups);
  const size_t merge_rows = split_units * pp_in.S * pp_in.H;
  const unsigned merge_blocks = (unsigned)std::max<size_t>(
      1, std::min<size_t>((merge_rows + 3) / 4, 2048));
  if (pp_in.out_dtype == MLA_F32)
    hipLaunchKernelGGL(split_merge_kernel<float>, dim3(merge_blocks), dim3(256), 0, st, mp);
  else if (pp_in.out_dtype == MLA_BF16)
    hipLaunchKernelGGL(split_merge_kernel<bf16>, dim3(merge_blocks), dim3(256), 0, st, mp);
  else
    hipLaunchKernelGGL(split_merge_kernel<f16>, dim3(merge_blocks), dim3(256), 0, st, mp);
  return hipGetLastError();
}

}  // namespace mla
