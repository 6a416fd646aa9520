// The split rule of mla_decode_partial: how every (part, sequence) key range
// is cut into 32-key tiles and chunks (sub-ranges run by one workgroup per
// query and merged by LSE inside the call). The kernel evaluates it on the
// device from the range arrays (block-wide sums), the library's plan query
// (mla_split_plan) on the host; both call these functions, so the rule is
// written once.
//
// The rule is the single-GPU counterpart of the K3 page's chunk-size
// decision (section 3.3): chunks of
//   c0 = max(4, ceil(T S / G)) tiles            (T = all tiles, G = 256)
// spread the work of S queries over about G workgroups; a range of nt tiles
// becomes max(1, ceil(nt / c)) near-equal chunks. When c0's chunks make
// between one and two rounds of G workgroups (the second round short, most
// compute units idle at the end), the smaller
//   c1 = max(4, ceil(2 S T / (4 G - S U)), ceil(S T / (2 G)))   (U ranges)
// that fills about two rounds (half a chunk of rounding per range) is taken
// if its chunks fit in two rounds. c1 >= S T / (2 G) bounds the chunk count
// by max(U + G / S, 2 G / S) + 1 and the cut chunks by 2 G / S + 1 (the grid
// and workspace bounds below).
#pragma once

#include <stdint.h>

namespace mla {

constexpr int kTile = 32;          // keys per tile (one LDS stage)
constexpr int kTargetGroups = 256; // workgroups one call aims to spread over
constexpr int kMinChunkTiles = 4;  // never cut a range into pieces below this

// tiles of 32 keys touched by the range [st, en) (tile boundaries are
// multiples of 32 logical positions)
__host__ __device__ inline int range_tiles(int st, int en) {
  return en > st ? (en - 1) / kTile - st / kTile + 1 : 0;
}

// chunks of a range of nt tiles: the explicit count `hint` (at most one per
// tile, at least one), else ceil(nt / c) (at least one)
__host__ __device__ inline int unit_chunks(int nt, int c, int hint) {
  if (hint > 0) return hint < (nt > 1 ? nt : 1) ? hint : (nt > 1 ? nt : 1);
  const int n = (nt + c - 1) / c;
  return n > 1 ? n : 1;
}

// the one-round chunk size c0
__host__ __device__ inline int chunk_tiles_one_round(long long total, int S) {
  const long long c = (total * S + kTargetGroups - 1) / kTargetGroups;
  return (int)(c > kMinChunkTiles ? c : kMinChunkTiles);
}

// the two-round chunk size c1, or 0 when S U >= 4 G (no such size)
__host__ __device__ inline int chunk_tiles_two_round(long long total, int S, long long U) {
  const long long su = (long long)S * U;
  if (4LL * kTargetGroups <= su) return 0;
  long long c1 = (2LL * S * total + 4LL * kTargetGroups - su - 1) / (4LL * kTargetGroups - su);
  const long long lo = (total * S + 2LL * kTargetGroups - 1) / (2LL * kTargetGroups);
  c1 = c1 > lo ? c1 : lo;
  return (int)(c1 > kMinChunkTiles ? c1 : kMinChunkTiles);
}

// c1 replaces c0 when it is smaller, c0's n0 chunks overflow one round and
// c1's n1 chunks fit in two
__host__ __device__ inline bool take_two_round(int c0, int c1, long long n0, long long n1, int S) {
  return c1 > 0 && c1 < c0 && (long long)S * n0 > kTargetGroups &&
         (long long)S * n1 <= 2LL * kTargetGroups;
}

// piece i of n of a range of nt tiles covers tiles [piece_tile(i), piece_tile(i + 1))
__host__ __device__ inline int piece_tile(int i, int nt, int n) {
  return (int)((long long)i * nt / n);
}

// a range is invalid (its results are NaN, nothing is read) when it starts
// below 0, ends before it starts or ends beyond the addressable positions
__host__ __device__ inline bool range_bad(int st, int en, long long capacity) {
  return st < 0 || en < st || (long long)en > capacity;
}

// bounds the launch sizes the grid and the workspace for
__host__ __device__ inline long long plan_max_chunks(long long U, int S, int hint) {
  if (hint > 0) return U * hint;
  const long long a = U + (kTargetGroups + S - 1) / S;
  const long long b = (2LL * kTargetGroups + S - 1) / S;
  return (a > b ? a : b) + 1;
}

__host__ __device__ inline long long plan_max_split_slots(long long U, int S, int hint) {
  if (hint == 1) return 0;
  if (hint > 1) return U * hint;
  return (2LL * kTargetGroups + S - 1) / S + 1;
}

// The automatic plan hands out chunk ids longest chunks first: chunks fall
// into kBuckets length buckets of the chunk size, bucket by bucket from the
// longest, in range order within a bucket, so the in-order dispatch of
// workgroups places long chunks early on ragged batches. A range of nt tiles
// in n chunks is in bucket len_bucket(ceil(nt / n), c).
constexpr int kBuckets = 8;

__host__ __device__ inline int len_bucket(int len, int c) {
  // len <= c + 1 < 2^27 tiles, so kBuckets len fits in 32 bits
  if (len >= c) return kBuckets - 1;
  const int b = (int)((unsigned)len * kBuckets / (unsigned)(c + 1));
  return b < kBuckets - 1 ? b : kBuckets - 1;
}

// A plan built on the host (mla_decode_partial_make_plan), int32 words:
//   header, kPlanHeader words: kPlanMagic, chunks, cut ranges, chunk tiles,
//     ranges U, queries S, num_splits, 0
//   at kPlanHeader: plan_max_chunks entries of kPlanEntry words, one per
//     chunk id: range, first tile, end tile, slot of its result (-1: the
//     part output), 0, 0, 0, 0
//   at plan_desc_offset: U descriptors of kPlanDesc words, one per cut range
//     in range order: range, first slot, pieces, 0
constexpr int kPlanMagic = 0x4D4C4131;
constexpr int kPlanHeader = 8;
constexpr int kPlanEntry = 8;
constexpr int kPlanDesc = 4;

__host__ __device__ inline long long plan_desc_offset(long long U, int S, int hint) {
  return kPlanHeader + kPlanEntry * plan_max_chunks(U, S, hint);
}

__host__ __device__ inline long long plan_table_words(long long U, int S, int hint) {
  return plan_desc_offset(U, S, hint) + kPlanDesc * U;
}

}  // namespace mla
