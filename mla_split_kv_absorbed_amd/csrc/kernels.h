// Launchers of the library's kernels (internal; the public ABI is mla_decode.h).
#pragma once

#include "common.h"

namespace mla {

// arguments of the decode prologue (mla_prologue_args, validated)
struct PrologueParams {
  const void* q_nope;
  const void* q_pe;
  const void* w_uk;
  const void* kv_new;
  const int32_t* positions;
  int B, S, H, T;
  double log2_theta;
  void* kv;
  const int32_t* block_table;
  int block_size, max_blocks, num_blocks, kv_seq_stride;
  void* q_lat;
  void* q_rope;
};

struct CombineParams {
  const void* parts_out;
  const void* parts_lse;
  const void* local_out;
  const void* local_lse;
  void* out;
  float* lse_out;
  int P, T, H;
  int part_dtype, lse_dtype, out_dtype;
};

// mla_decode_partial with an explicit workspace (validation, then launch);
// returns an MLA status code
int partial_call(const mla_partial_args* a, void* workspace, size_t workspace_bytes,
                 void* stream);
// workspace bytes a partial call needs, (size_t)-1 for invalid arguments
size_t partial_workspace_need(const mla_partial_args* a);

hipError_t launch_partial_simple(const PartialParams& pp, int dtype, hipStream_t st);
// Short ranges: a contiguous cache (block_size 0) with kv_seq_stride <=
// kShortKeys bounds every valid range by kShortKeys keys; bf16 / fp16 calls
// of that shape run on a vector kernel of one wave per (part, query, head)
// row instead of the matrix kernel.
constexpr int kShortKeys = 8;
hipError_t launch_partial_short(const PartialParams& pp, int dtype, hipStream_t st);
// MFMA path: q/kv dtype bf16 or f16, H % 128 == 0, block_size % 32 == 0 (or contiguous).
bool mfma_path_supported(int dtype, int H, int block_size);
// cur: a call of the short-range shape (bf16 / fp16 like pp, contiguous,
// kv_seq_stride <= kShortKeys) run in the same grid behind the history's
// chunks, or NULL
hipError_t launch_partial_mfma(const PartialParams& pp, int dtype, hipStream_t st,
                               const PartialParams* cur = nullptr);
// workgroups a short-range call adds to a combined launch
long long pair_blocks(const PartialParams& cur);
// Upper bound on split sub-ranges ("slots") an MFMA-path call may write.
size_t mfma_max_chunks(int B, int S, int P, int num_splits);
size_t mfma_workspace_bytes(int B, int S, int H, int P, int num_splits, int out_dtype);

hipError_t launch_combine(const CombineParams& c, hipStream_t st);

// combine fused with V-up: c.out_dtype is the compute type (bf16 / f16) of
// w_uv, out and lat_out; token blocks of tb = 16 or 32 tokens, nbw (1 .. 4)
// consecutive blocks of one head per workgroup; H * ceil(ceil(T / tb) / nbw)
// workgroups must fit in an int
struct CombineVupParams {
  CombineParams c;
  const void* w_uv;
  void* out;      // [T][H][128]
  void* lat_out;  // [T][H][512] or NULL
  int tb;
  int nbw;
};
hipError_t launch_combine_vup(const CombineVupParams& cv, hipStream_t st);
hipError_t launch_vup_simple(const void* x, const void* w, void* out, int T, int H, int dt,
                             hipStream_t st);
hipError_t launch_vup_mfma(const void* x, const void* w, void* out, int T, int H, int dt,
                           hipStream_t st);
hipError_t launch_absorb_mfma(const void* qn, const void* w, void* ql, int T, int H, int dt,
                              hipStream_t st);
// fused absorption + rotation + cache append (bf16 / f16)
hipError_t launch_prologue_mfma(const PrologueParams& pp, int dt, hipStream_t st);
// rotation + cache append alone (any dtype; absorption launched separately)
hipError_t launch_rope_append(const PrologueParams& pp, int dt, hipStream_t st);
hipError_t launch_absorb_simple(const void* qn, const void* w, void* ql, int T, int H, int dt,
                                hipStream_t st);

}  // namespace mla
