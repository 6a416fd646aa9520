/*
 * mla_decode.h -- C ABI of the absorbed split-KV MLA decode library
 * (libmla_decode.so, HIP kernels for gfx950 / MI355X).
 *
 * One decode step of Multi-head Latent Attention over a latent KV cache:
 *
 *   q_lat = W_UK[h] . q_nope                      mla_q_absorb
 *   (o_p, lse_p) = attention over part p's keys   mla_decode_partial
 *   o = LSE merge of the parts (+ a local part)   mla_lse_combine
 *   out = o . W_UV[h]  -> [T][H*128]               mla_vup
 *
 * The operations follow the "DCP decode streams / V-up" study page (vLLM
 * Ascend PR notes): a decode step splits the keys into parts along the
 * sequence (decode context parallelism), each part returns a partial output
 * and its log-sum-exp (background section), the partials are merged by LSE
 * into the exact full-sequence softmax (combine step, "local_output /
 * local_lse" read without packing), and the batch-major latent result goes
 * through one transpose-free batched V-up (V-up fusion section). The latent
 * row layout (c_KV 512 + k_R 64 = 576 values per token, shared by every head)
 * and the paged block sizes follow the "MLA multi-GPU sharding" page
 * (latent-vector and --block-size sections).
 *
 * Fixed dimensions: d_c = 512, d_R = 64, d_nope = d_v = 128.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless stated otherwise. The caller owns
 *    every buffer; the library allocates nothing in these calls, keeps no
 *    pointer after return, and does not synchronise the host.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream). Calls contain no host sync, no event creation and no
 *    allocation, so they may be recorded into a HIP graph.
 *  - Host-side validation happens before any launch; on error nothing is
 *    enqueued and a negative MLA_ERR_* code is returned. A failed launch
 *    returns MLA_ERR_HIP. Device faults surface at the caller's next sync.
 *  - Outputs must not overlap inputs (checked where the extents are known:
 *    MLA_ERR_ALIAS).
 *  - The row tensors (queries, cache, partial outputs and parts, weights,
 *    outputs, workspace) are accessed 16 bytes at a time: their pointers
 *    must be 16-byte aligned (MLA_ERR_RANGE otherwise; checked after the
 *    overlap check). LSE and int32 arrays need only their element alignment.
 *  - Results are bitwise reproducible for identical inputs and arguments
 *    (fixed reduction orders, no floating-point atomics).
 *  - Accumulation is fp32; results are rounded to nearest-even into the
 *    output dtype.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_D_C 512
#define MLA_D_R 64
#define MLA_D_ROW 576
#define MLA_D_NOPE 128
#define MLA_D_V 128

/* element types */
typedef enum { MLA_F32 = 0, MLA_BF16 = 1, MLA_F16 = 2 } mla_dtype;

/* key visibility inside a part's range [start, end):
 *  NONE          every key of the range is visible (the history segment).
 *  CAUSAL_WINDOW bottom-right aligned window: query s (0 <= s < S) sees the
 *                range's keys at offsets j <= (end - start) - S + s. With a
 *                range holding the S current-chunk tokens this is the MTP
 *                current-window mask (study page: the CURRENT call with its
 *                attn_mask). */
typedef enum { MLA_MASK_NONE = 0, MLA_MASK_CAUSAL_WINDOW = 1 } mla_mask;

/* status codes */
enum {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer is NULL                       */
  MLA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent           */
  MLA_ERR_DTYPE = -3,       /* unknown dtype or unsupported dtype combination   */
  MLA_ERR_RANGE = -4,       /* an argument value is out of its documented range */
  MLA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required       */
  MLA_ERR_UNSUPPORTED = -6, /* valid but not implemented (e.g. S > 64)          */
  MLA_ERR_HIP = -7,         /* a HIP runtime call or kernel launch failed       */
  MLA_ERR_ALIAS = -8        /* an output overlaps an input                      */
};

/* flags for mla_partial_args.flags */
#define MLA_FLAG_FORCE_SIMPLE 1u /* use the plain VALU kernel (testing aid) */

/*
 * Arguments of mla_decode_partial.
 *
 * Queries: T = B*S query tokens, t = b*S + s.
 *   q_lat  [T][H][512]  absorbed query (q_dtype)
 *   q_rope [T][H][64]   rotary query (q_dtype, already rotated)
 * Cache (kv_dtype == q_dtype), one row = c_KV (512) || k_R (64):
 *   paged      (block_size > 0): kv [num_blocks][block_size][576];
 *              block_table int32 [B][max_blocks]: logical token j of
 *              sequence b sits in row block_table[b][j / block_size],
 *              slot j % block_size.
 *   contiguous (block_size == 0, block_table == NULL, the study page's
 *              current-chunk convention): kv [B][kv_seq_stride][576].
 * Parts: P >= 1 parts; range_start/range_end int32 [P][B] (DEVICE arrays)
 *   give part p's logical key range [start, end) of sequence b. An empty
 *   range yields out = 0 and lse = -inf. A range outside
 *   [0, capacity] (capacity = max_blocks*block_size or kv_seq_stride) or a
 *   referenced block id outside [0, num_blocks) is detected on the device:
 *   that (part, sequence)'s out and lse are filled with NaN and nothing is
 *   read out of bounds.
 * Score: s_j = scale * (q_lat . c_j + q_rope . kR_j). lse is the natural
 *   log-sum-exp of the scaled scores of the visible keys.
 * Outputs:
 *   out [P][T][H][512] (out_dtype): sum_j softmax_j * c_j over the part
 *   lse [P][T][H]      (lse_dtype)
 * Workspace: `workspace_bytes` >= mla_decode_partial_workspace_size(args)
 *   bytes of device memory (may be 0 bytes / NULL when the size is 0). It is
 *   exclusive to the call until the stream has passed it; two calls that
 *   share a workspace must be ordered on one stream (or by events). It holds
 *   the results of sub-ranges (in out_dtype, with fp32 LSEs) until they are
 *   merged inside the call.
 * num_splits: 0 = automatic; otherwise each (part, sequence) range is cut
 *   into at most this many sub-ranges that are merged inside the call (the
 *   sub-ranges of one range run on one XCD when the range count P x B is a
 *   multiple of 8). With
 *   1 every range is one unit of work, dispatched in range order (best when
 *   the ranges have equal lengths and there are at least a few hundred of
 *   them; the automatic plan dispatches the longest first).
 * plan: NULL, or a DEVICE copy of the plan mla_decode_partial_make_plan built
 *   for these arguments and ranges (int32, 16-byte aligned, read only). The
 *   kernel then skips its own evaluation of the split rule (each workgroup
 *   reads its chunk), the launch has exactly the plan's chunks, and the
 *   sub-range merge is not launched when no range is cut. plan_chunks /
 *   plan_split_units: the plan's `chunks` / `split_ranges` (its
 *   mla_split_info), outside [1, max_chunks] / [0, min(P B, plan_chunks)]
 *   MLA_ERR_RANGE. A plan made for other arguments or ranges gives wrong
 *   results but never an access out of bounds (every entry is checked on the
 *   device against the range arrays and the workspace). The plain and the
 *   short-range kernels take none (MLA_ERR_UNSUPPORTED).
 */
typedef struct mla_partial_args {
  const void* q_lat;
  const void* q_rope;
  int q_dtype;
  int B, S, H;
  const void* kv;
  int kv_dtype;
  int block_size;
  const int32_t* block_table;
  int max_blocks;
  int num_blocks;
  int kv_seq_stride;
  int P;
  const int32_t* range_start;
  const int32_t* range_end;
  int mask;
  float scale;
  void* out;
  int out_dtype;
  void* lse;
  int lse_dtype;
  void* workspace;
  size_t workspace_bytes;
  int num_splits;
  unsigned flags;
  const int32_t* plan;
  int plan_chunks;
  int plan_split_units;
} mla_partial_args;

/* How mla_decode_partial divides its work (the split rule it evaluates on
 * the device from the range arrays), reported by mla_decode_partial_plan. */
typedef struct mla_split_info {
  int matrix_path;     /* 1: the matrix-core kernel (bf16 / fp16); 2: the
                          short-range kernel (bf16 / fp16 over a contiguous
                          cache with kv_seq_stride <= 8), one wave per (range,
                          query) and 4 heads; 0: the plain kernel (fp32, or
                          MLA_FLAG_FORCE_SIMPLE), one workgroup per (range,
                          query, head). Paths 0 and 2 cut nothing, need no
                          workspace and take no plan. */
  int chunk_tiles;     /* tiles of 32 keys per chunk of the automatic plan
                          (num_splits == 0); 0 with an explicit num_splits */
  int chunks;          /* chunks: each runs as one workgroup per query token
                          and group of 128 heads */
  int split_ranges;    /* ranges cut into more than one chunk (merged by LSE
                          inside the call) */
  int split_chunks;    /* chunks of those ranges (workspace slots in use) */
  int equal_splits;    /* when every range is valid and has the same nonzero
                          tile count: the chunk count per range the automatic
                          plan gives (1 = no range is cut); passing it as
                          num_splits yields the same pieces without the
                          in-kernel plan. 0 otherwise. */
  int max_chunks;      /* the launch's bound on `chunks` (grid size) */
  int max_split_slots; /* the workspace's bound on `split_chunks` */
} mla_split_info;

/* The split plan of mla_decode_partial for `a` with the given ranges
 * (K3 page, section 3.3: the chunk size chosen from the work and the
 * compute units available). range_start / range_end are HOST copies of
 * a->range_start / a->range_end ([P][B] int32); the argument struct is
 * validated as by mla_decode_partial (its device pointers are not read).
 * The rule, evaluated identically here and in the kernel: chunks of
 * c0 = max(4, ceil(T S / 256)) tiles (T = all tiles of the valid ranges);
 * when those make between one and two rounds of 256 workgroups, the smaller
 * c1 = max(4, ceil(2 S T / (1024 - S U)), ceil(S T / 512)) (U = P B ranges)
 * if its chunks fit in two rounds; a range of nt tiles becomes
 * max(1, ceil(nt / c)) near-equal chunks, chunk i covering tiles
 * [i nt / n, (i + 1) nt / n). With num_splits = k > 0 every range is cut
 * into exactly k such pieces. Returns MLA_OK and fills `info`, or an error
 * code (nothing is launched either way). */
int mla_decode_partial_plan(const mla_partial_args* a, const int32_t* range_start,
                            const int32_t* range_end, mla_split_info* info);

/* int32 words of a plan for these arguments (a pure function of P, B, S and
 * num_splits; `a->plan` is ignored); 0 for invalid arguments or the plain
 * and short-range kernels. */
size_t mla_decode_partial_plan_words(const mla_partial_args* a);

/* Builds on the host the plan mla_decode_partial would evaluate on the
 * device (the split rule of mla_decode_partial_plan, with the kernel's chunk
 * order: the pieces of a range in order, the automatic plan's chunks longest
 * first), so that a serving loop that holds its sequence lengths on the host
 * can hand it over instead (the `plan` argument). range_start / range_end:
 * HOST copies of the ranges; plan: HOST buffer of plan_words >=
 * mla_decode_partial_plan_words(a) int32 (MLA_ERR_WORKSPACE otherwise),
 * filled with the table (the caller copies it to device memory); info: as
 * mla_decode_partial_plan. `a->plan` is ignored. */
int mla_decode_partial_make_plan(const mla_partial_args* a, const int32_t* range_start,
                                 const int32_t* range_end, int32_t* plan, size_t plan_words,
                                 mla_split_info* info);

/* The pieces mla_decode_partial cuts a range into with num_splits = k:
 * piece i of range [s, e) covers its tiles [i nt / k, (i + 1) nt / k) (nt =
 * tiles of 32 logical positions the range touches, tile boundaries at
 * multiples of 32), clipped to [s, e); a piece with no tile is empty
 * (start = end). HOST arrays: range_start / range_end [n] in, piece_start /
 * piece_end [k][n] out. Passing the pieces as k parts with num_splits = 1
 * and merging them by LSE gives the call's own sub-range merge. Returns
 * MLA_ERR_RANGE for a range with start < 0 or end < start. */
int mla_cut_ranges(const int32_t* range_start, const int32_t* range_end, int n, int k,
                   int32_t* piece_start, int32_t* piece_end);

/* Bytes of device workspace mla_decode_partial needs for these arguments
 * (a pure function of the sizes, dtypes and flags; no device access).
 * Returns (size_t)-1 for invalid arguments. */
size_t mla_decode_partial_workspace_size(const mla_partial_args* a);

/* Split-KV partial attention: for every part p, query token t and head h,
 * the softmax-weighted latent sum and LSE over p's visible keys (study page:
 * the HISTORY and CURRENT attention calls, each returning output + LSE).
 * bf16 / fp16 run on the matrix-core kernel for any H, in groups of 128
 * heads that each read the part's keys once (a group with fewer real heads
 * computes the missing rows from zero queries and never stores them), except
 * over a contiguous cache with kv_seq_stride <= 8 (no valid range then holds
 * more than 8 keys: the study page's CURRENT call over the q_len tokens of
 * the chunk), which runs on a vector kernel of one wave per (part, query)
 * and 4 heads with an exact fp32 softmax; fp32 (and MLA_FLAG_FORCE_SIMPLE)
 * runs on the plain kernel, one workgroup per (part, query, head), and so
 * does a paged cache whose block_size is not a multiple of 32 (the matrix
 * kernel's 32-key tiles must not straddle blocks); mla_decode_partial_plan
 * reports the kernel a call takes (matrix_path). S <= 64
 * (MLA_ERR_UNSUPPORTED above).
 * Softmax range (K3 page, section 4.2: the online-softmax rescale is
 * mandatory): the matrix kernel exponentiates relative to a per-chunk
 * reference (bf16: 0, head maxima within +-64 in log2 units; fp16: each
 * head's maximum over the chunk's first 32 keys, later keys at most 15
 * log2 units above it, so fp16 weights stay below 2^15) and computes a
 * chunk again with each head's exact maximum when its scores leave that
 * window. Any finite scores give finite results. */
int mla_decode_partial(const mla_partial_args* a, void* stream);

/* The HISTORY and CURRENT partial calls of one decode step in one launch
 * (study page, design section: the current chunk's attention runs while the
 * history's does; here both share one grid instead of two streams). `hist`
 * must take the matrix-core kernel (bf16 / fp16) and `cur` the short-range
 * kernel (same dtype, contiguous cache with kv_seq_stride <= 8), else
 * MLA_ERR_UNSUPPORTED; each is validated as by mla_decode_partial (hist
 * with its own workspace and optional plan). The current call's workgroups
 * come after the history's chunks in dispatch order, so they run on the
 * compute units the history's schedule frees at its end. Neither call's
 * outputs (or hist's workspace) may overlap anything the other reads or
 * writes (MLA_ERR_ALIAS); reading the same queries is allowed. A pair whose
 * combined grid would pass 2^31 - 1 workgroups is MLA_ERR_SHAPE (the two
 * calls can then be made separately). Outputs are bitwise those of the two
 * separate calls. */
int mla_decode_partial_pair(const mla_partial_args* hist, const mla_partial_args* cur,
                            void* stream);

/* mla_decode_partial without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). It runs the same kernels with
 * the library's own device scratch as the workspace: a fixed array of
 * mla_noalloc_scratch_bytes() (96 MiB) that every GPU the library runs on
 * holds until the process ends (enough for every call with H <= 128 and
 * 16-bit outputs under the automatic plan). a->workspace and
 * a->workspace_bytes are ignored. The call allocates nothing; on a
 * device's first call it looks up that device's scratch address (the
 * stream's device must be current). Returns MLA_ERR_WORKSPACE when the
 * call needs more than the scratch holds, otherwise as mla_decode_partial.
 * Every call on one GPU shares that GPU's scratch: calls that overlap on
 * one GPU (other streams or host threads) race and must be ordered by the
 * caller. */
int mla_decode_partial_noalloc(const mla_partial_args* a, void* stream);

/* Bytes of the device scratch mla_decode_partial_noalloc uses. */
size_t mla_noalloc_scratch_bytes(void);

/* q absorption: q_lat[t][h][c] = sum_j W_UK[h][c][j] * q_nope[t][h][j].
 *   q_nope [T][H][128], w_uk [H][512][128], q_lat [T][H][512], all `dtype`.
 * (Not written out on the pages; it is the regrouping that lets the latent
 * cache serve as every head's key, see the K3 page section 2.1.) */
int mla_q_absorb(const void* q_nope, const void* w_uk, void* q_lat, int T, int H,
                 int dtype, void* stream);

/* LSE combine (study page: the combine that reads the received history
 * shards plus the local current part directly, without packing):
 *   m = max_i lse_i, w_i = exp(lse_i - m),
 *   out = sum_i w_i o_i / sum_i w_i, lse_out = m + ln sum_i w_i,
 * parts in index order, the local part last. Parts with lse = -inf weigh 0;
 * if all are empty, out = 0 and lse_out = -inf.
 *   parts_out [P][T][H][512] (part_dtype), parts_lse [P][T][H] (lse_dtype),
 *   local_out [T][H][512] / local_lse [T][H]: both NULL or both set (same
 *   dtypes as the parts); P may be 0 when a local part is given.
 *   out [T][H][512] (out_dtype); lse_out fp32 [T][H] or NULL. */
int mla_lse_combine(const void* parts_out, const void* parts_lse, int P, int part_dtype,
                    int lse_dtype, const void* local_out, const void* local_lse, int T, int H,
                    void* out, int out_dtype, float* lse_out, void* stream);

/* LSE combine fused with V-up: the result of mla_lse_combine followed by
 * mla_vup in one launch, the merged latent kept on chip (study page: the
 * combine step feeds the batch-major latent straight into the fused V-up).
 *   parts_out / parts_lse / P / part_dtype / lse_dtype / local_out /
 *   local_lse / T / H: as in mla_lse_combine.
 *   dtype: MLA_BF16 or MLA_F16 (MLA_ERR_UNSUPPORTED for MLA_F32: call the
 *   two entry points). The merged latent is rounded to `dtype` before the
 *   product, exactly as mla_lse_combine would store it for mla_vup.
 *   w_uv [H][512][128] (dtype); out [T][H][128] (dtype) == [T][H*128];
 *   lse_out fp32 [T][H] or NULL; lat_out [T][H][512] (dtype) or NULL: the
 *   merged latent as mla_lse_combine writes it.
 * Outputs must not overlap the inputs or each other (MLA_ERR_ALIAS).
 * MLA_ERR_SHAPE: T < 1, H outside [1, 65535], or T * H so large that the
 * launch would need more than 2^30 workgroups. */
int mla_combine_vup(const void* parts_out, const void* parts_lse, int P, int part_dtype,
                    int lse_dtype, const void* local_out, const void* local_lse, int T, int H,
                    const void* w_uv, int dtype, void* out, float* lse_out, void* lat_out,
                    void* stream);

/* V-up on the batch-major latent, transpose-free (study page, V-up fusion):
 *   out[t][h][v] = sum_c x[t][h][c] * W_UV[h][c][v]
 *   x [T][H][512], w_uv [H][512][128], out [T][H][128] == [T][H*128]. */
int mla_vup(const void* x, const void* w_uv, void* out, int T, int H, int dtype, void* stream);

/*
 * Arguments of mla_decode_prologue: the step before the attention path for
 * T = B*S new tokens (t = b*S + s, the s-th new token of sequence b).
 *   q_nope [T][H][128], q_pe [T][H][64] (before rotation),
 *   w_uk [H][512][128], kv_new [T][576] (the new tokens' c_KV, then their
 *   k_R before rotation), all `dtype`.
 *   positions int32 [T] (DEVICE): the logical position of each new token in
 *   its sequence, used as the rotation angle and as its cache slot. The S
 *   positions of one sequence must differ (two new tokens in one slot: which
 *   token's row the slot ends up holding is unspecified).
 *   rope_theta > 0: rotary base.
 *   Cache: the same layout as mla_partial_args (paged: kv, block_table
 *   [B][max_blocks], block_size > 0, num_blocks; contiguous: block_table
 *   NULL, block_size 0, kv_seq_stride rows per sequence).
 * Outputs: q_lat [T][H][512], q_rope [T][H][64] (rotated), and the cache
 *   row of every new token. A token whose position is negative or whose
 *   slot lies outside the block table, the cache or the contiguous stride is
 *   not written (detected on the device; nothing is written out of bounds).
 *   Only the new tokens' rows are written; kv_new must not overlap the cache.
 */
typedef struct mla_prologue_args {
  const void* q_nope;
  const void* q_pe;
  const void* w_uk;
  const void* kv_new;
  const int32_t* positions;
  int dtype;
  int B, S, H;
  float rope_theta;
  void* kv;
  const int32_t* block_table;
  int block_size, max_blocks, num_blocks;
  int kv_seq_stride;
  void* q_lat;
  void* q_rope;
} mla_prologue_args;

/* Fused decode prologue ("RTPLLM on K3" page: section 2.1, the input
 * projection yields the query's latent and rope parts and the compressed
 * latent the cache stores; section 4.1, the RoPE transform fused into one
 * kernel with the latent handling):
 *   q_lat[t][h]  = W_UK[h] . q_nope[t][h]                (as mla_q_absorb)
 *   q_rope[t][h] = rope(q_pe[t][h], positions[t])
 *   cache row of token t at position pos = positions[t] of sequence b:
 *     [kv_new[t][0:512] || rope(kv_new[t][512:576], pos)]
 * rope rotates each consecutive pair (x[2i], x[2i+1]) of the 64 rope values
 * by the angle pos * rope_theta^(-2i/64) (x[2i] cos - x[2i+1] sin,
 * x[2i] sin + x[2i+1] cos); the angle is formed in double precision.
 * bf16 / fp16 run as one kernel (matrix-core absorption with the rotation
 * and append in the same launch); fp32 as two. */
int mla_decode_prologue(const mla_prologue_args* a, void* stream);

/* Human-readable text for a status code (static string, never NULL). */
const char* mla_status_string(int status);

/* Library ABI version (this header: 2). */
int mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
