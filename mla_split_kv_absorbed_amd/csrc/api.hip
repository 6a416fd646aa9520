// C ABI of libmla_decode.so: argument validation, workspace sizing, dispatch.
// Every check happens on the host before any launch; on error nothing is
// enqueued.
#include <limits.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <vector>

#include "common.h"
#include "kernels.h"

#include <cmath>

using namespace mla;

namespace {

bool valid_dtype(int d) { return d == MLA_F32 || d == MLA_BF16 || d == MLA_F16; }

struct Extent {
  const void* p;
  size_t bytes;
};

bool overlap(Extent a, Extent b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool any_overlap(const Extent* outs, int no, const Extent* ins, int ni) {
  for (int i = 0; i < no; ++i) {
    for (int j = 0; j < ni; ++j)
      if (overlap(outs[i], ins[j])) return true;
    for (int j = i + 1; j < no; ++j)
      if (overlap(outs[i], outs[j])) return true;
  }
  return false;
}

// The row tensors (queries, cache, parts, weights, outputs, workspace) are
// read and written with 16-byte and LDS-direct accesses: their base pointers
// must be 16-byte aligned (NULL entries are skipped).
bool any_misaligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && ((uintptr_t)p & 15)) return true;
  return false;
}

// bf16 / fp16 over a contiguous cache of at most kShortKeys keys per
// sequence (the current-chunk call): the short-range kernel
bool use_short(const mla_partial_args* a) {
  return !(a->flags & MLA_FLAG_FORCE_SIMPLE) &&
         (a->q_dtype == MLA_BF16 || a->q_dtype == MLA_F16) && a->block_size == 0 &&
         a->kv_seq_stride <= kShortKeys;
}

bool use_mfma(const mla_partial_args* a) {
  return !(a->flags & MLA_FLAG_FORCE_SIMPLE) && !use_short(a) &&
         mfma_path_supported(a->q_dtype, a->H, a->block_size);
}

size_t partial_ws_bytes(const mla_partial_args* a) {
  if (!use_mfma(a)) return 0;
  return mfma_workspace_bytes(a->B, a->S, a->H, a->P, a->num_splits, a->out_dtype);
}

// Validation without the workspace check; returns MLA_OK or an error code.
int check_partial_args(const mla_partial_args* a) {
  if (!a) return MLA_ERR_NULL;
  if (!a->q_lat || !a->q_rope || !a->kv || !a->range_start || !a->range_end || !a->out ||
      !a->lse)
    return MLA_ERR_NULL;
  if (a->block_size > 0 && !a->block_table) return MLA_ERR_NULL;
  if (!valid_dtype(a->q_dtype) || !valid_dtype(a->kv_dtype) || !valid_dtype(a->out_dtype) ||
      !valid_dtype(a->lse_dtype))
    return MLA_ERR_DTYPE;
  if (a->q_dtype != a->kv_dtype) return MLA_ERR_DTYPE;
  if (a->B < 1 || a->S < 1 || a->H < 1 || a->P < 1) return MLA_ERR_SHAPE;
  if (a->S > 64 || a->H > 65535) return MLA_ERR_UNSUPPORTED;
  if ((long long)a->P * a->B * a->S > INT_MAX / 8) return MLA_ERR_SHAPE;
  if (a->block_size < 0) return MLA_ERR_SHAPE;
  if (a->block_size > 0) {
    if (a->max_blocks < 1 || a->num_blocks < 1) return MLA_ERR_SHAPE;
    if ((long long)a->max_blocks * a->block_size > INT_MAX) return MLA_ERR_SHAPE;
  } else {
    if (a->block_table) return MLA_ERR_SHAPE;
    if (a->kv_seq_stride < 1) return MLA_ERR_SHAPE;
  }
  if (a->mask != MLA_MASK_NONE && a->mask != MLA_MASK_CAUSAL_WINDOW) return MLA_ERR_RANGE;
  if (!isfinite(a->scale)) return MLA_ERR_RANGE;
  if (a->num_splits < 0 || a->num_splits > 4096) return MLA_ERR_RANGE;
  if (a->flags & ~MLA_FLAG_FORCE_SIMPLE) return MLA_ERR_RANGE;
  if (a->plan) {
    // a plan built on the host: only the matrix-core kernel takes one
    if (!use_mfma(a)) return MLA_ERR_UNSUPPORTED;
    const long long U = (long long)a->P * a->B;
    if (a->plan_chunks < 1 || a->plan_chunks > plan_max_chunks(U, a->S, a->num_splits) ||
        a->plan_split_units < 0 || a->plan_split_units > a->plan_chunks ||
        a->plan_split_units > U || ((uintptr_t)a->plan & 15))
      return MLA_ERR_RANGE;
  }
  return MLA_OK;
}

// the call's input and output extents (the workspace counted as an output)
void partial_extents(const mla_partial_args* a, size_t ws, Extent* ins, Extent* outs) {
  const size_t T = (size_t)a->B * a->S, H = a->H, P = a->P;
  const size_t e = elem_bytes(a->q_dtype);
  const size_t kv_rows = a->block_size > 0 ? (size_t)a->num_blocks * a->block_size
                                           : (size_t)a->B * a->kv_seq_stride;
  ins[0] = {a->q_lat, T * H * kDc * e};
  ins[1] = {a->q_rope, T * H * kDr * e};
  ins[2] = {a->kv, kv_rows * kRow * e};
  ins[3] = {a->block_table, a->block_table ? (size_t)a->B * a->max_blocks * 4 : 0};
  ins[4] = {a->range_start, P * a->B * 4};
  ins[5] = {a->range_end, P * a->B * 4};
  ins[6] = {a->plan,
            a->plan ? (size_t)plan_table_words((long long)P * a->B, a->S, a->num_splits) * 4 : 0};
  outs[0] = {a->out, P * T * H * kDc * elem_bytes(a->out_dtype)};
  outs[1] = {a->lse, P * T * H * elem_bytes(a->lse_dtype)};
  outs[2] = {a->workspace, ws};
}

int check_partial_alias(const mla_partial_args* a, size_t ws) {
  Extent ins[7], outs[3];
  partial_extents(a, ws, ins, outs);
  if (any_overlap(outs, 3, ins, 7)) return MLA_ERR_ALIAS;
  if (any_misaligned({a->q_lat, a->q_rope, a->kv, a->out, ws ? a->workspace : nullptr}))
    return MLA_ERR_RANGE;
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_abi_version(void) { return 2; }

const char* mla_status_string(int s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: a size is out of range or inconsistent";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: unknown or unsupported dtype combination";
    case MLA_ERR_RANGE: return "MLA_ERR_RANGE: an argument value is out of its documented range";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: valid but not implemented";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: a HIP runtime call or kernel launch failed";
    case MLA_ERR_ALIAS: return "MLA_ERR_ALIAS: an output overlaps an input";
    default: return "unknown status";
  }
}

size_t mla_decode_partial_workspace_size(const mla_partial_args* a) {
  if (check_partial_args(a) != MLA_OK) return (size_t)-1;
  return partial_ws_bytes(a);
}

int mla_decode_partial(const mla_partial_args* a, void* stream) {
  if (!a) return MLA_ERR_NULL;
  return mla::partial_call(a, a->workspace, a->workspace_bytes, stream);
}

}  // extern "C"

namespace mla {

size_t partial_workspace_need(const mla_partial_args* a) {
  if (check_partial_args(a) != MLA_OK) return (size_t)-1;
  return partial_ws_bytes(a);
}

// validation and launch of one partial call with the given workspace
// kernel parameters of a validated call
PartialParams partial_params(const mla_partial_args* a, void* workspace) {
  PartialParams pp;
  memset(&pp, 0, sizeof(pp));
  pp.q_lat = a->q_lat;
  pp.q_rope = a->q_rope;
  pp.kv = a->kv;
  pp.block_table = a->block_table;
  pp.range_start = a->range_start;
  pp.range_end = a->range_end;
  pp.out = a->out;
  pp.lse = a->lse;
  pp.B = a->B;
  pp.S = a->S;
  pp.H = a->H;
  pp.P = a->P;
  pp.block_size = a->block_size;
  pp.max_blocks = a->max_blocks;
  pp.num_blocks = a->num_blocks;
  pp.kv_seq_stride = a->kv_seq_stride;
  pp.mask = a->mask;
  pp.out_dtype = a->out_dtype;
  pp.lse_dtype = a->lse_dtype;
  pp.num_splits = a->num_splits;
  pp.plan = a->plan;
  pp.plan_chunks = a->plan_chunks;
  pp.plan_split_units = a->plan_split_units;
  pp.scale = a->scale;
  pp.capacity = a->block_size > 0 ? (long long)a->max_blocks * a->block_size
                                  : (long long)a->kv_seq_stride;
  if (use_mfma(a)) {
    pp.ws_out = workspace;  // workspace base; the launcher lays it out
    pp.max_chunks = (int)mfma_max_chunks(a->B, a->S, a->P, a->num_splits);
  }
  return pp;
}

// argument, workspace and alias checks of one call
int partial_check(const mla_partial_args* a, void* workspace, size_t workspace_bytes) {
  int st = check_partial_args(a);
  if (st != MLA_OK) return st;
  const size_t need = partial_ws_bytes(a);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MLA_ERR_WORKSPACE;
  mla_partial_args chk = *a;
  chk.workspace = workspace;
  return check_partial_alias(&chk, need > 0 ? workspace_bytes : 0);
}

int partial_call(const mla_partial_args* a, void* workspace, size_t workspace_bytes,
                 void* stream) {
  const int st = partial_check(a, workspace, workspace_bytes);
  if (st != MLA_OK) return st;
  const PartialParams pp = partial_params(a, workspace);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (use_short(a))
    e = launch_partial_short(pp, a->q_dtype, s);
  else if (use_mfma(a))
    e = launch_partial_mfma(pp, a->q_dtype, s);
  else
    e = launch_partial_simple(pp, a->q_dtype, s);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace mla

extern "C" {

int mla_decode_partial_pair(const mla_partial_args* hist, const mla_partial_args* cur,
                            void* stream) {
  if (!hist || !cur) return MLA_ERR_NULL;
  int st = check_partial_args(hist);
  if (st != MLA_OK) return st;
  st = check_partial_args(cur);
  if (st != MLA_OK) return st;
  if (!use_mfma(hist) || !use_short(cur)) return MLA_ERR_UNSUPPORTED;
  if (cur->q_dtype != hist->q_dtype) return MLA_ERR_DTYPE;
  st = mla::partial_check(hist, hist->workspace, hist->workspace_bytes);
  if (st != MLA_OK) return st;
  st = mla::partial_check(cur, cur->workspace, cur->workspace_bytes);
  if (st != MLA_OK) return st;
  // neither call may write what the other reads or writes (the workgroups of
  // both run at the same time)
  const size_t hws = partial_ws_bytes(hist) > 0 ? hist->workspace_bytes : 0;
  Extent ins[14], outs[6];
  partial_extents(hist, hws, ins, outs);
  partial_extents(cur, 0, ins + 7, outs + 3);
  if (any_overlap(outs, 6, ins, 14)) return MLA_ERR_ALIAS;
  const PartialParams hp = mla::partial_params(hist, hist->workspace);
  const PartialParams cp = mla::partial_params(cur, nullptr);
  // the combined grid's x extent: the history's bound plus the current call's
  // workgroups
  const long long hx = (long long)mla::mfma_max_chunks(hist->B, hist->S, hist->P,
                                                      hist->num_splits) * hist->S + 8LL * hist->S;
  if (hx + mla::pair_blocks(cp) > INT_MAX) return MLA_ERR_SHAPE;
  const hipError_t e = mla::launch_partial_mfma(hp, hist->q_dtype, (hipStream_t)stream, &cp);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_decode_partial_plan(const mla_partial_args* a, const int32_t* range_start,
                            const int32_t* range_end, mla_split_info* info) {
  int st = check_partial_args(a);
  if (st != MLA_OK) return st;
  if (!range_start || !range_end || !info) return MLA_ERR_NULL;
  const long long capacity = a->block_size > 0 ? (long long)a->max_blocks * a->block_size
                                               : (long long)a->kv_seq_stride;
  const long long U = (long long)a->P * a->B;
  memset(info, 0, sizeof(*info));
  info->matrix_path = use_mfma(a) ? 1 : use_short(a) ? 2 : 0;
  if (info->matrix_path != 1) {
    // the plain and the short-range kernels: one workgroup / wave per
    // (range, query, head), no chunks
    info->chunks = (int)U;
    return MLA_OK;
  }
  const int hint = a->num_splits;
  long long total = 0;
  int nt0 = -1;
  bool equal = true;
  for (long long u = 0; u < U; ++u) {
    const int s0 = range_start[u], e0 = range_end[u];
    const int nt = range_bad(s0, e0, capacity) ? 0 : range_tiles(s0, e0);
    if (range_bad(s0, e0, capacity) || nt == 0 || (nt0 >= 0 && nt != nt0)) equal = false;
    nt0 = nt;
    total += nt;
  }
  if (total > INT_MAX) return MLA_ERR_SHAPE;
  // the automatic plan's chunk size (used when num_splits is 0)
  int c_auto = chunk_tiles_one_round(total, a->S);
  {
    const int c1 = chunk_tiles_two_round(total, a->S, U);
    if (c1 > 0 && c1 < c_auto) {
      long long n0 = 0, n1 = 0;
      for (long long u = 0; u < U; ++u) {
        const int s0 = range_start[u], e0 = range_end[u];
        const int nt = range_bad(s0, e0, capacity) ? 0 : range_tiles(s0, e0);
        n0 += unit_chunks(nt, c_auto, 0);
        n1 += unit_chunks(nt, c1, 0);
      }
      if (take_two_round(c_auto, c1, n0, n1, a->S)) c_auto = c1;
    }
  }
  const int c = hint == 0 ? c_auto : 0;
  long long chunks = 0, split_units = 0, split_chunks = 0;
  for (long long u = 0; u < U; ++u) {
    const int s0 = range_start[u], e0 = range_end[u];
    const int nt = range_bad(s0, e0, capacity) ? 0 : range_tiles(s0, e0);
    const int n = unit_chunks(nt, c, hint);
    chunks += n;
    if (n > 1) {
      split_units += 1;
      split_chunks += n;
    }
  }
  // an explicit count cuts every range into exactly that many pieces (some
  // may be empty) and splits every range when it exceeds 1
  if (hint > 0) {
    chunks = U * hint;
    split_units = hint > 1 ? U : 0;
    split_chunks = hint > 1 ? U * hint : 0;
  }
  info->chunk_tiles = c;
  info->chunks = (int)chunks;
  info->split_ranges = (int)split_units;
  info->split_chunks = (int)split_chunks;
  info->equal_splits = equal && U > 0 ? unit_chunks(nt0, c_auto, 0) : 0;
  info->max_chunks = (int)plan_max_chunks(U, a->S, hint);
  info->max_split_slots = (int)plan_max_split_slots(U, a->S, hint);
  return MLA_OK;
}

size_t mla_decode_partial_plan_words(const mla_partial_args* a) {
  if (!a) return 0;
  mla_partial_args c = *a;
  c.plan = nullptr;  // the size of a plan does not depend on one being set
  if (check_partial_args(&c) != MLA_OK || !use_mfma(&c)) return 0;
  return (size_t)plan_table_words((long long)c.P * c.B, c.S, c.num_splits);
}

int mla_decode_partial_make_plan(const mla_partial_args* a, const int32_t* range_start,
                                 const int32_t* range_end, int32_t* plan, size_t plan_words,
                                 mla_split_info* info) {
  if (!a) return MLA_ERR_NULL;
  mla_partial_args c = *a;
  c.plan = nullptr;
  int st = check_partial_args(&c);
  if (st != MLA_OK) return st;
  if (!range_start || !range_end || !plan || !info) return MLA_ERR_NULL;
  if (!use_mfma(&c)) return MLA_ERR_UNSUPPORTED;
  const long long U = (long long)c.P * c.B;
  const int S = c.S, hint = c.num_splits;
  const long long words = plan_table_words(U, S, hint);
  if ((long long)plan_words < words) return MLA_ERR_WORKSPACE;
  st = mla_decode_partial_plan(&c, range_start, range_end, info);
  if (st != MLA_OK) return st;
  const long long capacity =
      c.block_size > 0 ? (long long)c.max_blocks * c.block_size : (long long)c.kv_seq_stride;
  std::vector<int> nt((size_t)U);
  for (long long u = 0; u < U; ++u) {
    const int s0 = range_start[u], e0 = range_end[u];
    nt[u] = range_bad(s0, e0, capacity) ? 0 : range_tiles(s0, e0);
  }
  memset(plan, 0, (size_t)words * 4);
  plan[0] = kPlanMagic;
  plan[1] = info->chunks;
  plan[2] = info->split_ranges;
  plan[3] = info->chunk_tiles;
  plan[4] = (int)U;
  plan[5] = S;
  plan[6] = hint;
  int32_t* ent = plan + kPlanHeader;
  int32_t* desc = plan + plan_desc_offset(U, S, hint);
  auto put = [&](long long id, long long u, int tb, int te, long long slot) {
    int32_t* e = ent + id * kPlanEntry;
    e[0] = (int)u;
    e[1] = tb;
    e[2] = te;
    e[3] = (int)slot;
  };
  if (hint > 0) {
    // the explicit count: chunk id -> (range, piece) as the device maps it,
    // the k pieces of a range on one XCD when the range count is a multiple of 8
    const int k = hint;
    for (long long id = 0; id < U * k; ++id) {
      long long u, i;
      if ((U & 7) == 0) {
        const long long pos = id >> 3;
        u = (id & 7) + 8 * (pos / k);
        i = pos % k;
      } else {
        u = id / k;
        i = id % k;
      }
      put(id, u, piece_tile((int)i, nt[u], k), piece_tile((int)i + 1, nt[u], k),
          k > 1 ? u * k + i : -1);
    }
    if (k > 1)
      for (long long u = 0; u < U; ++u) {
        desc[u * kPlanDesc + 0] = (int)u;
        desc[u * kPlanDesc + 1] = (int)(u * k);
        desc[u * kPlanDesc + 2] = k;
      }
    return MLA_OK;
  }
  // the automatic plan: chunk ids longest first by bucket, range order within a
  // bucket; slots and split indices in range order
  const int cs = info->chunk_tiles;
  std::vector<int> n((size_t)U), bucket((size_t)U);
  long long tot[kBuckets] = {0};
  for (long long u = 0; u < U; ++u) {
    n[u] = unit_chunks(nt[u], cs, 0);
    bucket[u] = len_bucket((nt[u] + n[u] - 1) / n[u], cs);
    tot[bucket[u]] += n[u];
  }
  long long run[kBuckets];
  for (int b = 0; b < kBuckets; ++b) {
    run[b] = 0;
    for (int b2 = b + 1; b2 < kBuckets; ++b2) run[b] += tot[b2];
  }
  long long soff = 0, poff = 0;
  for (long long u = 0; u < U; ++u) {
    const long long off = run[bucket[u]];
    run[bucket[u]] += n[u];
    for (int k = 0; k < n[u]; ++k)
      put(off + k, u, piece_tile(k, nt[u], n[u]), piece_tile(k + 1, nt[u], n[u]),
          n[u] > 1 ? soff + k : -1);
    if (n[u] > 1) {
      desc[poff * kPlanDesc + 0] = (int)u;
      desc[poff * kPlanDesc + 1] = (int)soff;
      desc[poff * kPlanDesc + 2] = n[u];
      soff += n[u];
      poff += 1;
    }
  }
  return MLA_OK;
}

int mla_cut_ranges(const int32_t* range_start, const int32_t* range_end, int n, int k,
                   int32_t* piece_start, int32_t* piece_end) {
  if (!range_start || !range_end || !piece_start || !piece_end) return MLA_ERR_NULL;
  if (n < 1 || k < 1 || (long long)n * k > INT_MAX) return MLA_ERR_SHAPE;
  for (int j = 0; j < n; ++j) {
    const int a0 = range_start[j], e0 = range_end[j];
    if (a0 < 0 || e0 < a0) return MLA_ERR_RANGE;
  }
  for (int j = 0; j < n; ++j) {
    const int a0 = range_start[j], e0 = range_end[j];
    const int nt = range_tiles(a0, e0), t0 = a0 / kTile;
    for (int i = 0; i < k; ++i) {
      int ps = a0, pe = a0;
      if (nt > 0) {
        const int lo = piece_tile(i, nt, k), hi = piece_tile(i + 1, nt, k);
        ps = lo == 0 ? a0 : (t0 + lo) * kTile;
        pe = hi > lo ? std::min(e0, (t0 + hi) * kTile) : ps;
      }
      piece_start[(size_t)i * n + j] = ps;
      piece_end[(size_t)i * n + j] = pe;
    }
  }
  return MLA_OK;
}

int mla_lse_combine(const void* parts_out, const void* parts_lse, int P, int part_dtype,
                    int lse_dtype, const void* local_out, const void* local_lse, int T, int H,
                    void* out, int out_dtype, float* lse_out, void* stream) {
  if (!out) return MLA_ERR_NULL;
  if ((local_out == nullptr) != (local_lse == nullptr)) return MLA_ERR_NULL;
  if (P > 0 && (!parts_out || !parts_lse)) return MLA_ERR_NULL;
  if (!valid_dtype(part_dtype) || !valid_dtype(lse_dtype) || !valid_dtype(out_dtype))
    return MLA_ERR_DTYPE;
  if (P < 0 || T < 1 || H < 1) return MLA_ERR_SHAPE;
  if (P + (local_out ? 1 : 0) < 1) return MLA_ERR_SHAPE;
  const size_t rows = (size_t)T * H;
  if ((rows + 3) / 4 > (size_t)INT_MAX) return MLA_ERR_SHAPE;
  const size_t pe = elem_bytes(part_dtype), le = elem_bytes(lse_dtype);
  Extent ins[4] = {{parts_out, (size_t)P * rows * kDc * pe},
                   {parts_lse, (size_t)P * rows * le},
                   {local_out, local_out ? rows * kDc * pe : 0},
                   {local_lse, local_lse ? rows * le : 0}};
  Extent outs[2] = {{out, rows * kDc * elem_bytes(out_dtype)},
                    {lse_out, lse_out ? rows * 4 : 0}};
  if (any_overlap(outs, 2, ins, 4)) return MLA_ERR_ALIAS;
  if (any_misaligned({parts_out, local_out, out})) return MLA_ERR_RANGE;
  CombineParams c;
  c.parts_out = parts_out;
  c.parts_lse = parts_lse;
  c.local_out = local_out;
  c.local_lse = local_lse;
  c.out = out;
  c.lse_out = lse_out;
  c.P = P;
  c.T = T;
  c.H = H;
  c.part_dtype = part_dtype;
  c.lse_dtype = lse_dtype;
  c.out_dtype = out_dtype;
  return launch_combine(c, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_combine_vup(const void* parts_out, const void* parts_lse, int P, int part_dtype,
                    int lse_dtype, const void* local_out, const void* local_lse, int T, int H,
                    const void* w_uv, int dtype, void* out, float* lse_out, void* lat_out,
                    void* stream) {
  if (!out || !w_uv) return MLA_ERR_NULL;
  if ((local_out == nullptr) != (local_lse == nullptr)) return MLA_ERR_NULL;
  if (P > 0 && (!parts_out || !parts_lse)) return MLA_ERR_NULL;
  if (!valid_dtype(part_dtype) || !valid_dtype(lse_dtype) || !valid_dtype(dtype))
    return MLA_ERR_DTYPE;
  if (P < 0 || T < 1 || H < 1 || H > 65535) return MLA_ERR_SHAPE;
  if (P + (local_out ? 1 : 0) < 1) return MLA_ERR_SHAPE;
  if (dtype == MLA_F32) return MLA_ERR_UNSUPPORTED;
  // token blocks: 32 tokens (two rows per wave) when there are at most 4
  // parts to hold in flight and more than 256 blocks of 16, else 16; each
  // workgroup takes as many consecutive blocks of one head (it loads W_UV[h]
  // once for all of them) as keep at least 256 workgroups, at most 4
  const int np = P + (local_out ? 1 : 0);
  const int tb = np <= 4 && (long long)H * ((T + 15) / 16) > 256 ? 32 : 16;
  const long long nb = (T + tb - 1) / tb;
  const int nbw = (int)std::max(1LL, std::min(4LL, (long long)H * nb / 256));
  if ((long long)H * ((nb + nbw - 1) / nbw) > (1LL << 30)) return MLA_ERR_SHAPE;
  const size_t rows = (size_t)T * H;
  const size_t pe = elem_bytes(part_dtype), le = elem_bytes(lse_dtype), e = elem_bytes(dtype);
  Extent ins[5] = {{parts_out, (size_t)P * rows * kDc * pe},
                   {parts_lse, (size_t)P * rows * le},
                   {local_out, local_out ? rows * kDc * pe : 0},
                   {local_lse, local_lse ? rows * le : 0},
                   {w_uv, (size_t)H * kDc * kDv * e}};
  Extent outs[3] = {{out, rows * kDv * e},
                    {lse_out, lse_out ? rows * 4 : 0},
                    {lat_out, lat_out ? rows * kDc * e : 0}};
  if (any_overlap(outs, 3, ins, 5)) return MLA_ERR_ALIAS;
  if (any_misaligned({parts_out, local_out, w_uv, out, lat_out})) return MLA_ERR_RANGE;
  CombineVupParams cv;
  cv.c.parts_out = parts_out;
  cv.c.parts_lse = parts_lse;
  cv.c.local_out = local_out;
  cv.c.local_lse = local_lse;
  cv.c.out = nullptr;
  cv.c.lse_out = lse_out;
  cv.c.P = P;
  cv.c.T = T;
  cv.c.H = H;
  cv.c.part_dtype = part_dtype;
  cv.c.lse_dtype = lse_dtype;
  cv.c.out_dtype = dtype;
  cv.w_uv = w_uv;
  cv.out = out;
  cv.lat_out = lat_out;
  cv.tb = tb;
  cv.nbw = nbw;
  return launch_combine_vup(cv, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_vup(const void* x, const void* w_uv, void* out, int T, int H, int dtype, void* stream) {
  if (!x || !w_uv || !out) return MLA_ERR_NULL;
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  if (T < 1 || H < 1 || H > 65535) return MLA_ERR_SHAPE;
  const size_t e = elem_bytes(dtype);
  Extent ins[2] = {{x, (size_t)T * H * kDc * e}, {w_uv, (size_t)H * kDc * kDv * e}};
  Extent outs[1] = {{out, (size_t)T * H * kDv * e}};
  if (any_overlap(outs, 1, ins, 2)) return MLA_ERR_ALIAS;
  if (any_misaligned({x, w_uv, out})) return MLA_ERR_RANGE;
  hipError_t he = dtype == MLA_F32
                    ? launch_vup_simple(x, w_uv, out, T, H, dtype, (hipStream_t)stream)
                    : launch_vup_mfma(x, w_uv, out, T, H, dtype, (hipStream_t)stream);
  return he == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_q_absorb(const void* q_nope, const void* w_uk, void* q_lat, int T, int H, int dtype,
                 void* stream) {
  if (!q_nope || !w_uk || !q_lat) return MLA_ERR_NULL;
  if (!valid_dtype(dtype)) return MLA_ERR_DTYPE;
  if (T < 1 || H < 1 || H > 65535) return MLA_ERR_SHAPE;
  const size_t e = elem_bytes(dtype);
  Extent ins[2] = {{q_nope, (size_t)T * H * kDn * e}, {w_uk, (size_t)H * kDc * kDn * e}};
  Extent outs[1] = {{q_lat, (size_t)T * H * kDc * e}};
  if (any_overlap(outs, 1, ins, 2)) return MLA_ERR_ALIAS;
  if (any_misaligned({q_nope, w_uk, q_lat})) return MLA_ERR_RANGE;
  hipError_t he = dtype == MLA_F32
                    ? launch_absorb_simple(q_nope, w_uk, q_lat, T, H, dtype, (hipStream_t)stream)
                    : launch_absorb_mfma(q_nope, w_uk, q_lat, T, H, dtype, (hipStream_t)stream);
  return he == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_decode_prologue(const mla_prologue_args* a, void* stream) {
  if (!a) return MLA_ERR_NULL;
  if (!a->q_nope || !a->q_pe || !a->w_uk || !a->kv_new || !a->positions || !a->kv ||
      !a->q_lat || !a->q_rope)
    return MLA_ERR_NULL;
  if (!valid_dtype(a->dtype)) return MLA_ERR_DTYPE;
  if (a->B < 1 || a->S < 1 || a->H < 1 || a->H > 65535) return MLA_ERR_SHAPE;
  if ((long long)a->B * a->S > (1 << 30)) return MLA_ERR_SHAPE;
  if (!(a->rope_theta > 0.f) || !std::isfinite(a->rope_theta)) return MLA_ERR_RANGE;
  size_t cache_rows;
  if (a->block_size > 0) {
    if (!a->block_table) return MLA_ERR_NULL;
    if (a->max_blocks < 1 || a->num_blocks < 1) return MLA_ERR_SHAPE;
    cache_rows = (size_t)a->num_blocks * a->block_size;
  } else {
    if (a->block_size < 0 || a->block_table) return MLA_ERR_SHAPE;
    if (a->kv_seq_stride < 1) return MLA_ERR_SHAPE;
    cache_rows = (size_t)a->B * a->kv_seq_stride;
  }
  const size_t T = (size_t)a->B * a->S, H = a->H, e = elem_bytes(a->dtype);
  Extent ins[7] = {{a->q_nope, T * H * kDn * e},
                   {a->q_pe, T * H * kDr * e},
                   {a->w_uk, H * kDc * kDn * e},
                   {a->kv_new, T * kRow * e},
                   {a->positions, T * 4},
                   {a->block_table, a->block_size > 0 ? (size_t)a->B * a->max_blocks * 4 : 0},
                   {a->kv, cache_rows * kRow * e}};
  Extent outs[3] = {{a->q_lat, T * H * kDc * e}, {a->q_rope, T * H * kDr * e},
                    {a->kv, cache_rows * kRow * e}};
  // the cache is written in place: check it against every input but itself
  if (any_overlap(outs, 2, ins, 7) || any_overlap(outs + 2, 1, ins, 6)) return MLA_ERR_ALIAS;
  if (any_misaligned({a->q_nope, a->q_pe, a->w_uk, a->kv_new, a->kv, a->q_lat, a->q_rope}))
    return MLA_ERR_RANGE;
  PrologueParams pp;
  pp.q_nope = a->q_nope;
  pp.q_pe = a->q_pe;
  pp.w_uk = a->w_uk;
  pp.kv_new = a->kv_new;
  pp.positions = a->positions;
  pp.B = a->B;
  pp.S = a->S;
  pp.H = a->H;
  pp.T = (int)T;
  pp.log2_theta = std::log2((double)a->rope_theta);
  pp.kv = a->kv;
  pp.block_table = a->block_size > 0 ? a->block_table : nullptr;
  pp.block_size = a->block_size;
  pp.max_blocks = a->max_blocks;
  pp.num_blocks = a->num_blocks;
  pp.kv_seq_stride = a->kv_seq_stride;
  pp.q_lat = a->q_lat;
  pp.q_rope = a->q_rope;
  hipStream_t st = (hipStream_t)stream;
  hipError_t he;
  if (a->dtype == MLA_F32) {
    he = launch_absorb_simple(a->q_nope, a->w_uk, a->q_lat, (int)T, a->H, a->dtype, st);
    if (he == hipSuccess) he = launch_rope_append(pp, a->dtype, st);
  } else {
    he = launch_prologue_mfma(pp, a->dtype, st);
  }
  return he == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
