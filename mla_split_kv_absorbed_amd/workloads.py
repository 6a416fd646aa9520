"""Seeded synthetic inputs for absorbed split-KV MLA decode.

This module is shared by the HIP path's tests/benchmark and by the oracle's
tests. It holds no attention arithmetic: it only draws random numbers, rounds
them once to a storage dtype, and lays them out (paged latent cache, block
table, per-part key ranges).

Shapes follow the pages' DeepSeek-style MLA: every cached token is one latent
row of d_c = 512 values (c_KV) followed by d_R = 64 rotary key values (k_R),
576 values in all, shared by every query head ("MLA multi-GPU sharding" page,
section on the latent vector c_t^KV and the decoupled k_t^R). The cache is
paged with 32- or 64-token blocks (same page, block-size section).

Recipe (per workload, numpy PCG64 seeded with 1000 + workload id unless a seed
is given): draw order lengths -> W_UK -> W_UV -> q_nope -> q_rope -> c_KV
(sequence-major, logical token order) -> k_R -> current-chunk c_KV / k_R ->
block permutation. Values are drawn in float64 and rounded once,
round-to-nearest-even, to the storage dtype. W ~ N(0, 1/512) (variance),
q, c_KV, k_R ~ N(0, 1).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

D_C = 512      # latent width (kv_lora_rank)
D_R = 64       # decoupled rotary key width
D_ROW = D_C + D_R
D_NOPE = 128   # per-head non-rotary query/key width
D_V = 128      # per-head value width

DTYPES = ("f32", "bf16", "f16")
ESIZE = {"f32": 4, "bf16": 2, "f16": 2}


# ----------------------------------------------------------------------------
# rounding to storage dtypes (input preparation, not part of the method)
# ----------------------------------------------------------------------------

def _round_sig(x: np.ndarray, sig_bits: int, min_quantum_exp: int) -> np.ndarray:
    """Round float64 values to `sig_bits` significant bits, ties to even, with
    gradual underflow below 2**min_quantum_exp. Exact: every step is a scaling
    by a power of two or numpy's half-to-even round of an exact value."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    qexp = np.maximum(e - sig_bits, min_quantum_exp)
    return np.ldexp(np.round(np.ldexp(x, -qexp)), qexp)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 -> value exactly representable in `dtype` (returned as
    float64). Round-to-nearest-even, one rounding step."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return _round_sig(x, 8, -133)
    if dtype == "f16":
        # numpy converts double -> half directly with round-half-even
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)
    raise ValueError(dtype)


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Exactly-representable float64 values -> storage array.
    f32 -> float32, f16 -> float16, bf16 -> uint16 bit patterns."""
    if dtype == "f32":
        return np.asarray(x64, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(x64).astype(np.float16)
    if dtype == "bf16":
        b32 = np.asarray(x64).astype(np.float32).view(np.uint32)
        return (b32 >> 16).astype(np.uint16)
    raise ValueError(dtype)


def from_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float64 (exact upcast)."""
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def draw_rounded(rng: np.random.Generator, shape, std: float, dtype: str):
    x = rng.standard_normal(shape) * std
    r = round_to(x, dtype)
    return to_storage(r, dtype)


def nan_storage(dtype: str):
    if dtype == "bf16":
        return np.uint16(0x7FC0)
    if dtype == "f16":
        return np.float16(np.nan)
    return np.float32(np.nan)


def storage_np_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


# ----------------------------------------------------------------------------
# workload table
# ----------------------------------------------------------------------------

@dataclass
class WorkloadSpec:
    wid: int
    name: str
    B: int
    H: int
    S: int                 # query tokens per sequence (q_len)
    dtype: str             # storage/compute dtype of q, cache, weights
    lengths: tuple         # ("fixed", L) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    block_size: int        # 0 = contiguous cache [B][L][576]
    parts: int             # history parts (DCP shards emulated on one GPU)
    part_out_dtype: str
    part_lse_dtype: str
    current: bool = False  # MTP current chunk (contiguous [B][S][576]) merged as local part
    out_dtype: Optional[str] = None  # combine output (latent) dtype; default dtype

    @property
    def scale(self) -> float:
        # 1/sqrt(d_nope + d_R) = 1/sqrt(192)
        return 1.0 / math.sqrt(D_NOPE + D_R)


SPECS = {
    0: WorkloadSpec(0, "tiny_fp32_B1_H16_L256_2parts", B=1, H=16, S=1, dtype="f32",
                    lengths=("fixed", 256), block_size=0, parts=2,
                    part_out_dtype="f32", part_lse_dtype="f32"),
    1: WorkloadSpec(1, "bf16_B32_H128_L4096_paged32_1part", B=32, H=128, S=1, dtype="bf16",
                    lengths=("fixed", 4096), block_size=32, parts=1,
                    part_out_dtype="bf16", part_lse_dtype="f32"),
    2: WorkloadSpec(2, "bf16_B32_H128_L32768_paged32_8parts", B=32, H=128, S=1, dtype="bf16",
                    lengths=("fixed", 32768), block_size=32, parts=8,
                    part_out_dtype="bf16", part_lse_dtype="bf16"),
    3: WorkloadSpec(3, "bf16_mtp_B64_H128_S2_hist1k-16k_paged32_4parts+current", B=64, H=128, S=2,
                    dtype="bf16", lengths=("uniform", 1024, 16384), block_size=32, parts=4,
                    part_out_dtype="bf16", part_lse_dtype="f32", current=True),
    4: WorkloadSpec(4, "fp16_B128_H128_L512-8192log_paged64_2parts", B=128, H=128, S=1, dtype="f16",
                    lengths=("loguniform", 512, 8192), block_size=64, parts=2,
                    part_out_dtype="f16", part_lse_dtype="f16"),
}


def spec(wid: int, **over) -> WorkloadSpec:
    """Workload spec, optionally with fields overridden (smaller parity cases)."""
    s = SPECS[wid]
    d = dict(s.__dict__)
    d.update(over)
    return WorkloadSpec(**d)


def draw_lengths(rng: np.random.Generator, sp: WorkloadSpec) -> np.ndarray:
    kind = sp.lengths[0]
    if kind == "fixed":
        return np.full(sp.B, sp.lengths[1], dtype=np.int64)
    if kind == "uniform":
        lo, hi = sp.lengths[1], sp.lengths[2]
        return rng.integers(lo, hi + 1, size=sp.B).astype(np.int64)
    if kind == "loguniform":
        lo, hi = sp.lengths[1], sp.lengths[2]
        u = rng.uniform(math.log(lo), math.log(hi), size=sp.B)
        return np.clip(np.round(np.exp(u)), lo, hi).astype(np.int64)
    raise ValueError(kind)


def part_ranges(lengths: np.ndarray, parts: int, align: int):
    """Block-aligned near-equal contiguous split of each sequence's keys.
    With nb = ceil(L/align) units, part p covers units
    [floor(p*nb/P), floor((p+1)*nb/P)), clipped to L. Returns int32 [P][B]
    start/end (logical token positions)."""
    B = len(lengths)
    st = np.zeros((parts, B), dtype=np.int32)
    en = np.zeros((parts, B), dtype=np.int32)
    for b in range(B):
        L = int(lengths[b])
        nb = -(-L // align)
        for p in range(parts):
            s0 = (p * nb) // parts * align
            s1 = ((p + 1) * nb) // parts * align
            st[p, b] = min(s0, L)
            en[p, b] = min(s1, L)
    return st, en


@dataclass
class Workload:
    spec: WorkloadSpec
    seed: int
    lengths: np.ndarray                 # [B] history/cached lengths
    w_uk: np.ndarray                    # [H][512][128] storage
    w_uv: np.ndarray                    # [H][512][128] storage
    q_nope: np.ndarray                  # [T][H][128] storage, t = b*S + s
    q_rope: np.ndarray                  # [T][H][64] storage
    kv: np.ndarray                      # paged [NB][bs][576] | contiguous [B][Lmax][576]
    block_table: Optional[np.ndarray]   # int32 [B][max_blocks] (-1 = unused) | None
    range_start: np.ndarray             # int32 [P][B]
    range_end: np.ndarray               # int32 [P][B]
    cur_kv: Optional[np.ndarray] = None  # contiguous [B][S][576] storage (MTP current chunk)
    extra: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return self.spec.B * self.spec.S

    def seq_rows64(self, b: int) -> np.ndarray:
        """Logical-order latent rows [L_b][576] of sequence b, as float64."""
        sp = self.spec
        L = int(self.lengths[b])
        if sp.block_size == 0:
            rows = self.kv[b, :L]
        else:
            bs = sp.block_size
            nb = -(-L // bs)
            blocks = self.block_table[b, :nb]
            rows = self.kv[blocks].reshape(nb * bs, D_ROW)[:L]
        return from_storage(rows, sp.dtype)

    def cur_rows64(self, b: int) -> np.ndarray:
        return from_storage(self.cur_kv[b], self.spec.dtype)

    def f64(self, name: str) -> np.ndarray:
        return from_storage(getattr(self, name), self.spec.dtype)


def make_workload(wid_or_spec, seed: Optional[int] = None, extra_blocks: int = 0,
                  poison: bool = True) -> Workload:
    """Build the seeded synthetic inputs of a workload.

    Unused cache slots (past a sequence's length inside its last block) and
    `extra_blocks` unreferenced blocks are filled with NaN when `poison` is
    set, so any read of them shows up in the results."""
    sp = SPECS[wid_or_spec] if isinstance(wid_or_spec, int) else wid_or_spec
    if seed is None:
        seed = 1000 + sp.wid
    rng = np.random.Generator(np.random.PCG64(seed))
    dt = sp.dtype
    B, H, S = sp.B, sp.H, sp.S
    T = B * S
    wstd = 1.0 / math.sqrt(D_C)

    lengths = draw_lengths(rng, sp)
    w_uk = draw_rounded(rng, (H, D_C, D_NOPE), wstd, dt)
    w_uv = draw_rounded(rng, (H, D_C, D_V), wstd, dt)
    q_nope = draw_rounded(rng, (T, H, D_NOPE), 1.0, dt)
    q_rope = draw_rounded(rng, (T, H, D_R), 1.0, dt)

    # latent rows, logical order, sequence-major; c_KV first, then k_R
    ntot = int(lengths.sum())
    c_all = np.empty((ntot, D_C), dtype=storage_np_dtype(dt))
    CH = 1 << 20
    for i in range(0, ntot, CH // D_C * 64):
        n = min(ntot - i, CH // D_C * 64)
        c_all[i:i + n] = draw_rounded(rng, (n, D_C), 1.0, dt)
    kr_all = np.empty((ntot, D_R), dtype=storage_np_dtype(dt))
    for i in range(0, ntot, CH // D_R * 8):
        n = min(ntot - i, CH // D_R * 8)
        kr_all[i:i + n] = draw_rounded(rng, (n, D_R), 1.0, dt)

    cur_kv = None
    if sp.current:
        cur_c = draw_rounded(rng, (B, S, D_C), 1.0, dt)
        cur_r = draw_rounded(rng, (B, S, D_R), 1.0, dt)
        cur_kv = np.concatenate([cur_c, cur_r], axis=2)

    offs = np.concatenate([[0], np.cumsum(lengths)])
    nanv = nan_storage(dt)
    if sp.block_size == 0:
        Lmax = int(lengths.max())
        kv = np.empty((B, Lmax, D_ROW), dtype=storage_np_dtype(dt))
        kv[...] = nanv if poison else 0
        for b in range(B):
            L = int(lengths[b])
            kv[b, :L, :D_C] = c_all[offs[b]:offs[b] + L]
            kv[b, :L, D_C:] = kr_all[offs[b]:offs[b] + L]
        block_table = None
        align = 32
    else:
        bs = sp.block_size
        nblk = -(-lengths // bs)
        NB = int(nblk.sum())
        perm = rng.permutation(NB + extra_blocks)
        used = perm[:NB] if extra_blocks == 0 else perm[:NB]
        kv = np.empty((NB + extra_blocks, bs, D_ROW), dtype=storage_np_dtype(dt))
        if poison:
            kv[...] = nanv
        else:
            kv[...] = 0
        max_blocks = int(nblk.max())
        block_table = np.full((B, max_blocks), -1, dtype=np.int32)
        boff = np.concatenate([[0], np.cumsum(nblk)])
        for b in range(B):
            L = int(lengths[b])
            ids = used[boff[b]:boff[b + 1]]
            block_table[b, :len(ids)] = ids
            rows_c = c_all[offs[b]:offs[b] + L]
            rows_r = kr_all[offs[b]:offs[b] + L]
            full = L // bs
            if full:
                kv[ids[:full], :, :D_C] = rows_c[:full * bs].reshape(full, bs, D_C)
                kv[ids[:full], :, D_C:] = rows_r[:full * bs].reshape(full, bs, D_R)
            rem = L - full * bs
            if rem:
                kv[ids[full], :rem, :D_C] = rows_c[full * bs:]
                kv[ids[full], :rem, D_C:] = rows_r[full * bs:]
        align = bs
    del c_all, kr_all
    rs, re = part_ranges(lengths, sp.parts, align)
    return Workload(sp, seed, lengths, w_uk, w_uv, q_nope, q_rope, kv, block_table,
                    rs, re, cur_kv)


# ----------------------------------------------------------------------------
# algorithmic work accounting (bytes that the method must move / flops it must
# do; the dense per-head K/V that absorption avoids is not counted)
# ----------------------------------------------------------------------------

def kv_bytes_per_token(dtype: str) -> int:
    return D_ROW * ESIZE[dtype]


def step_work(w: Workload) -> dict:
    """Algorithmic bytes and flops of one decode step (q-absorb, partial
    attention over all parts, LSE combine, V-up)."""
    sp = w.spec
    e = ESIZE[sp.dtype]
    T, H, P = w.T, sp.H, sp.parts
    keys = int(w.lengths.sum())
    cur_keys = sp.B * sp.S if sp.current else 0
    # (query, key, head) triples that are scored
    pairs = keys * sp.S * H
    if sp.current:
        pairs += sp.B * (sp.S * (sp.S + 1) // 2) * H
    kv_b = (keys + cur_keys) * D_ROW * e
    pe, le = ESIZE[sp.part_out_dtype], ESIZE[sp.part_lse_dtype]
    nparts = P + (1 if sp.current else 0)
    absorb_b = (T * H * D_NOPE + H * D_C * D_NOPE + T * H * D_C) * e
    calls = 2 if sp.current else 1   # history call (+ current-chunk call)
    partial_b = kv_b + calls * T * H * (D_C + D_R) * e + nparts * T * H * (D_C * pe + le)
    combine_b = nparts * T * H * (D_C * pe + le) + T * H * (D_C * e + 4)
    vup_b = (T * H * D_C + H * D_C * D_V + T * H * D_V) * e
    flops_attn = pairs * 2 * (D_ROW + D_C)
    flops_absorb = 2 * T * H * D_C * D_NOPE
    flops_vup = 2 * T * H * D_C * D_V
    flops_comb = nparts * T * H * D_C * 2
    return dict(
        kv_bytes=kv_b, absorb_bytes=absorb_b, partial_bytes=partial_b,
        combine_bytes=combine_b, vup_bytes=vup_b,
        total_bytes=absorb_b + partial_b + combine_b + vup_b,
        attn_flops=flops_attn, total_flops=flops_attn + flops_absorb + flops_vup + flops_comb,
        keys=keys, pairs=pairs,
    )
