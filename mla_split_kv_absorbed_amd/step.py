"""One absorbed split-KV MLA decode step on the device, as four library calls:

  mla_q_absorb -> mla_decode_partial (history parts [+ current chunk])
  -> mla_lse_combine -> mla_vup

This module only uploads a workload, allocates the outputs and marshals
arguments; all arithmetic happens in libmla_decode.so.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import _lib as L
from .workloads import D_C, D_V, Workload

# workgroups one partial-attention call aims to spread over (the kernel
# planner's target; one per compute unit), keys per tile and the smallest
# chunk the planner cuts (the library's own constants)
TARGET_GROUPS = 256
TILE = 32
MIN_CHUNK_TILES = 4

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Storage array (bf16 as uint16 bits) -> device tensor of `dtype`."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def split_hint(range_start: np.ndarray, range_end: np.ndarray, S: int) -> int:
    """Sub-split count for mla_decode_partial from the host-side ranges.

    When every range has the same length and the same number of 32-key tiles,
    the kernel's automatic plan would cut each range into the same number of
    chunks, longest first, which for equal ranges is range order. Passing
    that count explicitly lets the kernel skip the plan. It is 1 (no
    sub-splits) when the (range, query) units already fill the target
    workgroup count. Otherwise the count mirrors the plan: chunks of
    c = max(4, ceil(all tiles x S / 256)) tiles, or, when those make between
    one and two rounds of 256 workgroups, the smaller chunk that fills two
    rounds if its chunks fit in them. Ragged or empty ranges give 0 (let the
    kernel plan)."""
    st = np.asarray(range_start, np.int64).ravel()
    en = np.asarray(range_end, np.int64).ravel()
    if not st.size:
        return 0
    lens = en - st
    if lens.min() != lens.max() or lens.min() <= 0:
        return 0
    tiles = (en - 1) // TILE - st // TILE + 1
    if tiles.min() != tiles.max():
        return 0
    nt, units = int(tiles[0]), st.size
    if units * S >= TARGET_GROUPS:
        return 1
    G, total = TARGET_GROUPS, units * nt
    c = max(MIN_CHUNK_TILES, -(-total * S // G))
    if 4 * G > S * units:
        c1 = max(MIN_CHUNK_TILES, -(-2 * S * total // (4 * G - S * units)), -(-total * S // (2 * G)))
        if c1 < c and S * units * -(-nt // c) > G and S * units * -(-nt // c1) <= 2 * G:
            c = c1
    return max(1, -(-nt // c))


def cut_ranges(range_start: np.ndarray, range_end: np.ndarray, k: int):
    """Each range [start, end) cut into k pieces on 32-key tile boundaries:
    piece i takes tiles [i nt / k, (i + 1) nt / k) of the range's nt tiles
    (the kernel's own cut), clipped to the range. Returns [k][n] starts and
    ends; a piece with no tile is empty."""
    st = np.asarray(range_start, np.int64).ravel()
    en = np.asarray(range_end, np.int64).ravel()
    out_st = np.zeros((k, st.size), np.int32)
    out_en = np.zeros((k, st.size), np.int32)
    for j, (a, e) in enumerate(zip(st, en)):
        if e <= a:
            out_st[:, j] = out_en[:, j] = a
            continue
        t0, nt = a // TILE, (e - 1) // TILE - a // TILE + 1
        for i in range(k):
            lo, hi = i * nt // k, (i + 1) * nt // k
            ps = a if lo == 0 else (t0 + lo) * TILE
            pe = min(e, (t0 + hi) * TILE) if hi > lo else ps
            out_st[i, j], out_en[i, j] = ps, max(ps, pe)
    return out_st, out_en


class DecodeStep:
    """Device-resident inputs, outputs and workspace of one decode step."""

    def __init__(self, w: Workload, device="cuda", part_lse_dtype: Optional[str] = None,
                 num_splits: int = 0, flags: int = 0, q_lat_in: Optional[np.ndarray] = None,
                 side_stream: bool = False, fused_tail: bool = True, keep_latent: bool = False,
                 host_subranges: bool = False):
        """host_subranges: a single part without a current chunk, whose
        ranges the partial call would cut into k > 1 sub-ranges (equal ranges,
        bf16 / fp16), is instead cut on the host (cut_ranges) and passed as k
        parts, merged by the fused combine + V-up; the partial then runs
        without its own merge launch."""
        sp = w.spec
        self.w = w
        self.dev = torch.device(device)
        dt = sp.dtype
        self.dt = TORCH_DT[dt]
        B, H, S, T, P = sp.B, sp.H, sp.S, w.T, sp.parts
        self.B, self.H, self.S, self.T, self.P = B, H, S, T, P
        pdt = TORCH_DT[sp.part_out_dtype]
        ldt = TORCH_DT[part_lse_dtype or sp.part_lse_dtype]
        odt = TORCH_DT[sp.out_dtype or dt]
        dev = self.dev

        self.w_uk = to_device(w.w_uk, dt, dev)
        self.w_uv = to_device(w.w_uv, dt, dev)
        self.q_nope = to_device(w.q_nope, dt, dev)
        self.q_rope = to_device(w.q_rope, dt, dev)
        self.kv = to_device(w.kv, dt, dev)
        self.block_table = (torch.from_numpy(w.block_table).to(dev)
                            if w.block_table is not None else None)
        rs, re_ = w.range_start, w.range_end
        self.host_cut = 1
        if (host_subranges and P == 1 and not sp.current and num_splits == 0
                and dt in ("bf16", "f16")):
            k = split_hint(rs, re_, S)
            if k > 1:
                rs, re_ = cut_ranges(rs, re_, k)
                self.host_cut, P, self.P, num_splits = k, k, k, 1
        self.range_start = torch.from_numpy(np.ascontiguousarray(rs)).to(dev)
        self.range_end = torch.from_numpy(np.ascontiguousarray(re_)).to(dev)
        self.q_lat = torch.empty((T, H, D_C), dtype=self.dt, device=dev)
        self.absorb = q_lat_in is None
        if q_lat_in is not None:
            self.q_lat.copy_(to_device(q_lat_in, dt, dev))
        self.parts_out = torch.empty((P, T, H, D_C), dtype=pdt, device=dev)
        self.parts_lse = torch.empty((P, T, H), dtype=ldt, device=dev)
        self.lat = torch.empty((T, H, D_C), dtype=odt, device=dev)
        self.lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        self.out = torch.empty((T, H, D_V), dtype=self.dt, device=dev)

        explicit_splits = num_splits
        if num_splits == 0:
            num_splits = split_hint(w.range_start, w.range_end, S)
        self.num_splits = num_splits
        kw = dict(B=B, S=S, H=H, scale=sp.scale, num_splits=num_splits, flags=flags)
        if sp.block_size > 0:
            kw.update(block_table=self.block_table, block_size=sp.block_size,
                      num_blocks=w.kv.shape[0])
        else:
            kw.update(kv_seq_stride=w.kv.shape[1])
        self.hist_args = L.partial_args(self.q_lat, self.q_rope, self.kv, self.range_start,
                                        self.range_end, self.parts_out, self.parts_lse, **kw)
        ws = L.mla_decode_partial_workspace_size(self.hist_args)
        self.cur = None
        if sp.current:
            self.cur_kv = to_device(w.cur_kv, dt, dev)
            self.cur_start = torch.zeros((1, B), dtype=torch.int32, device=dev)
            self.cur_end = torch.full((1, B), S, dtype=torch.int32, device=dev)
            self.cur_out = torch.empty((T, H, D_C), dtype=pdt, device=dev)
            self.cur_lse = torch.empty((T, H), dtype=ldt, device=dev)
            self.cur_args = L.partial_args(self.q_lat, self.q_rope, self.cur_kv, self.cur_start,
                                           self.cur_end, self.cur_out, self.cur_lse,
                                           B=B, S=S, H=H, scale=sp.scale, kv_seq_stride=S,
                                           mask=L.MLA_MASK_CAUSAL_WINDOW,
                                           num_splits=explicit_splits or split_hint(
                                               np.zeros(B), np.full(B, S), S),
                                           flags=flags)
            ws = max(ws, L.mla_decode_partial_workspace_size(self.cur_args))
        self.workspace = torch.empty((max(ws, 1),), dtype=torch.uint8, device=dev)
        for a in [self.hist_args] + ([self.cur_args] if sp.current else []):
            a.workspace = self.workspace.data_ptr()
            a.workspace_bytes = self.workspace.numel()
        # Current-chunk attention on a side stream, concurrent with the
        # history partial (the study page's stream split). It gets its own
        # workspace: a workspace belongs to one call until its stream has
        # passed it. Every buffer it touches is owned by this object for its
        # whole life, so no allocator stream bookkeeping is needed.
        self.side = None
        if side_stream and sp.current:
            self.side = torch.cuda.Stream(device=dev)  # default priority
            self.cur_workspace = torch.empty((max(ws, 1),), dtype=torch.uint8, device=dev)
            self.cur_args.workspace = self.cur_workspace.data_ptr()
            self.cur_args.workspace_bytes = self.cur_workspace.numel()
            self.ev_q = torch.cuda.Event()    # q_lat ready (main -> side)
            self.ev_cur = torch.cuda.Event()  # current partial done (side -> main)
        # with a single part and no local part the partial already is the
        # merged latent; the combine is skipped
        self.skip_combine = (P == 1 and not sp.current and pdt == odt
                             and self.parts_lse.dtype == torch.float32)
        # combine and V-up as one launch (bf16 / fp16); the merged latent is
        # then written only with keep_latent
        self.fused_tail = (fused_tail and not self.skip_combine and odt == self.dt
                           and dt in ("bf16", "f16"))
        self.keep_latent = keep_latent or not self.fused_tail

    def run(self, stream=None):
        main = stream if stream is not None else torch.cuda.current_stream(self.dev)
        if self.absorb:
            L.mla_q_absorb(self.q_nope, self.w_uk, self.q_lat, main)
        if self.side is not None:
            # side stream: after q_lat, before the combine
            self.ev_q.record(main)
            self.side.wait_event(self.ev_q)
            L.mla_decode_partial(self.cur_args, self.side)
            self.ev_cur.record(self.side)
            L.mla_decode_partial(self.hist_args, main)
            main.wait_event(self.ev_cur)
        else:
            L.mla_decode_partial(self.hist_args, main)
            if self.w.spec.current:
                L.mla_decode_partial(self.cur_args, main)
        stream = main
        if self.fused_tail:
            L.mla_combine_vup(self.parts_out, self.parts_lse, self.w_uv, self.out, self.lse,
                              lat_out=self.lat if self.keep_latent else None,
                              local_out=self.cur_out if self.w.spec.current else None,
                              local_lse=self.cur_lse if self.w.spec.current else None,
                              stream=stream)
            return self.out
        if self.skip_combine:
            x = self.parts_out[0]
        else:
            L.mla_lse_combine(self.parts_out, self.parts_lse, self.lat, self.lse,
                              local_out=self.cur_out if self.w.spec.current else None,
                              local_lse=self.cur_lse if self.w.spec.current else None,
                              stream=stream)
            x = self.lat
        L.mla_vup(x, self.w_uv, self.out, stream)
        return self.out

    def final_lse(self) -> torch.Tensor:
        return self.parts_lse[0] if self.skip_combine else self.lse

    def final_latent(self) -> torch.Tensor:
        if not self.keep_latent:
            raise RuntimeError("the fused combine + V-up did not write the merged latent "
                               "(construct with keep_latent=True)")
        return self.parts_out[0] if self.skip_combine else self.lat
