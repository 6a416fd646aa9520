"""One absorbed split-KV MLA decode step on the device, as library calls:

  mla_q_absorb -> mla_decode_partial (history parts [+ current chunk], or
  both in one launch: mla_decode_partial_pair) -> mla_lse_combine -> mla_vup
  (the last two as one launch: mla_combine_vup)

This module only uploads a workload, allocates the outputs and marshals
arguments; all arithmetic happens in libmla_decode.so.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import _lib as L
from .workloads import D_C, D_V, Workload

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Storage array (bf16 as uint16 bits) -> device tensor of `dtype`."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DecodeStep:
    """Device-resident inputs, outputs and workspace of one decode step."""

    def __init__(self, w: Workload, device="cuda", part_lse_dtype: Optional[str] = None,
                 num_splits: int = 0, flags: int = 0, q_lat_in: Optional[np.ndarray] = None,
                 side_stream: bool = False, fused_tail: bool = True, keep_latent: bool = False,
                 host_subranges: bool = False, auto_plan: bool = False,
                 host_plan: bool = False, pair_current: bool = False):
        """num_splits: 0 lets the library plan; for equal ranges the plan's
        chunk count is then passed explicitly (the kernel skips its plan)
        unless auto_plan is set.
        host_plan: when the history call runs the automatic plan (ragged
        ranges, or auto_plan), the plan is built on the host from the ranges
        (mla_decode_partial_make_plan) and handed to the call in device
        memory, as a serving loop that holds its sequence lengths would.
        pair_current: when the current-chunk call takes the short-range
        kernel and the history call the matrix-core kernel, both run as one
        launch (mla_decode_partial_pair) instead of two; not with
        side_stream.
        host_subranges: a single part without a current chunk, whose
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
            k = self._plan(w, rs, re_, flags).equal_splits
            if k > 1:
                rs, re_ = L.mla_cut_ranges(rs, re_, k)
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
        kw = dict(B=B, S=S, H=H, scale=sp.scale, num_splits=num_splits, flags=flags)
        if sp.block_size > 0:
            kw.update(block_table=self.block_table, block_size=sp.block_size,
                      num_blocks=w.kv.shape[0])
        else:
            kw.update(kv_seq_stride=w.kv.shape[1])
        self.hist_args = L.partial_args(self.q_lat, self.q_rope, self.kv, self.range_start,
                                        self.range_end, self.parts_out, self.parts_lse, **kw)
        # equal ranges: pass the automatic plan's chunk count explicitly, so
        # the kernel cuts the same pieces without evaluating its plan
        if num_splits == 0 and not auto_plan:
            num_splits = L.mla_decode_partial_plan(self.hist_args, rs, re_).equal_splits
            self.hist_args.num_splits = num_splits
        self.num_splits = num_splits
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
                                           num_splits=explicit_splits, flags=flags)
            if explicit_splits == 0 and not auto_plan:
                self.cur_args.num_splits = L.mla_decode_partial_plan(
                    self.cur_args, np.zeros(B), np.full(B, S)).equal_splits
            ws = max(ws, L.mla_decode_partial_workspace_size(self.cur_args))
        self.workspace = torch.empty((max(ws, 1),), dtype=torch.uint8, device=dev)
        for a in [self.hist_args] + ([self.cur_args] if sp.current else []):
            a.workspace = self.workspace.data_ptr()
            a.workspace_bytes = self.workspace.numel()
        self.plan = None
        if (host_plan and self.hist_args.num_splits == 0
                and L.mla_decode_partial_plan_words(self.hist_args) > 0):
            table, info = L.mla_decode_partial_make_plan(self.hist_args, rs, re_)
            self.plan = torch.from_numpy(table).to(dev)
            self.hist_args.plan = self.plan.data_ptr()
            self.hist_args.plan_chunks = info.chunks
            self.hist_args.plan_split_units = info.split_ranges
        # the history and the current-chunk calls in one launch, when their
        # kernels allow it
        self.pair = False
        if pair_current and sp.current and not side_stream:
            hist_path = L.mla_decode_partial_plan(self.hist_args, rs, re_).matrix_path
            cur_path = L.mla_decode_partial_plan(self.cur_args, np.zeros(B, np.int32),
                                                 np.full(B, S, np.int32)).matrix_path
            self.pair = hist_path == 1 and cur_path == 2
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

    def _plan(self, w: Workload, rs, re_, flags) -> "L.SplitInfo":
        """The library's split plan for a single part with these ranges (the
        device pointers of the throwaway argument struct are never read)."""
        sp = w.spec
        dummy = torch.empty(1, dtype=self.dt)
        lse = torch.empty(1, dtype=torch.float32)
        kw = dict(B=sp.B, S=sp.S, H=sp.H, scale=sp.scale, flags=flags)
        if sp.block_size > 0:
            bt = torch.from_numpy(np.ascontiguousarray(w.block_table))
            kw.update(block_table=bt, block_size=sp.block_size, num_blocks=w.kv.shape[0])
        else:
            kw.update(kv_seq_stride=w.kv.shape[1])
        rs_t = torch.from_numpy(np.ascontiguousarray(rs, dtype=np.int32))
        a = L.partial_args(dummy, dummy, dummy, rs_t, rs_t, dummy, lse, **kw)
        return L.mla_decode_partial_plan(a, rs, re_)

    def run(self, stream=None, marks: Optional[dict] = None):
        """Enqueues one step. `marks` (optional) maps "current_done" and
        "tail_start" to timing events, recorded after the current-chunk
        partial (on its stream) and before the combine (on the main stream),
        so a caller can check the order the streams ran in."""
        main = stream if stream is not None else torch.cuda.current_stream(self.dev)
        marks = marks or {}
        if self.absorb:
            L.mla_q_absorb(self.q_nope, self.w_uk, self.q_lat, main)
        if self.side is not None:
            # side stream: after q_lat, before the combine
            self.ev_q.record(main)
            self.side.wait_event(self.ev_q)
            L.mla_decode_partial(self.cur_args, self.side)
            if "current_done" in marks:
                marks["current_done"].record(self.side)
            self.ev_cur.record(self.side)
            L.mla_decode_partial(self.hist_args, main)
            main.wait_event(self.ev_cur)
        elif self.pair:
            L.mla_decode_partial_pair(self.hist_args, self.cur_args, main)
            if "current_done" in marks:
                marks["current_done"].record(main)
        else:
            L.mla_decode_partial(self.hist_args, main)
            if self.w.spec.current:
                L.mla_decode_partial(self.cur_args, main)
                if "current_done" in marks:
                    marks["current_done"].record(main)
        if "tail_start" in marks:
            marks["tail_start"].record(main)
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
