"""A seeded sweep of random shapes through the whole decode step and the
partial call, each against the float64 oracle: batch sizes, head counts,
query lengths, block sizes (paged 32 / 64 / 128 and contiguous), part
counts, explicit and automatic split counts, ragged and empty ranges, and
the three storage types; every other case with the split plan built on the
host, and half the cases with a current chunk in the history call's launch.
A second sweep covers query lengths up to 8 with a current chunk and
sequences that share cache blocks. Sizes stay small enough for the oracle to
finish in seconds per case."""
import numpy as np
import pytest
import torch

import oracle.mla_oracle as mo
from mla_split_kv_absorbed_amd import _lib as L
from mla_split_kv_absorbed_amd import workloads as W
from mla_split_kv_absorbed_amd.step import DecodeStep
from tests.test_gpu_parity import check_partial, check_step, oracle_qlat, say

pytestmark = pytest.mark.gpu

N_CASES = 128


def draw_case(i):
    """Workload spec overrides and a split count for sweep case i."""
    r = np.random.Generator(np.random.PCG64(5000 + i))
    dtype = ["bf16", "f16", "bf16", "f16", "f32"][i % 5]
    bs = int(r.choice([0, 16, 32, 64, 128]))
    B = int(r.integers(1, 7))
    H = int(r.choice([8, 16, 40, 128, 130]))
    S = int(r.choice([1, 1, 2, 3]))
    parts = int(r.integers(1, 6))
    lo = int(r.integers(1, 200))
    hi = lo + int(r.integers(0, 1800))
    over = dict(B=B, H=H, S=S, dtype=dtype, block_size=bs, parts=parts,
                lengths=("uniform", lo, hi), current=bool(S > 1 and r.random() < 0.7),
                part_out_dtype=dtype if dtype != "f32" else "f32",
                part_lse_dtype=str(r.choice(["f32", dtype])))
    splits = int(r.choice([0, 0, 1, 2, 3, 7]))
    return over, splits


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_step_and_partial(i):
    over, splits = draw_case(i)
    wid = 2 if over["dtype"] != "f32" else 0
    sp = W.spec(wid, **over)
    say(f"[sweep {i}] {over} splits={splits}")
    w = W.make_workload(sp)
    # the whole step (absorb, partial over the parts [+ current], combine, V-up);
    # every other case hands the partial call a plan built on the host, and
    # every other case with a current chunk runs it in the history's launch
    st = DecodeStep(w, num_splits=splits, auto_plan=splits == 0, host_plan=i % 2 == 0,
                    pair_current=i % 4 < 2)
    st.run()
    torch.cuda.synchronize()
    extra = sp.part_lse_dtype if sp.part_lse_dtype != "f32" else None
    heads = sorted(set(list(range(0, sp.H, max(1, sp.H // 6))) + [sp.H - 1]))
    check_step(w, st, list(range(sp.B)), heads, extra)
    # the partial call alone, every row, from the oracle's own queries
    qs = oracle_qlat(w)
    sp2 = DecodeStep(w, q_lat_in=qs, num_splits=splits, auto_plan=splits == 0)
    sp2.parts_out.fill_(float("nan"))
    sp2.parts_lse.fill_(float("nan"))
    L.mla_decode_partial(sp2.hist_args)
    torch.cuda.synchronize()
    check_partial(w, sp2, qs)


# ---------------------------------------------------------------------------
# multi-token decoding and shared cache blocks
# ---------------------------------------------------------------------------

def draw_mtp_case(i):
    """Sweep case i of query lengths 1-8 (a current chunk for most S > 1),
    bf16 / fp16, and whether the sequences share cache blocks, the current
    chunk runs in the history's launch (else, in every other case, on a side
    stream), and the plan is built on the host."""
    r = np.random.Generator(np.random.PCG64(7000 + i))
    dt = ["bf16", "f16"][i % 2]
    S = int(r.integers(1, 9))
    over = dict(B=int(r.integers(2, 6)), H=int(r.choice([16, 128, 130])), S=S, dtype=dt,
                block_size=int(r.choice([16, 32, 64])), parts=int(r.integers(1, 5)),
                lengths=("uniform", int(r.integers(50, 400)), int(r.integers(400, 2500))),
                current=bool(S > 1 and r.random() < 0.8), part_out_dtype=dt,
                part_lse_dtype=str(r.choice(["f32", dt])))
    splits = int(r.choice([0, 0, 1, 2, 3]))
    return over, splits, bool(r.random() < 0.6), bool(r.random() < 0.5), bool(r.random() < 0.5)


@pytest.mark.parametrize("i", range(48))
def test_sweep_mtp_shared_blocks(i):
    """Whole step and partial call against the oracle; with `share`, every
    sequence after the first reads the first sequence's full cache blocks as
    its prefix (one physical block in several block-table rows, as prefix
    sharing makes it)."""
    over, splits, share, pair, host = draw_mtp_case(i)
    sp = W.spec(2 if over["dtype"] == "bf16" else 4, **over)
    say(f"[sweep-mtp {i}] {over} splits={splits} share={share} pair={pair} host={host}")
    w = W.make_workload(sp)
    if share:
        bs = sp.block_size
        full0 = int(w.lengths[0]) // bs
        for b in range(1, sp.B):
            k = min(full0, int(w.lengths[b]) // bs)
            w.block_table[b, :k] = w.block_table[0, :k]
    # a current chunk not paired with the history runs on a side stream in
    # every other such case
    side = sp.current and not pair and i % 2 == 1
    st = DecodeStep(w, num_splits=splits, auto_plan=splits == 0, host_plan=host and splits == 0,
                    pair_current=pair and sp.current, side_stream=side)
    st.run()
    torch.cuda.synchronize()
    extra = sp.part_lse_dtype if sp.part_lse_dtype != "f32" else None
    heads = sorted(set(list(range(0, sp.H, max(1, sp.H // 5))) + [sp.H - 1]))
    check_step(w, st, list(range(sp.B)), heads, extra)
    qs = oracle_qlat(w)
    st2 = DecodeStep(w, q_lat_in=qs, num_splits=splits, auto_plan=splits == 0)
    st2.parts_out.fill_(float("nan"))
    st2.parts_lse.fill_(float("nan"))
    L.mla_decode_partial(st2.hist_args)
    torch.cuda.synchronize()
    check_partial(w, st2, qs)
