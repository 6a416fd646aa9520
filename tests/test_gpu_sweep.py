"""A seeded sweep of random shapes through the whole decode step and the
partial call, each against the float64 oracle: batch sizes, head counts,
query lengths, block sizes (paged 32 / 64 / 128 and contiguous), part
counts, explicit and automatic split counts, ragged and empty ranges, and
the three storage types; every other case with the split plan built on the
host, and half the cases with a current chunk in the history call's launch. Sizes stay small enough for the oracle to finish in seconds per case."""
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
