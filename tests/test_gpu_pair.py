"""The HISTORY and CURRENT partial calls in one launch (mla_decode_partial_pair)
against the two separate calls and the float64 oracle.

The current chunk's short-range tasks ride in the matrix kernel's grid behind
the history's chunks. Each case checks that the paired step is bit for bit
the step made of two calls (both partial outputs, both LSEs and the final
output), that it matches the oracle's non-absorbed attention, and that the
current part's buffers, poisoned with NaN before the paired launch, are all
written. Cases: the MTP workload's shape at small size (bf16 and fp16, the
automatic plan built on the device and on the host), two head groups
(H = 200), 5 query tokens per sequence, and the full-size MTP workload on a
sample of sequences."""
import numpy as np
import pytest
import torch

from mla_split_kv_absorbed_amd import _lib as L
from mla_split_kv_absorbed_amd import workloads as W
from mla_split_kv_absorbed_amd.step import DecodeStep
from tests.test_gpu_parity import check_step, oracle_qlat, say

pytestmark = pytest.mark.gpu

CASES = {
    "bf16": (dict(B=6, lengths=("uniform", 100, 1500)), {}),
    "bf16_host_plan": (dict(B=6, lengths=("uniform", 100, 1500)), dict(host_plan=True)),
    "f16": (dict(B=5, lengths=("uniform", 60, 900), dtype="f16", part_out_dtype="f16",
                 part_lse_dtype="f16"), {}),
    "h200": (dict(B=3, H=200, lengths=("uniform", 200, 700)), {}),
    "s5": (dict(B=3, S=5, lengths=("uniform", 100, 600)), {}),
    "full": (None, dict(host_plan=True)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_pair_step(case):
    over, opts = CASES[case]
    sp = W.SPECS[3] if over is None else W.spec(3, **over)
    say(f"[pair] {case}")
    w = W.make_workload(sp)
    ser = DecodeStep(w, **opts)
    ser.run()
    pair = DecodeStep(w, pair_current=True, **opts)
    assert pair.pair
    for _ in range(2):
        pair.cur_out.fill_(float("nan"))
        pair.cur_lse.fill_(float("nan"))
        pair.parts_out.fill_(float("nan"))
        pair.run()
        torch.cuda.synchronize()
        assert torch.equal(pair.parts_out, ser.parts_out)
        assert torch.equal(pair.parts_lse, ser.parts_lse)
        assert torch.equal(pair.cur_out, ser.cur_out)
        assert torch.equal(pair.cur_lse, ser.cur_lse)
        assert torch.equal(pair.out, ser.out)
    seqs = list(range(sp.B)) if over is not None else [0, 21, 42, 63]
    heads = list(range(0, sp.H, 9))
    extra = sp.part_lse_dtype if sp.part_lse_dtype != "f32" else None
    check_step(w, pair, seqs, heads, extra)


def test_pair_invalid_ranges_are_contained():
    """Invalid ranges in either call of a pair (a history range starting
    below 0, a current range ending past the chunk) give NaN rows for those
    ranges only, exactly as the two separate calls do."""
    sp = W.spec(3, B=4, lengths=("uniform", 100, 900))
    say("[pair] invalid ranges")
    w = W.make_workload(sp)
    qs = oracle_qlat(w)  # the partial calls alone read q_lat: set it
    ser = DecodeStep(w, q_lat_in=qs)
    pair = DecodeStep(w, q_lat_in=qs, pair_current=True)
    assert pair.pair
    for st in (ser, pair):
        st.range_start[1, 2] = -1
        st.cur_end[0, 3] = sp.S + 1
        st.parts_out.fill_(0.5)
        st.cur_out.fill_(0.5)
        if st is ser:
            L.mla_decode_partial(st.hist_args)
            L.mla_decode_partial(st.cur_args)
        else:
            L.mla_decode_partial_pair(st.hist_args, st.cur_args)
    torch.cuda.synchronize()
    assert torch.equal(pair.parts_out.isnan(), ser.parts_out.isnan())
    assert torch.equal(pair.parts_out.nan_to_num(7.0), ser.parts_out.nan_to_num(7.0))
    assert torch.equal(pair.cur_out.nan_to_num(7.0), ser.cur_out.nan_to_num(7.0))
    assert torch.equal(pair.cur_lse.nan_to_num(7.0), ser.cur_lse.nan_to_num(7.0))
    S = sp.S
    assert bool(pair.parts_out[1, 2 * S:3 * S].isnan().all())
    assert bool(pair.cur_out[3 * S:4 * S].isnan().all())
    assert not bool(pair.cur_out[:3 * S].isnan().any())
