"""The allocation-free partial entry point (mla_decode_partial_noalloc)
against mla_decode_partial, through the C ABI: the same kernels over the
library's own device scratch instead of a caller workspace. Two calls in a
row, the second with a smaller input, each bit for bit equal to the
workspace entry point's result and within the oracle's tolerance; a call
without sub-ranges (only the workspace header); and the large call again
after the small ones, so a stale scratch from an earlier call cannot leak
into a later one."""
import numpy as np
import pytest
import torch

from mla_split_kv_absorbed_amd import _lib as L
from mla_split_kv_absorbed_amd import workloads as W
from mla_split_kv_absorbed_amd.step import DecodeStep
from tests.test_gpu_parity import check_partial, oracle_qlat, say

pytestmark = pytest.mark.gpu

# (workload, overrides, num_splits): the first uses the automatic plan's
# sub-ranges (scratch in use), the second is smaller with explicit pieces,
# the third needs no workspace at all
SEQUENCE = [
    (1, dict(B=6, lengths=("uniform", 900, 3000)), 0),
    (4, dict(B=3, lengths=("loguniform", 100, 900)), 3),
    (2, dict(B=2, lengths=("fixed", 500), parts=2), 1),
]


def run_both(wid, over, splits):
    sp = W.spec(wid, **over)
    w = W.make_workload(sp)
    qs = oracle_qlat(w)
    st = DecodeStep(w, q_lat_in=qs, num_splits=splits, auto_plan=True)
    need = L.mla_decode_partial_workspace_size(st.hist_args)
    assert need <= L.mla_noalloc_scratch_bytes()
    L.mla_decode_partial(st.hist_args)
    torch.cuda.synchronize()
    ref_o, ref_l = st.parts_out.clone(), st.parts_lse.clone()
    st.parts_out.fill_(float("nan"))
    st.parts_lse.fill_(float("nan"))
    # the caller's workspace fields are ignored
    st.hist_args.workspace, st.hist_args.workspace_bytes = None, 0
    L.mla_decode_partial_noalloc(st.hist_args)
    torch.cuda.synchronize()
    say(f"[noalloc] {sp.name} splits={splits} workspace {need} B")
    assert torch.equal(st.parts_out, ref_o) and torch.equal(st.parts_lse, ref_l)
    check_partial(w, st, qs)
    return need


def test_noalloc_matches_the_workspace_entry_point():
    needs = [run_both(*c) for c in SEQUENCE]
    assert needs[0] > needs[1] > needs[2] > 0
    # again, the large call after the small ones
    run_both(*SEQUENCE[0])


def test_noalloc_rejects_calls_beyond_the_scratch():
    sp = W.spec(2, H=512, B=2, lengths=("fixed", 256), parts=1)
    w = W.make_workload(sp)
    st = DecodeStep(w, auto_plan=True)
    assert L.mla_decode_partial_workspace_size(st.hist_args) > L.mla_noalloc_scratch_bytes()
    with pytest.raises(L.MLAError) as e:
        L.mla_decode_partial_noalloc(st.hist_args)
    assert e.value.status == -5
