"""The partial call given a plan built on the host (mla_decode_partial_make_plan)
against the same call planning on the device: the same chunks run the same
arithmetic, so the outputs and LSEs must be equal bit for bit. Ragged and
equal ranges, one and two queries, two groups of 128 heads, paged and
contiguous caches, explicit split counts, a plan that cuts no range (no merge
launch), and the allocation-free entry point; one case also against the
oracle."""
import numpy as np
import pytest
import torch

from mla_split_kv_absorbed_amd import _lib as L
from mla_split_kv_absorbed_amd import workloads as W
from mla_split_kv_absorbed_amd.step import DecodeStep
from tests.test_gpu_parity import check_partial, oracle_qlat, say

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_paged32_ragged": (2, dict(B=6, parts=2, lengths=("uniform", 50, 3000)), 0),
    "f16_paged64_loguniform": (4, dict(B=8, lengths=("loguniform", 40, 5000)), 0),
    "bf16_two_queries": (3, dict(B=4, lengths=("uniform", 100, 2500), current=False), 0),
    "bf16_130_heads": (2, dict(B=3, H=130, parts=2, lengths=("uniform", 100, 2000)), 0),
    "bf16_contiguous_k3": (1, dict(B=3, lengths=("fixed", 1500), block_size=0, parts=2), 3),
    "f16_paged64_k1": (4, dict(B=5, lengths=("loguniform", 40, 900)), 1),
    "bf16_no_cut": (2, dict(B=40, parts=2, lengths=("uniform", 60, 200)), 0),
}


def attach_plan(st, w):
    """Builds the history call's plan on the host and hands it over."""
    table, info = L.mla_decode_partial_make_plan(st.hist_args, w.range_start, w.range_end)
    st.plan = torch.from_numpy(table).to(st.dev)
    st.hist_args.plan = st.plan.data_ptr()
    st.hist_args.plan_chunks = info.chunks
    st.hist_args.plan_split_units = info.split_ranges
    return info


def run(w, qs, k, plan, noalloc=False):
    st = DecodeStep(w, q_lat_in=qs, num_splits=k, auto_plan=k == 0)
    info = attach_plan(st, w) if plan else None
    st.parts_out.fill_(float("nan"))
    st.parts_lse.fill_(float("nan"))
    if noalloc:
        L.mla_decode_partial_noalloc(st.hist_args)
    else:
        L.mla_decode_partial(st.hist_args)
    torch.cuda.synchronize()
    return st, info


@pytest.mark.parametrize("name", sorted(CASES))
def test_host_plan_matches_device_plan(name):
    wid, over, k = CASES[name]
    sp = W.spec(wid, **over)
    say(f"[host plan] {name}")
    w = W.make_workload(sp)
    qs = oracle_qlat(w)
    dev, _ = run(w, qs, k, plan=False)
    host, info = run(w, qs, k, plan=True)
    if name == "bf16_no_cut":
        assert info.split_ranges == 0
    assert torch.equal(host.parts_out, dev.parts_out)
    assert torch.equal(host.parts_lse, dev.parts_lse)
    assert not torch.isnan(host.parts_lse).any()


def test_host_plan_noalloc_and_oracle():
    """The allocation-free entry point with a host plan, against the oracle."""
    sp = W.spec(4, B=6, lengths=("loguniform", 40, 3000))
    w = W.make_workload(sp)
    qs = oracle_qlat(w)
    st, info = run(w, qs, 0, plan=True, noalloc=True)
    assert info.split_ranges > 0
    check_partial(w, st, qs)


def test_step_with_host_plan():
    """DecodeStep(host_plan=True) on a ragged batch: the plan is used (the
    history call plans automatically) and the step equals the default one."""
    sp = W.spec(4, B=6, lengths=("loguniform", 60, 2500))
    w = W.make_workload(sp)
    a = DecodeStep(w, host_plan=True)
    b = DecodeStep(w)
    assert a.plan is not None and b.plan is None
    a.run()
    b.run()
    torch.cuda.synchronize()
    assert torch.equal(a.out, b.out)
