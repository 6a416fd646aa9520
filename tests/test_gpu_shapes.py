"""GPU parity of shapes beyond the five workloads, against the float64
oracle: head counts that are not 128 (the study page's TP8 / DCP8 run gives
each rank 16 of DeepSeek's 128 heads) and multi-token queries whose causal
window spans several 32-key tiles (S up to the entry point's limit of 64).

Head counts run on the matrix-core kernel in groups of 128 heads (a partial
group computes zero-query rows that are never stored); the tests check
every stored row and that nothing is written past H."""
import numpy as np
import pytest
import torch

import oracle.mla_oracle as mo
from mla_split_kv_absorbed_amd import _lib as L
from mla_split_kv_absorbed_amd import workloads as W
from mla_split_kv_absorbed_amd.step import DecodeStep
from tests.test_gpu_parity import (TOL, check_partial, check_step, f64, half_ulp, oracle_qlat,
                                   run_partial, say)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H,dtype", [(16, "bf16"), (16, "f16"), (64, "bf16"), (200, "bf16"),
                                     (256, "f16")])
def test_partial_head_counts(H, dtype):
    """The matrix kernel at H != 128: every part against the oracle, for the
    automatic plan and one explicit split count."""
    wid = 2 if dtype == "bf16" else 4
    sp = W.spec(wid, H=H, B=3, lengths=("uniform", 200, 1400), parts=2)
    say(f"[heads] H={H} {dtype}")
    w = W.make_workload(sp)
    qs = oracle_qlat(w)
    probe = DecodeStep(w, q_lat_in=qs)
    info = L.mla_decode_partial_plan(probe.hist_args, w.range_start, w.range_end)
    assert info.matrix_path == 1
    for splits in (0, 3):
        st = run_partial(w, qs, num_splits=splits)
        check_partial(w, st, qs)


@pytest.mark.parametrize("H", [16, 200])
def test_step_head_counts(H):
    """A whole decode step (absorb, partial, combine + V-up) at H = 16 and
    H = 200 against the oracle's non-absorbed attention."""
    sp = W.spec(2, H=H, B=2, lengths=("fixed", 900), parts=3)
    w = W.make_workload(sp)
    st = DecodeStep(w)
    st.run()
    torch.cuda.synchronize()
    heads = list(range(0, H, max(1, H // 12))) + [H - 1]
    check_step(w, st, list(range(sp.B)), sorted(set(heads)), sp.part_lse_dtype)


def test_partial_heads_not_written_past_h():
    """Rows past H in the output buffers stay untouched (H = 16: the group's
    112 zero-query rows are never stored)."""
    sp = W.spec(2, H=16, B=2, lengths=("fixed", 500), parts=2)
    w = W.make_workload(sp)
    qs = oracle_qlat(w)
    st = DecodeStep(w, q_lat_in=qs)
    P, T = sp.parts, w.T
    big_o = torch.full((P * T * 16 * 512 + 4096,), float("nan"), dtype=torch.bfloat16,
                       device="cuda")
    big_l = torch.full((P * T * 16 + 4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
    st.hist_args.out = big_o.data_ptr()
    st.hist_args.lse = big_l.data_ptr()
    L.mla_decode_partial(st.hist_args)
    torch.cuda.synchronize()
    n_o, n_l = P * T * 16 * 512, P * T * 16
    assert torch.isfinite(big_o[:n_o]).all().item()
    assert torch.isnan(big_o[n_o:]).all().item()
    assert torch.isfinite(big_l[:n_l]).all().item()
    assert torch.isnan(big_l[n_l:]).all().item()


@pytest.mark.parametrize("S", [3, 8, 33, 64])
def test_step_mtp_query_lengths(S):
    """Multi-token decode with S query tokens: history parts plus the S-token
    current chunk under the current-window mask, merged as the local part,
    against the oracle (query s sees the history and current keys 0..s)."""
    B = 2 if S > 8 else 3
    sp = W.spec(3, S=S, B=B, lengths=("uniform", 100, 900))
    say(f"[mtp] S={S}")
    w = W.make_workload(sp)
    st = DecodeStep(w)
    st.run()
    torch.cuda.synchronize()
    check_step(w, st, list(range(sp.B)), list(range(0, sp.H, 13)))


@pytest.mark.parametrize("S,dtype", [(3, "bf16"), (33, "bf16"), (64, "bf16"), (33, "f16")])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_partial_causal_window_long(S, dtype, splits):
    """The current-window mask over whole history ranges: query s of S sees
    the range's keys up to end - S + s, so for S > 32 the masked keys reach
    over more than the last tile (and, cut into pieces, over whole chunks)."""
    wid = 2 if dtype == "bf16" else 4
    sp = W.spec(wid, S=S, B=2, lengths=("uniform", 70, 700), parts=2)
    w = W.make_workload(sp)
    qs = oracle_qlat(w)
    st = DecodeStep(w, q_lat_in=qs, num_splits=splits, auto_plan=True)
    st.hist_args.mask = L.MLA_MASK_CAUSAL_WINDOW
    L.mla_decode_partial(st.hist_args)
    torch.cuda.synchronize()
    ql, qr = W.from_storage(qs, sp.dtype), w.f64("q_rope")
    go, gl = f64(st.parts_out), f64(st.parts_lse)
    otol, ltol = TOL[sp.dtype]
    heads = list(range(0, sp.H, 7))
    for b in range(sp.B):
        sl = slice(b * S, (b + 1) * S)
        rows = w.seq_rows64(b)
        for p in range(sp.parts):
            o, l = mo.latent_partial(ql[sl][:, heads], qr[sl][:, heads], rows,
                                     int(w.range_start[p, b]), int(w.range_end[p, b]), sp.scale,
                                     causal=True)
            g_o, g_l = go[p, sl][:, heads], gl[p, sl][:, heads]
            empty = ~np.isfinite(l)
            assert np.all(g_l[empty] == -np.inf) and np.all(g_o[empty] == 0)
            fin = ~empty
            assert (np.abs(g_o - o) - half_ulp(o, sp.part_out_dtype))[fin].max() <= otol
            assert np.all(np.abs(g_l[fin] - l[fin]) <= ltol + half_ulp(l[fin], sp.part_lse_dtype))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_partial_long_sequence(dtype):
    """One sequence of 256K keys, the longest here: the plan cuts its range
    into 256 pieces (the workspace's largest use at one range), merged inside
    the call; sampled heads of the merged part against the oracle."""
    wid = 2 if dtype == "bf16" else 4
    sp = W.spec(wid, B=1, lengths=("fixed", 262144), parts=1)
    say(f"[long] {dtype} L=262144")
    w = W.make_workload(sp)
    qs = oracle_qlat(w)
    st = DecodeStep(w, q_lat_in=qs)
    assert st.num_splits > 1
    L.mla_decode_partial(st.hist_args)
    torch.cuda.synchronize()
    heads = [0, 45, 127]
    ql, qr = W.from_storage(qs, sp.dtype), w.f64("q_rope")
    o, l = mo.latent_partial(ql[:, heads], qr[:, heads], w.seq_rows64(0),
                             int(w.range_start[0, 0]), int(w.range_end[0, 0]), sp.scale)
    go, gl = f64(st.parts_out)[0][:, heads], f64(st.parts_lse)[0][:, heads]
    otol, ltol = TOL[sp.dtype]
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    assert (np.abs(go - o) - half_ulp(o, sp.part_out_dtype)).max() <= otol
    assert np.all(np.abs(gl - l) <= ltol + half_ulp(l, sp.part_lse_dtype))
