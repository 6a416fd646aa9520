"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
the same seeded inputs.

Tolerances (max abs error):
  bf16 / fp16 workloads: outputs <= 1e-2, LSE <= 1e-3; where a workload stores
  the per-part LSE in a 16-bit type, the merged LSE may additionally carry that
  storage rounding (half an ulp of the stored value), and a second run with
  fp32 part LSEs must meet 1e-3 outright. A part's latent output checked on
  its own may likewise carry the rounding to its storage type.
  fp32 workload: outputs and LSE <= 1e-5.
Every oracle comparison of outputs also gates the normwise relative error
||gpu - oracle||_2 / ||oracle||_2 over the checked rows: bf16 <= 1e-2, fp16
<= 5e-3, fp32 <= 1e-6.
"""
import math

import numpy as np
import pytest
import torch

import bench

import oracle.mla_oracle as mo
from mla_split_kv_absorbed_amd import _lib as L
from mla_split_kv_absorbed_amd import workloads as W
from mla_split_kv_absorbed_amd.step import DecodeStep, to_device

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "bf16": (1e-2, 1e-3), "f16": (1e-2, 1e-3)}
# normwise relative error of the outputs, ||gpu - oracle||_2 / ||oracle||_2 over
# the checked rows: the absolute 1e-2 alone is a quarter of the outputs' RMS
# at long contexts, so this second gate catches a wrong result that stays
# small in absolute terms. The fp32 gate is four times the largest error of a
# plain fp32 evaluation of the step (every sum sequential, no fused multiply-add)
# over the sweep's fp32 shapes, 1.3e-6 at 128 heads (tests/test_f32_gate.py):
# a gate below that would fail correct fp32 arithmetic
REL_GATE = {"f32": 5e-6, "bf16": 1e-2, "f16": 5e-3}


def half_ulp(v, dtype):
    """Half an ulp of `dtype` at |v| (0 for fp32 storage)."""
    if dtype == "f32":
        return np.zeros_like(v)
    bits = 8 if dtype == "bf16" else 11
    e = np.floor(np.log2(np.maximum(np.abs(v), 1e-30)))
    return np.exp2(e - bits)


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------
# full decode step
# ---------------------------------------------------------------------------

SMALL = {
    "cfg0": (0, {}),
    "cfg1_small": (1, dict(B=4, lengths=("fixed", 1000))),
    "cfg2_small": (2, dict(B=3, lengths=("fixed", 4000))),
    "cfg3_small": (3, dict(B=4, lengths=("uniform", 100, 1500))),
    "cfg4_small": (4, dict(B=6, lengths=("loguniform", 60, 2000))),
}


def oracle_step(w, seqs, heads):
    sp = w.spec
    cur = (lambda b: w.cur_rows64(b)) if sp.current else None
    return mo.mla_decode_step(w.f64("q_nope"), w.f64("q_rope"), w.seq_rows64, w.f64("w_uk"),
                              w.f64("w_uv"), sp.scale, sp.S, cur_rows=cur, seqs=seqs,
                              heads=heads)


def check_step(w, st, seqs, heads, lse_tol_extra_dtype=None):
    sp = w.spec
    ref_o, ref_l = oracle_step(w, seqs, heads)
    out = f64(st.out)
    lse = f64(st.final_lse())
    otol, ltol = TOL[sp.dtype]
    rows = [b * sp.S + s for b in seqs for s in range(sp.S)]
    err_o = np.abs(out[rows][:, heads] - ref_o[rows][:, heads]).max()
    d_l = np.abs(lse[rows][:, heads] - ref_l[rows][:, heads])
    allow = ltol + (half_ulp(ref_l[rows][:, heads], lse_tol_extra_dtype)
                    if lse_tol_extra_dtype else 0.0)
    ref = ref_o[rows][:, heads]
    rel = float(np.linalg.norm(out[rows][:, heads] - ref) / max(np.linalg.norm(ref), 1e-300))
    say(f"  {sp.name}: max|dout|={err_o:.3e} max|dlse|={d_l.max():.3e} rel={rel:.3e}")
    assert np.all(np.isfinite(out[rows][:, heads]))
    assert rel <= REL_GATE[sp.dtype], rel
    assert err_o <= otol
    assert np.all(d_l <= allow)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_step_small(name):
    wid, over = SMALL[name]
    sp = W.spec(wid, **over)
    say(f"[step] {name} {sp}")
    w = W.make_workload(sp)
    st = DecodeStep(w)
    st.run()
    torch.cuda.synchronize()
    heads = list(range(sp.H)) if sp.H <= 16 else list(range(0, sp.H, 9))
    extra = sp.part_lse_dtype if sp.part_lse_dtype != "f32" else None
    check_step(w, st, list(range(sp.B)), heads, extra)
    if extra:
        st32 = DecodeStep(w, part_lse_dtype="f32")
        st32.run()
        torch.cuda.synchronize()
        check_step(w, st32, list(range(sp.B)), heads)


def test_step_host_subranges():
    """A single part cut into sub-ranges on the host and passed as parts
    (merged by the fused combine + V-up) matches the oracle, ragged last tile
    included, and the step built the default way."""
    sp = W.spec(1, B=4, lengths=("fixed", 1000))
    w = W.make_workload(sp)
    st = DecodeStep(w, host_subranges=True)
    assert st.host_cut == 8 and st.P == 8 and st.fused_tail
    st.run()
    ref = DecodeStep(w)
    ref.run()
    torch.cuda.synchronize()
    check_step(w, st, list(range(sp.B)), list(range(0, sp.H, 9)))
    otol, _ = TOL[sp.dtype]
    assert (st.out.float() - ref.out.float()).abs().max().item() <= otol


FULL = [1, 2, 3, 4]


@pytest.mark.parametrize("wid", FULL)
def test_step_full_size_sampled(wid):
    """The full workload in the benchmark's launch configuration; the oracle
    computes a sample of (sequence, head) outputs one by one (4 sequences x
    4 heads: each pair materialises that head's keys and values over the
    whole sequence). Where the workload stores part LSEs in 16 bits, the
    same step with fp32 part LSEs must also meet 1e-3 outright."""
    sp = W.SPECS[wid]
    say(f"[full] {sp.name}: generating")
    w = W.make_workload(sp)
    st = DecodeStep(w, **bench.BENCH_STEP_OPTS)
    say(f"[full] {sp.name}: running (host sub-ranges: {st.host_cut})")
    st.run()
    torch.cuda.synchronize()
    r = np.random.Generator(np.random.PCG64(7 + wid))
    seqs = sorted(r.choice(sp.B, size=4, replace=False).tolist())
    heads = sorted(r.choice(sp.H, size=4, replace=False).tolist())
    extra = sp.part_lse_dtype if sp.part_lse_dtype != "f32" else None
    check_step(w, st, seqs, heads, extra)
    # every output finite
    assert torch.isfinite(st.out).all().item()
    if extra:
        del st
        st32 = DecodeStep(w, part_lse_dtype="f32", **bench.BENCH_STEP_OPTS)
        st32.run()
        torch.cuda.synchronize()
        check_step(w, st32, seqs, heads)


# ---------------------------------------------------------------------------
# the partial-attention entry point in isolation
# ---------------------------------------------------------------------------

def oracle_qlat(w):
    """q_lat = W_UK q_nope from the oracle, rounded to the storage dtype
    (an input for both sides, never a GPU value)."""
    ql = mo.q_absorb(w.f64("q_nope"), w.f64("w_uk"))
    return W.to_storage(W.round_to(ql, w.spec.dtype), w.spec.dtype)


def run_partial(w, q_lat_store, flags=0, num_splits=0, part_lse_dtype=None, ranges=None,
                block_table=None):
    # num_splits 0: the in-kernel automatic plan, also for equal ranges
    st = DecodeStep(w, flags=flags, num_splits=num_splits, part_lse_dtype=part_lse_dtype,
                    q_lat_in=q_lat_store, auto_plan=num_splits == 0)
    if ranges is not None:
        st.range_start.copy_(torch.from_numpy(ranges[0]))
        st.range_end.copy_(torch.from_numpy(ranges[1]))
    if block_table is not None:
        st.block_table.copy_(torch.from_numpy(block_table))
    L.mla_decode_partial(st.hist_args)
    torch.cuda.synchronize()
    return st


def check_partial(w, st, q_lat_store, seqs=None, heads=None, ranges=None):
    sp = w.spec
    ql = W.from_storage(q_lat_store, sp.dtype)
    qr = w.f64("q_rope")
    rs, re = ranges if ranges is not None else (w.range_start, w.range_end)
    out = f64(st.parts_out)
    lse = f64(st.parts_lse)
    otol, ltol = TOL[sp.dtype]
    lsed = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[st.parts_lse.dtype]
    seqs = range(sp.B) if seqs is None else seqs
    worst_o = worst_l = worst_rel = 0.0
    for b in seqs:
        rows = w.seq_rows64(b)
        sl = slice(b * sp.S, (b + 1) * sp.S)
        for p in range(sp.parts):
            o, l = mo.latent_partial(ql[sl], qr[sl], rows, int(rs[p, b]), int(re[p, b]), sp.scale)
            hh = slice(None) if heads is None else heads
            go, gl = out[p, sl][:, hh], lse[p, sl][:, hh]
            o, l = o[:, hh], l[:, hh]
            empty = ~np.isfinite(l)
            assert np.all(gl[empty] == -np.inf) and np.all(go[empty] == 0)
            fin = ~empty
            if fin.any():
                # the partial output is stored in its own dtype: allow that rounding
                odt = {torch.bfloat16: "bf16", torch.float16: "f16",
                       torch.float32: "f32"}[st.parts_out.dtype]
                excess = np.abs(go - o) - half_ulp(o, odt)
                worst_o = max(worst_o, excess[fin].max())
                nref = np.linalg.norm(o[fin])
                if nref > 0:
                    worst_rel = max(worst_rel, float(np.linalg.norm((go - o)[fin]) / nref))
                dl = np.abs(gl - l)[fin]
                allow = ltol + half_ulp(l[fin], lsed)
                assert np.all(dl <= allow), (p, b, dl.max())
                worst_l = max(worst_l, dl.max())
    say(f"  partial {sp.name}: max|dout|={worst_o:.3e} max|dlse|={worst_l:.3e} "
        f"rel={worst_rel:.3e}")
    assert worst_o <= otol
    assert worst_rel <= REL_GATE[sp.dtype], worst_rel


PARTIAL_CASES = {
    "bf16_paged32_ragged_mfma": (2, dict(B=3, lengths=("fixed", 2000)), 0),
    "bf16_paged32_ragged_simple": (2, dict(B=2, lengths=("fixed", 700)), L.MLA_FLAG_FORCE_SIMPLE),
    "f16_paged64_ragged_mfma": (4, dict(B=5, lengths=("loguniform", 40, 1500)), 0),
    "f16_paged64_simple": (4, dict(B=3, lengths=("loguniform", 40, 600)), L.MLA_FLAG_FORCE_SIMPLE),
    "bf16_contiguous_mfma": (1, dict(B=2, lengths=("fixed", 777), block_size=0, parts=3), 0),
    "f32_contiguous_simple": (0, dict(B=2, lengths=("fixed", 300), parts=3), 0),
}


@pytest.mark.parametrize("name", sorted(PARTIAL_CASES))
def test_partial(name):
    wid, over, flags = PARTIAL_CASES[name]
    sp = W.spec(wid, **over)
    say(f"[partial] {name}")
    w = W.make_workload(sp)
    qs = oracle_qlat(w)
    st = run_partial(w, qs, flags=flags)
    check_partial(w, st, qs)


@pytest.mark.parametrize("splits", [1, 2, 5, 0])
def test_partial_split_count_invariance(splits):
    """Cutting each range into sub-ranges merged inside the call gives the
    same result within tolerance."""
    sp = W.spec(1, B=2, lengths=("fixed", 1500))
    w = W.make_workload(sp)
    qs = oracle_qlat(w)
    st = run_partial(w, qs, num_splits=splits)
    check_partial(w, st, qs)


@pytest.mark.parametrize("B,lengths,splits", [
    (8, ("fixed", 700), 3),           # 22 tiles per range, uneven pieces
    (8, ("uniform", 40, 2000), 8),    # ragged: some ranges shorter than 8 tiles
    (16, ("uniform", 100, 1200), 5),  # two ranges per XCD residue
])
def test_partial_split_xcd_grouped(B, lengths, splits):
    """With an explicit split count and a range count that is a multiple of
    8, the pieces of a range run on one XCD (a different chunk order); the
    merged result still matches the oracle, empty pieces included."""
    sp = W.spec(1, B=B, lengths=lengths)
    say(f"[xcd-grouped] B={B} lengths={lengths} splits={splits}")
    w = W.make_workload(sp)
    assert (sp.parts * B) % 8 == 0
    qs = oracle_qlat(w)
    st = run_partial(w, qs, num_splits=splits)
    check_partial(w, st, qs)


@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_partial_full_size_every_row(wid):
    """Every (part, query, head) row of a full-size workload, in the launch
    the decode step makes, against the oracle's latent partial (all rows:
    the latent partial needs no per-head keys, so the oracle covers the
    whole launch in seconds). Outputs are first poisoned with NaN, so a
    chunk lost or computed twice by the in-kernel plan would show.
    Workloads 1, 3 and 4 cut their ranges into sub-ranges (one part of 32
    sequences, ragged lengths); workload 2 is the benchmark's own launch
    (8 parts x 32 sequences, no sub-ranges)."""
    sp = W.SPECS[wid]
    say(f"[every-row] {sp.name}")
    w = W.make_workload(sp)
    qs = oracle_qlat(w)
    st = DecodeStep(w, q_lat_in=qs)
    st.parts_out.fill_(float("nan"))
    st.parts_lse.fill_(float("nan"))
    L.mla_decode_partial(st.hist_args)
    torch.cuda.synchronize()
    assert torch.isfinite(st.parts_out).all().item()
    assert not torch.isnan(st.parts_lse).any().item()
    check_partial(w, st, qs)


# (flags, num_splits): the matrix kernel with its in-kernel plan (0) and with
# explicit split counts (1, 3: the closed-form chunks), and the plain kernel
EDGE_PATHS = [(0, 0), (0, 1), (0, 3), (L.MLA_FLAG_FORCE_SIMPLE, 0)]


@pytest.mark.parametrize("flags,splits", EDGE_PATHS)
def test_partial_edge_ranges(flags, splits):
    """Empty ranges, single-key ranges, ranges starting mid-block, a zero
    length sequence and unaligned starts."""
    sp = W.spec(2, B=4, lengths=("fixed", 300), parts=4)
    w = W.make_workload(sp)
    qs = oracle_qlat(w)
    rs = np.array([[0, 5, 0, 299], [0, 37, 1, 299], [10, 37, 1, 299], [10, 300, 2, 300]],
                  dtype=np.int32)
    re = np.array([[0, 37, 1, 299], [10, 37, 1, 300], [10, 300, 2, 300], [300, 300, 300, 300]],
                  dtype=np.int32)
    st = run_partial(w, qs, flags=flags, num_splits=splits, ranges=(rs, re))
    check_partial(w, st, qs, ranges=(rs, re))


@pytest.mark.parametrize("bs", [16, 48, 32, 64, 0])
@pytest.mark.parametrize("dtype,splits", [("bf16", 0), ("f16", 3), ("bf16", 1)])
def test_partial_block_sizes_unaligned_starts(bs, dtype, splits):
    """Paged caches of 32- and 64-row blocks and a contiguous cache on the
    matrix kernel, 16- and 48-row blocks on the plain kernel (a 32-key tile
    would span two blocks), with seeded random ranges whose starts fall
    anywhere inside a block, some ending inside the first tile. Outputs
    poisoned with NaN first; every row against the oracle."""
    wid = 2 if dtype == "bf16" else 4
    sp = W.spec(wid, B=5, lengths=("uniform", 300, 900), parts=3, block_size=bs,
                part_out_dtype=dtype, part_lse_dtype="f32")
    say(f"[block-size {bs}] {dtype} splits={splits}")
    w = W.make_workload(sp)
    r = np.random.Generator(np.random.PCG64(600 + bs))
    rs = np.zeros((sp.parts, sp.B), np.int32)
    re = np.zeros((sp.parts, sp.B), np.int32)
    for b in range(sp.B):
        n = int(w.lengths[b])
        cuts = np.sort(r.integers(0, n + 1, size=2 * sp.parts))
        rs[:, b], re[:, b] = cuts[0::2], cuts[1::2]
    rs[0, 0], re[0, 0] = 17, 29      # inside one tile, after its 16-row boundary
    rs[1, 1], re[1, 1] = 50, 51      # a single key
    qs = oracle_qlat(w)
    info = L.mla_decode_partial_plan(
        DecodeStep(w, q_lat_in=qs).hist_args, rs.reshape(-1), re.reshape(-1))
    assert info.matrix_path == (1 if bs % 32 == 0 else 0)
    st = run_partial(w, qs, num_splits=splits, ranges=(rs, re))
    assert torch.isfinite(st.parts_out).all().item()
    check_partial(w, st, qs, ranges=(rs, re))


@pytest.mark.parametrize("flags,splits", EDGE_PATHS)
def test_partial_invalid_metadata_is_contained(flags, splits):
    """A range past the table or a bad block id poisons only its own
    (part, sequence) with NaN; nothing is read out of bounds."""
    sp = W.spec(2, B=3, lengths=("fixed", 256), parts=2)
    w = W.make_workload(sp)
    qs = oracle_qlat(w)
    rs, re = w.range_start.copy(), w.range_end.copy()
    re[1, 0] = 100000          # beyond the table capacity
    rs[0, 2] = 20
    re[0, 2] = 10              # start > end
    bt = w.block_table.copy()
    bt[1, 1] = 1 << 30         # a referenced block id out of range
    st = run_partial(w, qs, flags=flags, num_splits=splits, ranges=(rs, re), block_table=bt)
    out, lse = f64(st.parts_out), f64(st.parts_lse)
    bad = {(1, 0), (0, 2), (0, 1)}
    for p in range(2):
        for b in range(3):
            if (p, b) in bad:
                assert np.all(np.isnan(out[p, b])) and np.all(np.isnan(lse[p, b])), (p, b)
            else:
                assert np.all(np.isfinite(out[p, b])) and np.all(np.isfinite(lse[p, b]))


def test_partial_deterministic_and_permutation_invariant():
    """Bitwise equal on repeat, and bitwise equal when the physical blocks are
    laid out in a different permutation."""
    sp = W.spec(2, B=2, lengths=("fixed", 1111), parts=3)
    w1 = W.make_workload(sp)
    w2 = W.make_workload(sp, extra_blocks=5)   # other permutation, more blocks
    qs = oracle_qlat(w1)
    a = run_partial(w1, qs)
    b = run_partial(w1, qs)
    c = run_partial(w2, qs)
    assert torch.equal(a.parts_out, b.parts_out) and torch.equal(a.parts_lse, b.parts_lse)
    assert torch.equal(a.parts_out, c.parts_out) and torch.equal(a.parts_lse, c.parts_lse)


def test_partial_causal_window():
    """The MTP current segment: two queries over a contiguous 2-token chunk."""
    sp = W.spec(3, B=3, lengths=("fixed", 64))
    w = W.make_workload(sp)
    qs = oracle_qlat(w)
    st = DecodeStep(w, q_lat_in=qs)
    L.mla_decode_partial(st.cur_args)
    torch.cuda.synchronize()
    ql, qr = W.from_storage(qs, sp.dtype), w.f64("q_rope")
    go, gl = f64(st.cur_out), f64(st.cur_lse)
    for b in range(sp.B):
        sl = slice(b * 2, b * 2 + 2)
        o, l = mo.latent_partial(ql[sl], qr[sl], w.cur_rows64(b), 0, 2, sp.scale, causal=True)
        assert (np.abs(go[sl] - o) - half_ulp(o, "bf16")).max() <= 1e-2
        assert np.abs(gl[sl] - l).max() <= 1e-3


def test_partial_extreme_scores():
    """One part's keys are aligned with the queries so its scores sit far
    above the rest: no overflow, and the merged step still matches."""
    sp = W.spec(1, B=1, lengths=("fixed", 512), parts=1, part_out_dtype="f32")
    w = W.make_workload(sp)
    # tokens 192..223: c_KV = large multiple of head 0's absorbed query
    ql = mo.q_absorb(w.f64("q_nope"), w.f64("w_uk"))
    qv = np.concatenate([ql[0, 0], w.f64("q_rope")[0, 0]])
    vec = W.round_to(qv / np.linalg.norm(qv) * 60.0, "bf16")
    blocks = w.block_table[0, 200 // 32:232 // 32]
    for i, blk in enumerate(blocks):
        w.kv[blk, :, :] = W.to_storage(vec, "bf16")[None, :]
    qs = W.to_storage(W.round_to(ql, "bf16"), "bf16")
    st = run_partial(w, qs)
    check_partial(w, st, qs, heads=[0, 1, 2, 64])


# ---------------------------------------------------------------------------
# combine, V-up and q-absorb in isolation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("pdt,ldt,local", [("bf16", "bf16", False), ("bf16", "f32", True),
                                           ("f16", "f16", False), ("f32", "f32", True)])
def test_combine(pdt, ldt, local):
    r = np.random.Generator(np.random.PCG64(99))
    P, T, H = 5, 7, 16
    outs = r.standard_normal((P, T, H, 512)) * 0.1
    lses = r.uniform(2, 12, size=(P, T, H))
    lses[1, 0, :] = -np.inf                # empty part
    lses[:, 1, 3] = -np.inf                # fully empty row
    outs[1, 0, :] = 0
    outs[:, 1, 3] = 0
    lses[2, 2, :] += 80.0                  # extreme part
    o_s = W.round_to(outs, pdt)
    l_s = np.where(np.isfinite(lses), W.round_to(np.where(np.isfinite(lses), lses, 0), ldt), -np.inf)
    n = P - 1 if local else P
    ref_o, ref_l = mo.lse_combine(o_s, l_s)
    dev = "cuda"
    tp = to_device(W.to_storage(o_s, pdt), pdt, dev)
    tl = to_device(W.to_storage(l_s, ldt), ldt, dev)
    out = torch.empty((T, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    if local:
        L.mla_lse_combine(tp[:n].contiguous(), tl[:n].contiguous(), out, lse,
                          local_out=tp[n].contiguous(), local_lse=tl[n].contiguous())
    else:
        L.mla_lse_combine(tp, tl, out, lse)
    torch.cuda.synchronize()
    go, gl = f64(out), f64(lse)
    fin = np.isfinite(ref_l)
    assert np.all(gl[~fin] == -np.inf) and np.all(go[~fin] == 0)
    assert np.abs(go - ref_o).max() <= 1e-5
    assert np.abs(gl[fin] - ref_l[fin]).max() <= 2e-5 * max(1.0, np.abs(ref_l[fin]).max())


@pytest.mark.parametrize("pdt,ldt,dt,n,local,T,H", [
    ("bf16", "bf16", "bf16", 8, False, 32, 128),   # 8 parts, 16-token blocks
    ("bf16", "f32", "bf16", 4, True, 128, 128),    # parts + current: 16-token blocks, 4 per workgroup
    ("f16", "f16", "f16", 2, False, 37, 16),       # ragged last token block
    ("f32", "f32", "bf16", 0, True, 5, 8),         # a local part alone
    ("f16", "f16", "f16", 2, False, 128, 128),     # 32-token blocks, 2 per workgroup
    ("bf16", "f32", "bf16", 3, False, 200, 128),   # 32-token blocks, 3 per workgroup, ragged
    ("f16", "f32", "f16", 5, True, 100, 128),      # 6 parts, 16-token blocks, 3 per workgroup
    ("f32", "f32", "bf16", 3, False, 70, 128),     # fp32 parts, 32-token blocks
    ("f32", "f16", "f16", 6, True, 90, 128),       # fp32 parts, 16-token blocks, 3 per workgroup
    ("bf16", "bf16", "bf16", 10, False, 40, 64),   # more parts than are loaded ahead
])
def test_combine_vup_fused(pdt, ldt, dt, n, local, T, H):
    """mla_combine_vup equals mla_lse_combine (latent in the compute type)
    followed by mla_vup bit for bit (output, LSE, merged latent), and the
    oracle's combine + V-up within the storage rounding."""
    r = np.random.Generator(np.random.PCG64(123))
    P = n + (1 if local else 0)
    outs = r.standard_normal((P, T, H, 512)) * 0.1
    lses = r.uniform(2, 12, size=(P, T, H))
    lses[0, 0, :] = -np.inf                # empty part
    outs[0, 0, :] = 0
    lses[:, 1, 3] = -np.inf                # fully empty row
    outs[:, 1, 3] = 0
    lses[P - 1, 2, :] += 80.0              # extreme part
    o_s = W.round_to(outs, pdt)
    l_s = np.where(np.isfinite(lses), W.round_to(np.where(np.isfinite(lses), lses, 0), ldt), -np.inf)
    wuv = W.round_to(r.standard_normal((H, 512, 128)) / math.sqrt(512), dt)
    dev = "cuda"
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
    tp = to_device(W.to_storage(o_s, pdt), pdt, dev)
    tl = to_device(W.to_storage(l_s, ldt), ldt, dev)
    tw = to_device(W.to_storage(wuv, dt), dt, dev)
    parts = (tp[:n].contiguous(), tl[:n].contiguous()) if n else (None, None)
    loc = dict(local_out=tp[n].contiguous(), local_lse=tl[n].contiguous()) if local else {}
    # two calls
    lat2 = torch.empty((T, H, 512), dtype=tdt, device=dev)
    lse2 = torch.empty((T, H), dtype=torch.float32, device=dev)
    out2 = torch.empty((T, H, 128), dtype=tdt, device=dev)
    L.mla_lse_combine(parts[0], parts[1], lat2, lse2, **loc)
    L.mla_vup(lat2, tw, out2)
    # fused, poisoned outputs first
    lat = torch.full((T, H, 512), float("nan"), dtype=tdt, device=dev)
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device=dev)
    out = torch.full((T, H, 128), float("nan"), dtype=tdt, device=dev)
    L.mla_combine_vup(parts[0], parts[1], tw, out, lse, lat_out=lat, **loc)
    out_nolat = torch.full((T, H, 128), float("nan"), dtype=tdt, device=dev)
    L.mla_combine_vup(parts[0], parts[1], tw, out_nolat, None, **loc)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(out_nolat, out2)
    assert torch.equal(lat, lat2)
    assert torch.equal(torch.isnan(lse), torch.isnan(lse2)) and not torch.isnan(lse).any()
    assert torch.equal(lse, lse2)
    ref_o, ref_l = mo.lse_combine(o_s, l_s)
    ref = mo.v_up(W.round_to(ref_o, dt), wuv)
    go = f64(out)
    assert np.all(np.abs(go - ref) <= half_ulp(ref, dt) + 1e-3)
    fin = np.isfinite(ref_l)
    assert np.all(f64(lse)[~fin] == -np.inf)
    assert np.abs(f64(lse)[fin] - ref_l[fin]).max() <= 2e-5 * max(1.0, np.abs(ref_l[fin]).max())


def _vup_absorb_shapes():
    """(dt, T, H): the fixed case per type, then seeded random token and
    head counts (token blocks of the matrix kernels cut anywhere, one head,
    more than 128 heads)."""
    cases = [(dt, 37, 24) for dt in ("f32", "bf16", "f16")]
    r = np.random.Generator(np.random.PCG64(77))
    for i in range(18):
        cases.append((("f32", "bf16", "f16")[i % 3], int(r.choice([1, 2, 31, 33, 64, 127, 129, 300])),
                      int(r.choice([1, 7, 16, 128, 130]))))
    return cases


@pytest.mark.parametrize("dt,T,H", _vup_absorb_shapes())
def test_vup_and_absorb(dt, T, H):
    r = np.random.Generator(np.random.PCG64(5 + T * 1000 + H))
    x = W.round_to(r.standard_normal((T, H, 512)) * 0.05, dt)
    wuv = W.round_to(r.standard_normal((H, 512, 128)) / math.sqrt(512), dt)
    qn = W.round_to(r.standard_normal((T, H, 128)), dt)
    wuk = W.round_to(r.standard_normal((H, 512, 128)) / math.sqrt(512), dt)
    dev = "cuda"
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dt]
    out = torch.empty((T, H, 128), dtype=tdt, device=dev)
    ql = torch.empty((T, H, 512), dtype=tdt, device=dev)
    L.mla_vup(to_device(W.to_storage(x, dt), dt, dev), to_device(W.to_storage(wuv, dt), dt, dev),
              out)
    L.mla_q_absorb(to_device(W.to_storage(qn, dt), dt, dev),
                   to_device(W.to_storage(wuk, dt), dt, dev), ql)
    torch.cuda.synchronize()
    for got, ref in ((f64(out), mo.v_up(x, wuv)), (f64(ql), mo.q_absorb(qn, wuk))):
        if dt == "f32":
            assert np.abs(got - ref).max() <= 1e-5
        else:
            # one rounding of the fp32 result to the storage type
            assert np.all(np.abs(got - ref) <= 2 * half_ulp(ref, dt) + 1e-4)


SIDE_CASES = {
    "bf16": dict(),
    "f16": dict(dtype="f16", part_out_dtype="f16", part_lse_dtype="f16"),
    "f32": dict(dtype="f32", part_out_dtype="f32", part_lse_dtype="f32"),
}


@pytest.mark.parametrize("case", ["bf16", "f16", "f32", "bf16_full"])
def test_side_stream_step(case):
    """The current-chunk partial on a side stream (study page: the CURRENT
    attention on its own stream while HISTORY runs; its tests assert the
    order and cover BF16 / FP16 / FP32):
      - the step matches the oracle (all sequences, sampled heads; at full
        size a sample of sequences);
      - it is bit for bit the serial step;
      - the combine starts after the side stream's partial has finished
        (event timestamps; a negative gap would mean the combine read a
        current part that was not yet written);
      - the current part's outputs and q_lat are poisoned with NaN before
        every run, so a stale read would also show in the result."""
    full = case.endswith("_full")
    dt = case.split("_")[0]
    if full:
        sp = W.SPECS[3]
    else:
        sp = W.spec(3, B=6, lengths=("uniform", 100, 1500), **SIDE_CASES[dt])
    say(f"[side] {case}")
    w = W.make_workload(sp)
    ser = DecodeStep(w)
    ser.run()
    side = DecodeStep(w, side_stream=True)
    assert side.side is not None
    torch.cuda.synchronize()
    seqs = list(range(sp.B)) if not full else [0, 17, 40, 63]
    heads = list(range(0, sp.H, 9))
    extra = sp.part_lse_dtype if sp.part_lse_dtype != "f32" else None
    for _ in range(3):
        side.cur_out.fill_(float("nan"))
        side.cur_lse.fill_(float("nan"))
        side.q_lat.fill_(float("nan"))
        marks = {"current_done": torch.cuda.Event(enable_timing=True),
                 "tail_start": torch.cuda.Event(enable_timing=True)}
        side.run(marks=marks)
        torch.cuda.synchronize()
        gap_ms = marks["current_done"].elapsed_time(marks["tail_start"])
        assert gap_ms >= 0.0, gap_ms
        assert torch.equal(side.out, ser.out)
        assert torch.equal(side.final_lse(), ser.final_lse())
    check_step(w, side, seqs, heads, extra)


def draw_combine_case(i):
    r = np.random.Generator(np.random.PCG64(8000 + i))
    dts = ["bf16", "f16", "f32"]
    pdt, ldt = str(r.choice(dts)), str(r.choice(dts))
    dt = ["bf16", "f16"][i % 2]
    P = int(r.choice([1, 2, 3, 5, 8, 9, 12, 33, 64, 65, 80]))
    local = bool(r.random() < 0.4)
    H = int(r.choice([1, 3, 16, 64, 128]))
    T = int(max(1, min(int(r.integers(1, 160)), 120000 // (P * H))))
    return r, pdt, ldt, dt, P, local, T, H


@pytest.mark.parametrize("i", range(32))
def test_combine_vup_random(i):
    """Seeded random merges: 1 to 80 parts (more than the 8 loaded ahead,
    and more than the 64 LSEs one load round covers), a local part or not,
    every storage type of parts and LSEs, 1 to 128 heads, ragged token
    counts; scattered empty parts, fully empty rows and parts 80 above the
    rest. mla_lse_combine against the oracle; mla_combine_vup bit for bit
    equal to mla_lse_combine + mla_vup, and against the oracle's combine and
    V-up within the storage rounding."""
    r, pdt, ldt, dt, P, local, T, H = draw_combine_case(i)
    say(f"[combine-random {i}] P={P} local={local} T={T} H={H} parts {pdt} lse {ldt} out {dt}")
    outs = r.standard_normal((P, T, H, 512)) * 0.1
    lses = r.uniform(-5, 15, size=(P, T, H))
    empty = r.random((P, T, H)) < 0.05
    lses[empty] = -np.inf
    outs[empty] = 0
    if T > 1:
        lses[:, T - 1, 0] = -np.inf        # a fully empty row
        outs[:, T - 1, 0] = 0
    hot = r.random(P) < 0.15
    lses[hot] += 80.0
    o_s = W.round_to(outs, pdt)
    l_s = np.where(np.isfinite(lses), W.round_to(np.where(np.isfinite(lses), lses, 0), ldt), -np.inf)
    wuv = W.round_to(r.standard_normal((H, 512, 128)) / math.sqrt(512), dt)
    n = P - 1 if local else P
    dev = "cuda"
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
    tp = to_device(W.to_storage(o_s, pdt), pdt, dev)
    tl = to_device(W.to_storage(l_s, ldt), ldt, dev)
    tw = to_device(W.to_storage(wuv, dt), dt, dev)
    parts = (tp[:n].contiguous(), tl[:n].contiguous()) if n else (None, None)
    loc = dict(local_out=tp[n].contiguous(), local_lse=tl[n].contiguous()) if local else {}
    ref_o, ref_l = mo.lse_combine(o_s, l_s)
    fin = np.isfinite(ref_l)
    # the combine alone, fp32 output
    c_out = torch.empty((T, H, 512), dtype=torch.float32, device=dev)
    c_lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    L.mla_lse_combine(parts[0], parts[1], c_out, c_lse, **loc)
    # two calls in the compute type, then the fused call
    lat2 = torch.empty((T, H, 512), dtype=tdt, device=dev)
    lse2 = torch.empty((T, H), dtype=torch.float32, device=dev)
    out2 = torch.empty((T, H, 128), dtype=tdt, device=dev)
    L.mla_lse_combine(parts[0], parts[1], lat2, lse2, **loc)
    L.mla_vup(lat2, tw, out2)
    lat = torch.full((T, H, 512), float("nan"), dtype=tdt, device=dev)
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device=dev)
    out = torch.full((T, H, 128), float("nan"), dtype=tdt, device=dev)
    L.mla_combine_vup(parts[0], parts[1], tw, out, lse, lat_out=lat, **loc)
    torch.cuda.synchronize()
    go, gl = f64(c_out), f64(c_lse)
    assert np.all(gl[~fin] == -np.inf) and np.all(go[~fin] == 0)
    assert np.abs(go - ref_o).max() <= 1e-5
    assert np.abs(gl[fin] - ref_l[fin]).max() <= 2e-5 * max(1.0, np.abs(ref_l[fin]).max())
    assert torch.equal(out, out2) and torch.equal(lat, lat2) and torch.equal(lse, lse2)
    ref = mo.v_up(W.round_to(ref_o, dt), wuv)
    assert np.all(np.abs(f64(out) - ref) <= half_ulp(ref, dt) + 1e-3)
