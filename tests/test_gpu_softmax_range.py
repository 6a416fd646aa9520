"""GPU parity at extreme score ranges: the partial kernel's softmax against the
float64 oracle when heads' maxima sit far from 0 and far from each other.

The RTPLLM-on-K3 page makes the online-softmax rescale mandatory (section
4.2) and reports that its missing-rescale bug only showed in a unit test with
extreme values, where one slice's maximum sits far above the others (section
5.2, first pitfall). The kernel takes each head's exponent reference from the
first tile of each chunk and replays a chunk whose later scores rise more
than the weight type allows above it (2^15 for fp16 weights, 2^64 for bf16);
these inputs drive both paths.

Construction (every value is an input, rounded to storage once; the oracle
sees the same rounded values):
  k_R[j][0] = 1 for every key,     q_rope[t][h][0] = shift(h) / scale
  k_R[j][1] = 1 in one part only,  q_rope[t][h][1] = 80 / scale
  k_R[j][2] = 1 on sparse "spike" keys (j % 97 == 50), q_rope[t][h][2] = spike(h) / scale
so every score of head h moves by shift(h) natural units, the keys of one
part by another +80, and the spike keys by spike(h). With the N(0, 1) scores
of the rest, head maxima land near shift + 3: +12, +40, -12, -20 and more.
The spike keys sit inside ranges, so chunks whose first tile holds none of
them meet a later maximum 15 (fp16: above its 2^15 window) or 50 (bf16:
above 2^64) natural units higher and are replayed.
"""
import numpy as np
import pytest
import torch

import oracle.mla_oracle as mo
from mla_split_kv_absorbed_amd import _lib as L
from mla_split_kv_absorbed_amd import workloads as W
from mla_split_kv_absorbed_amd.step import DecodeStep
from tests.test_gpu_parity import TOL, check_partial, f64, half_ulp, oracle_qlat, say

pytestmark = pytest.mark.gpu

# head h: shift SHIFTS[h % 8], spike SPIKES[(h // 8) % 3] (natural units)
SHIFTS = [9.0, 37.0, -15.0, -23.0, 0.0, 20.0, -40.0, 60.0]
SPIKES = [0.0, 15.0, 50.0]
HOT_PART = 1
SPIKE_EVERY, SPIKE_AT = 97, 50


def shape_scores(w):
    """Rewrites the workload's k_R columns 0..2 (valid keys only; the NaN
    poison of unused slots stays) and q_rope columns 0..2 as above."""
    sp = w.spec
    dt = sp.dtype
    one = W.to_storage(np.array([1.0]), dt)[0]
    zero = W.to_storage(np.array([0.0]), dt)[0]
    for b in range(sp.B):
        n = int(w.lengths[b])
        j = np.arange(n)
        hot = (j >= w.range_start[HOT_PART, b]) & (j < w.range_end[HOT_PART, b])
        spike = (j % SPIKE_EVERY) == SPIKE_AT
        if sp.block_size > 0:
            bs = sp.block_size
            blk = w.block_table[b, j // bs]
            slot = j % bs
            w.kv[blk, slot, W.D_C + 0] = one
            w.kv[blk, slot, W.D_C + 1] = np.where(hot, one, zero)
            w.kv[blk, slot, W.D_C + 2] = np.where(spike, one, zero)
        else:
            w.kv[b, :n, W.D_C + 0] = one
            w.kv[b, :n, W.D_C + 1] = np.where(hot, one, zero)
            w.kv[b, :n, W.D_C + 2] = np.where(spike, one, zero)
    qr = W.from_storage(w.q_rope, dt)
    for h in range(sp.H):
        qr[:, h, 0] = SHIFTS[h % 8] / sp.scale
        qr[:, h, 1] = 80.0 / sp.scale
        qr[:, h, 2] = SPIKES[(h // 8) % 3] / sp.scale
    w.q_rope = W.to_storage(W.round_to(qr, dt), dt)


CASES = {
    # fp16, paged 64, ragged lengths: the automatic plan and explicit counts
    "f16_auto": (4, dict(B=5, lengths=("loguniform", 300, 3000)), 0),
    "f16_splits1": (4, dict(B=5, lengths=("loguniform", 300, 3000)), 1),
    "f16_splits3": (4, dict(B=5, lengths=("loguniform", 300, 3000)), 3),
    # bf16, paged 32, 4 parts of equal length
    "bf16_auto": (2, dict(B=3, lengths=("fixed", 2600), parts=4), 0),
    "bf16_splits3": (2, dict(B=3, lengths=("fixed", 2600), parts=4), 3),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_partial_extreme_head_maxima(name):
    wid, over, splits = CASES[name]
    sp = W.spec(wid, **over)
    say(f"[extreme] {name}")
    w = W.make_workload(sp)
    shape_scores(w)
    qs = oracle_qlat(w)
    # splits 0: the in-kernel automatic plan (not the equal-range shortcut)
    st = DecodeStep(w, q_lat_in=qs, num_splits=splits, auto_plan=True)
    L.mla_decode_partial(st.hist_args)
    torch.cuda.synchronize()
    assert torch.isfinite(st.parts_out).all().item()
    assert not torch.isnan(st.parts_lse).any().item()
    # the maxima really are extreme
    ql = W.from_storage(qs, sp.dtype)
    qr = w.f64("q_rope")
    _, l_hot = mo.latent_partial(ql[:1], qr[:1], w.seq_rows64(0),
                                 int(w.range_start[HOT_PART, 0]), int(w.range_end[HOT_PART, 0]),
                                 sp.scale)
    assert l_hot.max() > 150 and l_hot.min() < 60
    check_partial(w, st, qs)
    # the parts merged by LSE equal attention over the whole sequence
    T, H = w.T, sp.H
    out = torch.empty((T, H, W.D_C), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    L.mla_lse_combine(st.parts_out, st.parts_lse, out, lse)
    torch.cuda.synchronize()
    go, gl = f64(out), f64(lse)
    otol, ltol = TOL[sp.dtype]
    lsed = sp.part_lse_dtype
    odt = sp.part_out_dtype
    for b in range(sp.B):
        o, l = mo.latent_partial(ql[b:b + 1], qr[b:b + 1], w.seq_rows64(b), 0,
                                 int(w.lengths[b]), sp.scale)
        err_o = (np.abs(go[b] - o[0]) - half_ulp(o[0], odt)).max()
        err_l = np.abs(gl[b] - l[0])
        assert np.all(np.isfinite(go[b]))
        assert err_o <= otol, (b, err_o)
        assert np.all(err_l <= ltol + half_ulp(l[0], lsed)), (b, err_l.max())


def test_partial_fp16_window_edges():
    """fp16 heads whose second-half keys score 10 or 11.5 natural units
    above the rest, around the edge of the 2^15 weight window over the first
    tile (15 log2 units = 10.4 natural units; the random part moves each
    head's maxima by a unit or two either way): with one chunk per range and
    with the automatic plan's chunks, nothing overflows and every part
    matches the oracle."""
    sp = W.spec(4, B=2, lengths=("fixed", 640), parts=1)
    w = W.make_workload(sp)
    dt = sp.dtype
    one = W.to_storage(np.array([1.0]), dt)[0]
    zero = W.to_storage(np.array([0.0]), dt)[0]
    for b in range(sp.B):
        n = int(w.lengths[b])
        j = np.arange(n)
        blk, slot = w.block_table[b, j // 64], j % 64
        w.kv[blk, slot, W.D_C + 0] = np.where(j >= 320, one, zero)  # second half
        # the rope part carries only the shift
        w.kv[blk, slot, W.D_C + 1:] = zero
    qr = W.from_storage(w.q_rope, dt)
    qr[:, :, 1:] = 0.0
    for h in range(sp.H):
        qr[:, h, 0] = (10.0 if h % 2 == 0 else 11.5) / sp.scale
    w.q_rope = W.to_storage(W.round_to(qr, dt), dt)
    qs = oracle_qlat(w)
    for splits in (1, 0):
        st = DecodeStep(w, q_lat_in=qs, num_splits=splits, auto_plan=True)
        L.mla_decode_partial(st.hist_args)
        torch.cuda.synchronize()
        assert torch.isfinite(st.parts_out).all().item()
        check_partial(w, st, qs)


# ---------------------------------------------------------------------------
# randomized extreme shapes
# ---------------------------------------------------------------------------
# Seeded random cases of the same construction, with more freedom: per-head
# shifts in [-60, 60], a per-head score ramp of up to +-35 natural units from
# the first key of a sequence to its last (a rising ramp keeps lifting the
# maximum past the first tile's reference, the replay's trigger), spikes of
# 0 to 45 units every 20 to 300 keys, a hot part (+30 or +80) or none, fp16
# and bf16, block sizes 16 to 128, 1 to 4 parts, explicit and automatic
# split counts, and 16-bit or fp32 part LSEs. Column 3 of k_R carries the
# ramp j / (n - 1), q_rope[t][h][3] its slope.

def draw_extreme(i):
    r = np.random.Generator(np.random.PCG64(9000 + i))
    dt = ["f16", "bf16"][i % 2]
    wid = 4 if dt == "f16" else 2
    parts = int(r.integers(1, 5))
    lo = int(r.integers(40, 800))
    hi = lo + int(r.integers(0, 3000))
    over = dict(B=int(r.integers(1, 5)), H=int(r.choice([16, 128])), lengths=("uniform", lo, hi),
                block_size=int(r.choice([16, 32, 64, 128])), parts=parts, part_out_dtype=dt,
                part_lse_dtype=str(r.choice(["f32", dt])))
    splits = int(r.choice([0, 0, 1, 2, 3, 5]))
    prm = dict(shift=r.uniform(-60, 60, size=16), slope=r.uniform(-35, 35, size=16),
               spike=r.choice([0.0, 8.0, 12.0, 20.0, 45.0], size=16),
               every=int(r.integers(20, 300)), hot=float(r.choice([0.0, 30.0, 80.0])),
               hotpart=int(r.integers(0, parts)))
    prm["at"] = int(r.integers(0, prm["every"]))
    return wid, over, splits, prm


def shape_random(w, prm):
    sp = w.spec
    dt = sp.dtype
    one = W.to_storage(np.array([1.0]), dt)[0]
    zero = W.to_storage(np.array([0.0]), dt)[0]
    for b in range(sp.B):
        n = int(w.lengths[b])
        j = np.arange(n)
        hot = (j >= w.range_start[prm["hotpart"], b]) & (j < w.range_end[prm["hotpart"], b])
        spike = (j % prm["every"]) == prm["at"]
        ramp = W.to_storage(W.round_to(j / max(n - 1, 1), dt), dt)
        cols = {0: np.full(n, one), 1: np.where(hot, one, zero), 2: np.where(spike, one, zero),
                3: ramp}
        for c, v in cols.items():
            if sp.block_size > 0:
                w.kv[w.block_table[b, j // sp.block_size], j % sp.block_size, W.D_C + c] = v
            else:
                w.kv[b, :n, W.D_C + c] = v
    qr = W.from_storage(w.q_rope, dt)
    for h in range(sp.H):
        qr[:, h, 0] = prm["shift"][h % 16] / sp.scale
        qr[:, h, 1] = prm["hot"] / sp.scale
        qr[:, h, 2] = prm["spike"][h % 16] / sp.scale
        qr[:, h, 3] = prm["slope"][h % 16] / sp.scale
    w.q_rope = W.to_storage(W.round_to(qr, dt), dt)


@pytest.mark.parametrize("i", range(48))
def test_partial_extreme_random(i):
    """Every part against the oracle (outputs poisoned with NaN first), then
    the parts merged by LSE against attention over the whole sequence.
    With fp32 part LSEs (a second run of the same inputs) the merge meets
    the plain tolerances. With 16-bit part LSEs each stored LSE is off by up
    to half an ulp of its type at |LSE| (0.25 natural units for bf16 near
    100) plus the kernel's LSE error d, which moves a normalised merge weight
    by a factor of at most exp(2 d); the merged row then moves by at most
    (exp(2 d) - 1) times the spread of the part rows around it. Both bounds
    come from the oracle's own per-part results."""
    wid, over, splits, prm = draw_extreme(i)
    sp = W.spec(wid, **over)
    say(f"[extreme-random {i}] {over} splits={splits} hot={prm['hot']}")
    w = W.make_workload(sp)
    shape_random(w, prm)
    qs = oracle_qlat(w)
    ql = W.from_storage(qs, sp.dtype)
    qr = w.f64("q_rope")
    otol, ltol = TOL[sp.dtype]
    T, H = w.T, sp.H

    def run(lse_dtype):
        st = DecodeStep(w, q_lat_in=qs, num_splits=splits, auto_plan=True,
                        part_lse_dtype=lse_dtype)
        st.parts_out.fill_(float("nan"))
        L.mla_decode_partial(st.hist_args)
        out = torch.empty((T, H, W.D_C), dtype=torch.float32, device="cuda")
        lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
        L.mla_lse_combine(st.parts_out, st.parts_lse, out, lse)
        torch.cuda.synchronize()
        assert torch.isfinite(st.parts_out).all().item()
        return st, f64(out), f64(lse)

    st, go, gl = run(None)
    check_partial(w, st, qs)
    _, go32, gl32 = run("f32")
    odt = sp.part_out_dtype
    for b in range(sp.B):
        o, l = mo.latent_partial(ql[b:b + 1], qr[b:b + 1], w.seq_rows64(b), 0,
                                 int(w.lengths[b]), sp.scale)
        o, l = o[0], l[0]
        e32 = (np.abs(go32[b] - o) - half_ulp(o, odt)).max()
        assert e32 <= otol, (b, e32)
        assert np.all(np.abs(gl32[b] - l) <= ltol), b
        d = np.zeros_like(l)
        spread = np.zeros_like(l)
        for p in range(sp.parts):
            po, pl = mo.latent_partial(ql[b:b + 1], qr[b:b + 1], w.seq_rows64(b),
                                       int(w.range_start[p, b]), int(w.range_end[p, b]),
                                       sp.scale)
            fin = np.isfinite(pl[0])
            hu = half_ulp(np.where(fin, pl[0], 0.0), sp.part_lse_dtype)
            d = np.maximum(d, np.where(fin, hu + ltol, 0.0))
            spread = np.maximum(spread, np.where(fin, np.abs(po[0] - o).max(axis=-1), 0.0))
        allow = (np.expm1(2 * d) * (spread + otol))[..., None] + otol
        eo = np.abs(go[b] - o) - half_ulp(o, odt)
        assert np.all(np.isfinite(go[b])), b
        assert np.all(eo <= allow), (b, float((eo - allow).max()))
        assert np.all(np.abs(gl[b] - l) <= ltol + d), b
