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
