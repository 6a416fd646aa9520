"""The fp32 normwise gate of the GPU parity tests against the rounding of
plain fp32 arithmetic (CPU only).

A plain fp32 evaluation of the decode step (q absorption, scores over the
576 latent and rotary dimensions, max-subtracted softmax over the visible
keys, weighted latent sum, V-up), with every product rounded to fp32 and
every sum taken sequentially in fp32, is compared with the float64 oracle on
the sweep's fp32 shapes (without a current chunk) with the largest such
error. The GPU path's error must stay within the gate, so the gate must leave
room above what correct fp32 arithmetic gives: at least three times the
plain evaluation's error."""
import numpy as np
import pytest

import oracle.mla_oracle as mo
from mla_split_kv_absorbed_amd import workloads as W
from tests.test_gpu_parity import REL_GATE
from tests.test_gpu_sweep import draw_case


def seq_dot(a, b):
    """Sum over the last axis of a * b, products and running sum in fp32."""
    p = (a.astype(np.float32) * b.astype(np.float32)).astype(np.float32)
    return np.cumsum(p, axis=-1, dtype=np.float32)[..., -1]


def plain_f32_step(w, heads):
    sp = w.spec
    f = np.float32
    qn, qr = w.f64("q_nope"), w.f64("q_rope")
    wuk, wuv = w.f64("w_uk"), w.f64("w_uv")
    out = np.zeros((sp.B * sp.S, sp.H, 128))
    for b in range(sp.B):
        rows = w.seq_rows64(b).astype(f)  # [L][576], the stored values
        for s in range(sp.S):
            t = b * sp.S + s
            for h in heads:
                ql = seq_dot(wuk[h], qn[t, h][None, :])  # [512]
                sc = seq_dot(rows[:, :512], ql[None, :]) + seq_dot(rows[:, 512:], qr[t, h][None, :])
                sc = (sc.astype(f) * f(sp.scale)).astype(f)
                p = np.exp(sc - sc.max()).astype(f)
                o = np.cumsum(p[:, None] * rows[:, :512], axis=0, dtype=f)[-1] / np.cumsum(p, dtype=f)[-1]
                out[t, h] = seq_dot(o[None, :].astype(f), wuv[h].astype(f).T)  # [128]
    return out


@pytest.mark.parametrize("case", [4, 49, 124])
def test_f32_gate_above_plain_fp32_rounding(case):
    over, _ = draw_case(case)
    assert over["dtype"] == "f32" and not over["current"]
    sp = W.spec(0, **over)
    w = W.make_workload(sp)
    heads = sorted(set(list(range(0, sp.H, max(1, sp.H // 6))) + [sp.H - 1]))
    ref, _ = mo.mla_decode_step(w.f64("q_nope"), w.f64("q_rope"), w.seq_rows64, w.f64("w_uk"),
                                w.f64("w_uv"), sp.scale, sp.S, seqs=list(range(sp.B)), heads=heads)
    got = plain_f32_step(w, heads)
    r = list(range(sp.B * sp.S))
    rel = np.linalg.norm(got[r][:, heads] - ref[r][:, heads]) / np.linalg.norm(ref[r][:, heads])
    assert 0 < rel and 3 * rel <= REL_GATE["f32"], rel
