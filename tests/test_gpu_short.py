"""GPU parity of the short-range partial kernel against the float64 oracle.

A bf16 / fp16 partial call over a contiguous cache whose per-sequence stride
is at most 8 keys (the MTP current chunk of the study page: q_len queries
over the chunk's own q_len keys) runs on a vector kernel (one wave per
(part, query) and 4 heads) instead of the matrix kernel. Every row is
checked: random sub-ranges of the stride (empty, partial and full), both
masks, head counts that are multiples neither of 128 nor of 4, fp32 and
16-bit output / LSE storage, invalid ranges (NaN rows, nothing read),
NaN-poisoned positions outside every range, and scores far from zero in
fp16. Tolerances as in test_gpu_parity:
outputs 1e-2, LSE 1e-3, plus half an ulp of a 16-bit storage type."""
import numpy as np
import pytest
import torch

import oracle.mla_oracle as mo
from mla_split_kv_absorbed_amd import _lib as L
from mla_split_kv_absorbed_amd import workloads as W
from mla_split_kv_absorbed_amd.step import TORCH_DT, to_device
from tests.test_gpu_parity import TOL, f64, half_ulp, say

pytestmark = pytest.mark.gpu


def make_inputs(seed, dtype, B, S, H, K, q_std=0.5):
    rng = np.random.Generator(np.random.PCG64(seed))
    ql = W.draw_rounded(rng, (B * S, H, 512), q_std, dtype)
    qr = W.draw_rounded(rng, (B * S, H, 64), q_std, dtype)
    kv = W.draw_rounded(rng, (B, K, 576), 1.0, dtype)
    return rng, ql, qr, kv


def run_short(dtype, ql, qr, kv, rs, re_, B, S, H, mask, out_dt="same", lse_dt="f32",
              poison=True):
    """One partial call through the C ABI; positions outside every range are
    NaN-poisoned first (so a read of them shows up as NaN)."""
    dev = "cuda"
    K = kv.shape[1]
    kv_dev = kv.copy()
    if poison:
        used = np.zeros((B, K), bool)
        for p in range(rs.shape[0]):
            for b in range(B):
                s0, e0 = int(rs[p, b]), int(re_[p, b])
                if 0 <= s0 <= e0 <= K:
                    used[b, s0:e0] = True
        kv_dev[~used] = W.nan_storage(dtype)
    P, T = rs.shape[0], B * S
    odt = TORCH_DT[dtype if out_dt == "same" else out_dt]
    out = torch.full((P, T, H, 512), 7.0, dtype=odt, device=dev)
    lse = torch.full((P, T, H), 7.0, dtype=TORCH_DT[lse_dt], device=dev)
    qld, qrd, kvd = (to_device(x, dtype, dev) for x in (ql, qr, kv_dev))
    rsd = torch.from_numpy(np.ascontiguousarray(rs, np.int32)).to(dev)
    red = torch.from_numpy(np.ascontiguousarray(re_, np.int32)).to(dev)
    a = L.partial_args(qld, qrd, kvd, rsd, red, out, lse, B=B, S=S, H=H, kv_seq_stride=K,
                       mask=mask, scale=1.0 / np.sqrt(192.0))
    info = L.mla_decode_partial_plan(a, rs, re_)
    assert info.matrix_path == 2
    assert L.mla_decode_partial_workspace_size(a) == 0
    L.mla_decode_partial(a)
    torch.cuda.synchronize()
    return f64(out), f64(lse), a.scale


def check_rows(dtype, ql, qr, kv, rs, re_, B, S, H, mask, go, gl, scale, out_dt, lse_dt):
    qlf, qrf, kvf = (W.from_storage(x, dtype) for x in (ql, qr, kv))
    otol, ltol = TOL[dtype]
    od = dtype if out_dt == "same" else out_dt
    K = kv.shape[1]
    for p in range(rs.shape[0]):
        for b in range(B):
            s0, e0 = int(rs[p, b]), int(re_[p, b])
            sl = slice(b * S, (b + 1) * S)
            g_o, g_l = go[p, sl], gl[p, sl]
            if s0 < 0 or e0 < s0 or e0 > K:
                assert np.all(np.isnan(g_o)) and np.all(np.isnan(g_l)), (p, b)
                continue
            o, l = mo.latent_partial(qlf[sl], qrf[sl], kvf[b], s0, e0, scale,
                                     causal=mask == L.MLA_MASK_CAUSAL_WINDOW)
            empty = ~np.isfinite(l)
            assert np.all(g_l[empty] == -np.inf) and np.all(g_o[empty] == 0), (p, b)
            fin = ~empty
            assert np.all(np.isfinite(g_o[fin])) and np.all(np.isfinite(g_l[fin]))
            err = (np.abs(g_o - o) - half_ulp(o, od))[fin]
            assert err.size == 0 or err.max() <= otol, (p, b, err.max())
            assert np.all(np.abs(g_l[fin] - l[fin]) <= ltol + half_ulp(l[fin], lse_dt)), (p, b)


CASES = [
    # dtype, S, H, K, mask, out dtype, lse dtype
    ("bf16", 2, 128, 2, L.MLA_MASK_CAUSAL_WINDOW, "same", "f32"),
    ("bf16", 2, 128, 2, L.MLA_MASK_CAUSAL_WINDOW, "same", "bf16"),
    ("f16", 2, 128, 2, L.MLA_MASK_CAUSAL_WINDOW, "same", "f16"),
    ("bf16", 5, 16, 5, L.MLA_MASK_CAUSAL_WINDOW, "f32", "f32"),
    ("f16", 8, 202, 8, L.MLA_MASK_CAUSAL_WINDOW, "same", "f32"),
    ("bf16", 1, 6, 8, L.MLA_MASK_NONE, "same", "f32"),
    ("f16", 3, 128, 7, L.MLA_MASK_NONE, "f32", "f16"),
    ("bf16", 8, 128, 1, L.MLA_MASK_CAUSAL_WINDOW, "bf16", "f32"),
]


@pytest.mark.parametrize("case", CASES,
                         ids=lambda c: f"{c[0]}_S{c[1]}_H{c[2]}_K{c[3]}_m{c[4]}_{c[5]}_{c[6]}")
def test_short_ranges(case):
    dtype, S, H, K, mask, out_dt, lse_dt = case
    B, P = 5, 3
    say(f"[short] {case}")
    rng, ql, qr, kv = make_inputs(11 + S * 7 + K, dtype, B, S, H, K)
    # part 0: the whole stride (the current chunk), part 1: random
    # sub-ranges (some empty), part 2: prefixes of random length
    rs = np.zeros((P, B), np.int32)
    re_ = np.zeros((P, B), np.int32)
    re_[0] = K
    a = rng.integers(0, K + 1, size=B)
    c = rng.integers(0, K + 1, size=B)
    rs[1], re_[1] = np.minimum(a, c), np.maximum(a, c)
    re_[2] = rng.integers(0, K + 1, size=B)
    go, gl, scale = run_short(dtype, ql, qr, kv, rs, re_, B, S, H, mask, out_dt, lse_dt)
    check_rows(dtype, ql, qr, kv, rs, re_, B, S, H, mask, go, gl, scale, out_dt, lse_dt)


def test_short_invalid_ranges_are_contained():
    """Ranges that start below 0, end before they start or end past the
    stride give NaN rows; the valid rows of the same call stay exact."""
    dtype, B, S, H, K = "bf16", 6, 2, 128, 4
    rng, ql, qr, kv = make_inputs(5, dtype, B, S, H, K)
    rs = np.array([[0, -1, 3, 0, 2, 1]], np.int32)
    re_ = np.array([[4, 2, 2, 5, 4, 1]], np.int32)
    go, gl, scale = run_short(dtype, ql, qr, kv, rs, re_, B, S, H, L.MLA_MASK_CAUSAL_WINDOW)
    check_rows(dtype, ql, qr, kv, rs, re_, B, S, H, L.MLA_MASK_CAUSAL_WINDOW, go, gl, scale,
               "same", "f32")
    assert np.all(np.isnan(go[0, 2:4])) and np.all(np.isfinite(go[0, 0:2]))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shift", [40.0, -20.0, 12.0])
def test_short_extreme_scores(dtype, shift):
    """Key 0 of every sequence is a multiple of head 0's query, so that head's
    score sits near `shift` (natural units) while the others stay near 0: the
    fp32 online softmax keeps every result finite and exact."""
    B, S, H, K = 3, 2, 128, 2
    rng, ql, qr, kv = make_inputs(23, dtype, B, S, H, K, q_std=0.05)
    qlf, qrf = W.from_storage(ql, dtype), W.from_storage(qr, dtype)
    scale = 1.0 / np.sqrt(192.0)
    kvf = W.from_storage(kv, dtype)
    for b in range(B):
        q0 = np.concatenate([qlf[b * S, 0], qrf[b * S, 0]])
        kvf[b, 0] = q0 * (shift / (scale * float(q0 @ q0)))
    kv = W.to_storage(W.round_to(kvf, dtype), dtype)
    rs = np.zeros((1, B), np.int32)
    re_ = np.full((1, B), K, np.int32)
    go, gl, sc = run_short(dtype, ql, qr, kv, rs, re_, B, S, H, L.MLA_MASK_CAUSAL_WINDOW)
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    check_rows(dtype, ql, qr, kv, rs, re_, B, S, H, L.MLA_MASK_CAUSAL_WINDOW, go, gl, sc,
               "same", "f32")
