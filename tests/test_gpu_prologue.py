"""GPU parity of the fused decode prologue (rotary embedding, q absorption,
paged cache append) through the C ABI, against the float64 oracle on the same
seeded inputs, and a decode step that starts from pre-rotation inputs.

Tolerances: the appended latent is a copy (bit exact); rotated values are
computed in fp32 from a double-precision angle and rounded once, so they may
differ from the oracle by half an ulp of the storage type plus fp32 rounding
(2e-6 relative); absorbed queries as in the absorption test (two half-ulps
plus 1e-4); every cache row that is not a valid new token's slot keeps its
bytes.
"""
import numpy as np
import pytest
import torch

import oracle.mla_oracle as mo
from mla_split_kv_absorbed_amd import _lib as L
from mla_split_kv_absorbed_amd import workloads as W
from mla_split_kv_absorbed_amd.step import to_device

pytestmark = pytest.mark.gpu

D_C, D_R, D_N = 512, 64, 128
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
# fp32 rotation of pairs whose values stay below ~4: three roundings of terms
# up to ~8 in magnitude, plus fp32 cos/sin
ROT_TOL = 2e-6


def half_ulp(v, dtype):
    if dtype == "f32":
        bits = 24
    else:
        bits = 8 if dtype == "bf16" else 11
    e = np.floor(np.log2(np.maximum(np.abs(v), 1e-30)))
    return np.exp2(e - bits)


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def make_inputs(seed, dt, B, S, H, paged, bs=32, nblk=6, spare=3, stride=200):
    """Seeded storage-rounded inputs; positions include one invalid token."""
    r = np.random.Generator(np.random.PCG64(seed))
    T = B * S
    g = lambda *shape, sc=1.0: W.round_to(r.standard_normal(shape) * sc, dt)
    inp = dict(q_nope=g(T, H, D_N), q_pe=g(T, H, D_R), w_uk=g(H, D_C, D_N, sc=512 ** -0.5),
               kv_new=g(T, D_C + D_R))
    if paged:
        perm = r.permutation(B * nblk + spare).astype(np.int32)
        inp["block_table"] = perm[:B * nblk].reshape(B, nblk)
        inp["cache"] = g((B * nblk + spare) * bs, D_C + D_R)
        cap = nblk * bs
    else:
        inp["block_table"] = None
        inp["cache"] = g(B * stride, D_C + D_R)
        cap = stride
    # each sequence's new tokens at consecutive positions from a random start
    # (distinct slots, as the prologue requires)
    pos = np.array([int(r.integers(0, cap - S)) + np.arange(S) for b in range(B)],
                   np.int32).reshape(-1)
    pos[1] = cap + 7          # past the capacity: must not be written
    if T > 3:
        pos[3] = -2           # negative: must not be written
    inp["positions"] = pos
    inp.update(B=B, S=S, H=H, bs=bs if paged else 0, stride=0 if paged else stride, cap=cap)
    return inp


def run_gpu(inp, dt):
    dev = torch.device("cuda")
    dtt = TORCH[dt]
    up = lambda x: to_device(W.to_storage(x, dt), dt, dev)
    tens = {k: up(inp[k]) for k in ("q_nope", "q_pe", "w_uk", "kv_new")}
    cache = up(inp["cache"])
    bt = torch.from_numpy(inp["block_table"]).to(dev) if inp["block_table"] is not None else None
    pos = torch.from_numpy(inp["positions"]).to(dev)
    T, H = inp["B"] * inp["S"], inp["H"]
    q_lat = torch.empty((T, H, D_C), dtype=dtt, device=dev)
    q_rope = torch.empty((T, H, D_R), dtype=dtt, device=dev)
    nb = inp["cache"].shape[0] // inp["bs"] if inp["bs"] else 0
    a = L.prologue_args(tens["q_nope"], tens["q_pe"], tens["w_uk"], tens["kv_new"], pos, cache,
                        q_lat, q_rope, B=inp["B"], S=inp["S"], block_table=bt,
                        block_size=inp["bs"], num_blocks=nb, kv_seq_stride=inp["stride"])
    before = cache.clone()
    L.mla_decode_prologue(a)
    torch.cuda.synchronize()
    return q_lat, q_rope, cache, before


def valid(inp, t):
    p = int(inp["positions"][t])
    return 0 <= p < inp["cap"]


@pytest.mark.parametrize("dt,paged,H", [("bf16", True, 128), ("f16", True, 16),
                                        ("bf16", False, 128), ("f32", True, 16),
                                        ("f32", False, 128)])
def test_prologue_matches_oracle(dt, paged, H):
    inp = make_inputs(11, dt, B=5, S=2, H=H, paged=paged)
    q_lat, q_rope, cache, before = run_gpu(inp, dt)
    B, S = inp["B"], inp["S"]
    # oracle on the valid tokens only (invalid ones are not written)
    pos = inp["positions"]
    ok = np.array([valid(inp, t) for t in range(B * S)])
    pos_o = np.where(ok, pos, 0)
    ql, qr, new = mo.decode_prologue(inp["q_nope"], inp["q_pe"], inp["w_uk"], inp["kv_new"],
                                     pos_o, inp["cache"], inp["block_table"], inp["bs"],
                                     inp["stride"], B, S, D_C)
    # q_rope of every token, the invalid ones included, is the rotation at
    # the given position
    qr = mo.rope(inp["q_pe"], pos[:, None].astype(np.int64))
    g_ql, g_qr = f64(q_lat), f64(q_rope)
    tol_q = 2 * half_ulp(ql, dt) + (1e-4 if dt != "f32" else 1e-5)
    assert np.all(np.abs(g_ql - ql) <= tol_q)
    assert np.all(np.abs(g_qr - qr) <= half_ulp(qr, dt) + ROT_TOL * (np.abs(qr) + 1))
    got = f64(cache)
    written = set()
    for t in range(B * S):
        if not ok[t]:
            continue
        row = mo.cache_slot(t // S, int(pos[t]), inp["block_table"], inp["bs"], inp["stride"])
        written.add(row)
        assert np.array_equal(got[row, :D_C], inp["kv_new"][t, :D_C])
        want = mo.rope(inp["kv_new"][t, D_C:], int(pos[t]))
        assert np.all(np.abs(got[row, D_C:] - want) <= half_ulp(want, dt) + ROT_TOL * (np.abs(want) + 1))
    others = np.array([r for r in range(got.shape[0]) if r not in written])
    assert torch.equal(cache[torch.from_numpy(others).cuda()], before[torch.from_numpy(others).cuda()])


def test_prologue_then_attention():
    """A decode step from pre-rotation inputs: the prologue appends the S new
    tokens behind each sequence's history and rotates the query; partial
    attention over [0, L_b + S) with the current-window mask then matches the
    oracle's latent attention over the oracle's updated cache, with the
    oracle's own rotated and absorbed queries (no GPU value enters the
    oracle side)."""
    dt, B, S, H, bs = "bf16", 3, 2, 128, 32
    r = np.random.Generator(np.random.PCG64(21))
    lengths = np.array([700, 1000, 45], np.int32)  # history tokens (last block not full)
    nblk = [int(-(-(L + S) // bs)) for L in lengths]
    maxb = max(nblk)
    perm = r.permutation(sum(nblk) + 2).astype(np.int32)
    bt = np.full((B, maxb), perm[-1], np.int32)  # unused entries: a spare block
    k = 0
    for b in range(B):
        bt[b, :nblk[b]] = perm[k:k + nblk[b]]
        k += nblk[b]
    rows_total = (sum(nblk) + 2) * bs
    g = lambda *shape, sc=1.0: W.round_to(r.standard_normal(shape) * sc, dt)
    cache = g(rows_total, D_C + D_R)
    T = B * S
    q_nope, q_pe = g(T, H, D_N), g(T, H, D_R)
    w_uk = g(H, D_C, D_N, sc=512 ** -0.5)
    kv_new = g(T, D_C + D_R)
    pos = np.array([lengths[b] + s for b in range(B) for s in range(S)], np.int32)
    inp = dict(q_nope=q_nope, q_pe=q_pe, w_uk=w_uk, kv_new=kv_new, cache=cache,
               block_table=bt, positions=pos, B=B, S=S, H=H, bs=bs, stride=0)
    q_lat, q_rope, gcache, _ = run_gpu(inp, dt)
    dev = torch.device("cuda")
    start = torch.zeros((1, B), dtype=torch.int32, device=dev)
    end = torch.from_numpy((lengths + S).astype(np.int32)[None, :]).to(dev)
    out = torch.empty((1, T, H, D_C), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, T, H), dtype=torch.float32, device=dev)
    a = L.partial_args(q_lat, q_rope, gcache, start, end, out, lse, B=B, S=S, H=H,
                       block_table=torch.from_numpy(bt).to(dev), block_size=bs,
                       num_blocks=rows_total // bs, mask=L.MLA_MASK_CAUSAL_WINDOW,
                       scale=192 ** -0.5)
    ws = torch.empty(max(1, L.mla_decode_partial_workspace_size(a)), dtype=torch.uint8,
                     device=dev)
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    L.mla_decode_partial(a)
    torch.cuda.synchronize()
    # oracle: prologue, then latent attention over each sequence's rows
    ql, qr, new = mo.decode_prologue(q_nope, q_pe, w_uk, kv_new, pos, cache, bt, bs, 0, B, S, D_C)
    # the oracle's own queries and appended rows, rounded once to the storage
    # type (the query buffers and the cache hold that type)
    ql, qr, new = W.round_to(ql, dt), W.round_to(qr, dt), W.round_to(new, dt)
    go, gl = f64(out[0]), f64(lse[0])
    heads = list(range(0, H, 11))
    for b in range(B):
        n = int(lengths[b]) + S
        rows = new[[mo.cache_slot(b, j, bt, bs, 0) for j in range(n)]]
        sl = slice(b * S, (b + 1) * S)
        o, l = mo.latent_partial(ql[sl][:, heads], qr[sl][:, heads], rows, 0, n, 192 ** -0.5,
                                 causal=True)
        excess = np.abs(go[sl][:, heads] - o) - half_ulp(o, dt)
        assert excess.max() <= 1e-2, (b, excess.max())
        assert np.abs(gl[sl][:, heads] - l).max() <= 1e-3, b


@pytest.mark.parametrize("i", range(48))
def test_prologue_random_shapes(i):
    """Seeded random shapes of the same check: fp32 / bf16 / fp16, paged
    (block sizes 16-128, 1-39 blocks per sequence) or contiguous (strides to
    5000), 1-6 sequences of 1-4 new tokens, 8-130 heads; positions up to a
    few thousand (the rotation angle is reduced in double precision)."""
    r = np.random.Generator(np.random.PCG64(3000 + i))
    dt = ["bf16", "f16", "f32"][i % 3]
    paged = bool(r.random() < 0.7)
    B, S = int(r.integers(1, 7)), int(r.integers(1, 5))
    if B * S < 2:  # the input builder marks token 1 invalid
        S = 2
    H = int(r.choice([8, 16, 64, 128, 130]))
    bs = int(r.choice([16, 32, 64, 128]))
    nblk = int(r.integers(1, 40))
    stride = int(r.integers(S + 8, 5000))
    if paged and nblk * bs < S + 8:
        nblk = (S + 8) // bs + 1
    inp = make_inputs(4000 + i, dt, B=B, S=S, H=H, paged=paged, bs=bs, nblk=nblk, stride=stride)
    q_lat, q_rope, cache, before = run_gpu(inp, dt)
    pos = inp["positions"]
    ok = np.array([valid(inp, t) for t in range(B * S)])
    ql, _, _ = mo.decode_prologue(inp["q_nope"], inp["q_pe"], inp["w_uk"], inp["kv_new"],
                                  np.where(ok, pos, 0), inp["cache"], inp["block_table"],
                                  inp["bs"], inp["stride"], B, S, D_C)
    qr = mo.rope(inp["q_pe"], pos[:, None].astype(np.int64))
    g_ql, g_qr = f64(q_lat), f64(q_rope)
    assert np.all(np.abs(g_ql - ql) <= 2 * half_ulp(ql, dt) + (1e-4 if dt != "f32" else 1e-5))
    assert np.all(np.abs(g_qr - qr) <= half_ulp(qr, dt) + ROT_TOL * (np.abs(qr) + 1))
    got = f64(cache)
    written = set()
    for t in range(B * S):
        if not ok[t]:
            continue
        row = mo.cache_slot(t // S, int(pos[t]), inp["block_table"], inp["bs"], inp["stride"])
        written.add(row)
        assert np.array_equal(got[row, :D_C], inp["kv_new"][t, :D_C])
        want = mo.rope(inp["kv_new"][t, D_C:], int(pos[t]))
        assert np.all(np.abs(got[row, D_C:] - want) <= half_ulp(want, dt) + ROT_TOL * (np.abs(want) + 1))
    assert len(written) == int(ok.sum())  # distinct slots
    others = np.array([rr for rr in range(got.shape[0]) if rr not in written])
    assert torch.equal(cache[torch.from_numpy(others).cuda()], before[torch.from_numpy(others).cuda()])
