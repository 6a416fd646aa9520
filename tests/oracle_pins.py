"""Pins for the CPU oracle: checks against facts that do not come from the
oracle itself (brute force, a library routine it does not use, algebraic
identities, closed forms, the pages' printed layout sizes).

Each pin takes the oracle module as an argument and returns its worst error
(or raises), so the planted-mistake tests can run the same pins against a
deliberately broken copy of the oracle.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-12


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def tiny_problem(seed=0, B=2, H=2, S=1, lengths=(5, 8), d_c=8, d_r=4, d_nope=4, d_v=4,
                 current=False, wscale=0.5):
    r = _rng(seed)
    return dict(
        w_uk=r.standard_normal((H, d_c, d_nope)) * wscale,
        w_uv=r.standard_normal((H, d_c, d_v)) * wscale,
        q_nope=r.standard_normal((B * S, H, d_nope)),
        q_rope=r.standard_normal((B * S, H, d_r)),
        rows=[r.standard_normal((lengths[b], d_c + d_r)) for b in range(B)],
        cur=[r.standard_normal((S, d_c + d_r)) for b in range(B)] if current else None,
        B=B, H=H, S=S, d_c=d_c, d_r=d_r, scale=1.0 / math.sqrt(d_nope + d_r),
    )


def run_step(mo, pr):
    cur = (lambda b: pr["cur"][b]) if pr["cur"] is not None else None
    return mo.mla_decode_step(pr["q_nope"], pr["q_rope"], lambda b: pr["rows"][b],
                              pr["w_uk"], pr["w_uv"], pr["scale"], pr["S"], cur_rows=cur)


# ---------------------------------------------------------------------------
# brute force: explicit loops, exp(s)/sum exp(s) with no max subtraction
# ---------------------------------------------------------------------------

def brute_force_step(pr):
    B, H, S, d_c = pr["B"], pr["H"], pr["S"], pr["d_c"]
    w_uk, w_uv = pr["w_uk"], pr["w_uv"]
    d_nope, d_v = w_uk.shape[2], w_uv.shape[2]
    out = np.zeros((B * S, H, d_v))
    lse = np.zeros((B * S, H))
    for b in range(B):
        hist = [list(x) for x in pr["rows"][b]]
        cur = [list(x) for x in pr["cur"][b]] if pr["cur"] is not None else []
        for s in range(S):
            keys = hist + cur[: s + 1]
            t = b * S + s
            for h in range(H):
                scores, vals = [], []
                for row in keys:
                    k = []
                    for i in range(d_nope):
                        acc = 0.0
                        for c in range(d_c):
                            acc += row[c] * w_uk[h][c][i]
                        k.append(acc)
                    k += row[d_c:]
                    v = []
                    for i in range(d_v):
                        acc = 0.0
                        for c in range(d_c):
                            acc += row[c] * w_uv[h][c][i]
                        v.append(acc)
                    q = list(pr["q_nope"][t][h]) + list(pr["q_rope"][t][h])
                    dot = 0.0
                    for i in range(len(q)):
                        dot += q[i] * k[i]
                    scores.append(pr["scale"] * dot)
                    vals.append(v)
                z = 0.0
                for sc in scores:
                    z += math.exp(sc)
                for i in range(d_v):
                    acc = 0.0
                    for j, sc in enumerate(scores):
                        acc += math.exp(sc) / z * vals[j][i]
                    out[t][h][i] = acc
                lse[t][h] = math.log(z)
    return out, lse


def pin_brute_force(mo):
    err = 0.0
    cases = [dict(seed=1), dict(seed=2, lengths=(1, 7)),
             dict(seed=3, S=2, current=True, lengths=(3, 6)),
             dict(seed=4, S=2, current=True, lengths=(0, 2))]
    for kw in cases:
        pr = tiny_problem(**kw)
        o, l = run_step(mo, pr)
        ob, lb = brute_force_step(pr)
        err = max(err, np.abs(o - ob).max(), np.abs(l - lb).max())
    return err


# ---------------------------------------------------------------------------
# library routine the oracle does not use: torch SDPA in float64 on the CPU
# ---------------------------------------------------------------------------

def pin_sdpa(mo):
    import torch
    r = _rng(11)
    H, L, d_c, d_r, d_n = 16, 256, 512, 64, 128
    w_uk = r.standard_normal((H, d_c, d_n)) / math.sqrt(d_c)
    w_uv = r.standard_normal((H, d_c, d_n)) / math.sqrt(d_c)
    q_nope = r.standard_normal((1, H, d_n))
    q_rope = r.standard_normal((1, H, d_r))
    rows = r.standard_normal((L, d_c + d_r))
    scale = 1.0 / math.sqrt(d_n + d_r)
    o, _ = mo.mla_decode_step(q_nope, q_rope, lambda b: rows, w_uk, w_uv, scale, 1)
    err = 0.0
    c = torch.from_numpy(rows[:, :d_c])
    kr = torch.from_numpy(rows[:, d_c:])
    for h in range(H):
        K = torch.cat([c @ torch.from_numpy(w_uk[h]), kr], dim=1)          # [L,192]
        V = c @ torch.from_numpy(w_uv[h])                                 # [L,128]
        q = torch.cat([torch.from_numpy(q_nope[0, h]), torch.from_numpy(q_rope[0, h])])
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[None, None, None, :], K[None, None], V[None, None], scale=scale)[0, 0, 0]
        err = max(err, float((ref - torch.from_numpy(o[0, h])).abs().max()))
    return err


# ---------------------------------------------------------------------------
# absorption: an absorbed implementation written only here must agree
# ---------------------------------------------------------------------------

def absorbed_step(pr):
    B, H, S, d_c = pr["B"], pr["H"], pr["S"], pr["d_c"]
    out = np.zeros((B * S, H, pr["w_uv"].shape[2]))
    lse = np.zeros((B * S, H))
    for b in range(B):
        rows = pr["rows"][b]
        for s in range(S):
            keys = rows if pr["cur"] is None else np.concatenate([rows, pr["cur"][b][: s + 1]])
            t = b * S + s
            for h in range(H):
                q_lat = np.einsum("cj,j->c", pr["w_uk"][h], pr["q_nope"][t, h])
                sc = pr["scale"] * (keys[:, :d_c] @ q_lat + keys[:, d_c:] @ pr["q_rope"][t, h])
                m = sc.max()
                p = np.exp(sc - m)
                o_lat = (p[:, None] * keys[:, :d_c]).sum(0) / p.sum()
                out[t, h] = np.einsum("c,cv->v", o_lat, pr["w_uv"][h])
                lse[t, h] = m + math.log(p.sum())
    return out, lse


def pin_absorption(mo):
    err = 0.0
    for kw in [dict(seed=5, lengths=(6, 3)), dict(seed=6, S=2, current=True),
               dict(seed=7, d_c=32, d_r=8, d_nope=8, d_v=8, lengths=(40, 17), H=3)]:
        pr = tiny_problem(**kw)
        o, l = run_step(mo, pr)
        oa, la = absorbed_step(pr)
        err = max(err, np.abs(o - oa).max() / max(1.0, np.abs(oa).max()), np.abs(l - la).max())
    # the library-shaped pieces: q_absorb -> latent_partial -> v_up == step
    pr = tiny_problem(seed=8, d_c=16, d_r=4, d_nope=8, d_v=8, lengths=(9, 12), H=2)
    o, l = run_step(mo, pr)
    q_lat = mo.q_absorb(pr["q_nope"], pr["w_uk"])
    for b in range(pr["B"]):
        n = pr["rows"][b].shape[0]
        ol, ll = mo.latent_partial(q_lat[b:b + 1], pr["q_rope"][b:b + 1], pr["rows"][b], 0, n,
                                   pr["scale"])
        ov = mo.v_up(ol, pr["w_uv"])
        err = max(err, np.abs(ov - o[b:b + 1]).max(), np.abs(ll - l[b:b + 1]).max())
    # q_absorb against explicit loops
    qn, wk = pr["q_nope"], pr["w_uk"]
    ql = mo.q_absorb(qn, wk)
    for t in range(qn.shape[0]):
        for h in range(qn.shape[1]):
            for c in range(wk.shape[1]):
                acc = 0.0
                for j in range(wk.shape[2]):
                    acc += wk[h][c][j] * qn[t][h][j]
                err = max(err, abs(acc - ql[t, h, c]))
    return err


# ---------------------------------------------------------------------------
# split invariance of the LSE combine, two-part closed form
# ---------------------------------------------------------------------------

def pin_split_invariance(mo):
    r = _rng(21)
    err = 0.0
    d_c, d_r, H, S = 16, 4, 3, 1
    for trial in range(12):
        L = int(r.integers(1, 60))
        rows = r.standard_normal((L, d_c + d_r))
        q_lat = r.standard_normal((S, H, d_c))
        q_rope = r.standard_normal((S, H, d_r))
        whole_o, whole_l = mo.latent_partial(q_lat, q_rope, rows, 0, L, 0.3)
        P = int(r.integers(1, 7))
        cuts = np.sort(r.integers(0, L + 1, size=P - 1))
        if trial % 3 == 0 and P > 1:
            cuts[0] = 0                     # an empty part first
        if trial % 3 == 1:
            cuts = np.sort(np.concatenate([cuts, [L - 1, L]]))[: P - 1] if P > 1 else cuts
        bounds = [0] + list(cuts) + [L]
        outs, lses = [], []
        for p in range(len(bounds) - 1):
            o, l = mo.latent_partial(q_lat, q_rope, rows, bounds[p], bounds[p + 1], 0.3)
            outs.append(o)
            lses.append(l)
        co, cl = mo.lse_combine(np.stack(outs), np.stack(lses))
        err = max(err, np.abs(co - whole_o).max(), np.abs(cl - whole_l).max())
    # two parts, closed form with explicit exponentials (small values)
    o1, o2 = r.standard_normal(5), r.standard_normal(5)
    l1, l2 = 0.7, -1.3
    co, cl = mo.lse_combine(np.stack([o1, o2]), np.array([l1, l2]))
    e1, e2 = math.exp(l1), math.exp(l2)
    err = max(err, np.abs(co - (e1 * o1 + e2 * o2) / (e1 + e2)).max(),
              abs(cl - math.log(e1 + e2)))
    # an empty part carries no weight; all-empty gives 0 / -inf
    co, cl = mo.lse_combine(np.stack([o1, np.full(5, 7.0)]), np.array([l1, -math.inf]))
    err = max(err, np.abs(co - o1).max(), abs(cl - l1))
    co, cl = mo.lse_combine(np.zeros((3, 5)), np.full(3, -math.inf))
    if not (np.all(co == 0) and cl == -math.inf):
        return math.inf
    return err


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def pin_closed_forms(mo):
    r = _rng(31)
    err = 0.0
    d = 6
    K = r.standard_normal((1, d))
    V = r.standard_normal((1, 3))
    q = r.standard_normal((1, d))
    o, l = mo.attend(q, K, V, 0.5)                            # one key
    err = max(err, np.abs(o[0] - V[0]).max(), abs(l[0] - 0.5 * float(q[0] @ K[0])))
    L = 9
    K = r.standard_normal((L, d))
    V = r.standard_normal((L, 3))
    o, l = mo.attend(np.zeros((1, d)), K, V, 0.5)              # q = 0
    err = max(err, np.abs(o[0] - V.mean(0)).max(), abs(l[0] - math.log(L)))
    Kr = np.repeat(K[:1], L, axis=0)
    Vr = np.repeat(V[:1], L, axis=0)
    o, l = mo.attend(q, Kr, Vr, 0.5)                           # one key repeated
    s0 = 0.5 * float(q[0] @ K[0])
    err = max(err, np.abs(o[0] - V[0]).max(), abs(l[0] - (s0 + math.log(L))))
    o, l = mo.attend(q, K[:2], V[:2], 0.5)                     # two keys
    s = 0.5 * (K[:2] @ q[0])
    p0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
    err = max(err, np.abs(o[0] - (p0 * V[0] + (1 - p0) * V[1])).max())
    # empty key set
    o, l = mo.attend(q, K[:0], V[:0], 0.5)
    if not (np.all(o == 0) and l[0] == -math.inf):
        return math.inf
    return err


def pin_extreme_part(mo):
    """One part's scores sit ~80 above the rest: no overflow, and the merge
    of the parts still equals the unsplit result."""
    r = _rng(41)
    d_c, d_r, H, L = 16, 4, 2, 48
    rows = r.standard_normal((L, d_c + d_r))
    q_lat = r.standard_normal((1, H, d_c))
    q_rope = r.standard_normal((1, H, d_r))
    # align part 2's keys with the query so its scores are large
    for h in range(H):
        pass
    qv = np.concatenate([q_lat[0, 0], q_rope[0, 0]])
    rows[32:40] = qv / np.dot(qv, qv) * 80.0 / 0.25 + 0.01 * rows[32:40]
    whole_o, whole_l = mo.latent_partial(q_lat, q_rope, rows, 0, L, 0.25)
    outs, lses = [], []
    for a, b in [(0, 16), (16, 32), (32, 40), (40, 48)]:
        o, l = mo.latent_partial(q_lat, q_rope, rows, a, b, 0.25)
        outs.append(o)
        lses.append(l)
    co, cl = mo.lse_combine(np.stack(outs), np.stack(lses))
    if not (np.all(np.isfinite(co)) and np.all(np.isfinite(cl))):
        return math.inf
    if whole_l[0, 0] < 60:
        return math.inf        # the construction must really produce extreme scores
    return max(np.abs(co - whole_o).max() / np.abs(whole_o).max(),
               np.abs(cl - whole_l).max() / np.abs(whole_l).max())


def pin_causal_window(mo):
    """MTP: query 0 == a one-query step over history + current token 0;
    query 1 == a one-query step over history + both current tokens."""
    pr = tiny_problem(seed=51, S=2, current=True, lengths=(4, 6))
    o2, l2 = run_step(mo, pr)
    err = 0.0
    for s in range(2):
        pr1 = dict(pr)
        pr1["S"] = 1
        pr1["q_nope"] = pr["q_nope"][s::2]
        pr1["q_rope"] = pr["q_rope"][s::2]
        pr1["rows"] = [np.concatenate([pr["rows"][b], pr["cur"][b][: s + 1]]) for b in range(2)]
        pr1["cur"] = None
        o1, l1 = run_step(mo, pr1)
        err = max(err, np.abs(o1 - o2[s::2]).max(), np.abs(l1 - l2[s::2]).max())
    # the latent partial's causal flag against the same reading
    r = _rng(52)
    rows = r.standard_normal((2, 20))
    ql, qr = r.standard_normal((2, 1, 16)), r.standard_normal((2, 1, 4))
    o, l = mo.latent_partial(ql, qr, rows, 0, 2, 0.3, causal=True)
    o0, l0 = mo.latent_partial(ql[:1], qr[:1], rows, 0, 1, 0.3)
    o1, l1 = mo.latent_partial(ql[1:], qr[1:], rows, 0, 2, 0.3)
    err = max(err, np.abs(o[0] - o0[0]).max(), np.abs(l[0] - l0[0]).max(),
              np.abs(o[1] - o1[0]).max(), np.abs(l[1] - l1[0]).max())
    return err


def pin_vup_bmm(mo):
    import torch
    r = _rng(61)
    T, H = 5, 4
    x = r.standard_normal((T, H, 512))
    w = r.standard_normal((H, 512, 128))
    ref = torch.bmm(torch.from_numpy(x).transpose(0, 1).contiguous(),
                    torch.from_numpy(w)).transpose(0, 1).numpy()
    return float(np.abs(mo.v_up(x, w) - ref).max())


def pin_layout_sizes(mo):
    with open(os.path.join(GOLDEN, "layout_sizes.json")) as f:
        g = json.load(f)
    per_tok = mo.latent_bytes_per_token(g["d_c"], g["d_R"], g["elem_bytes"])
    bad = 0.0
    bad = max(bad, abs(round(per_tok / 1000.0, 2) - g["per_token_kB_decimal_2dp"]))
    for bs, kib in g["block_KiB"].items():
        bad = max(bad, abs(mo.block_bytes(int(bs), g["d_c"], g["d_R"], g["elem_bytes"]) - kib * 1024))
    return bad


# ---------------------------------------------------------------------------
# the decode prologue: rotary embedding and cache append
# ---------------------------------------------------------------------------

def pin_rope_closed_forms(mo):
    """Closed forms of the rotation: position 0 is the identity; a unit vector
    in pair i at position p lands at (cos, sin) of p * theta^(-2i/d) (pair 0
    has frequency 1, pair 1 of d = 4 has theta^(-1/2)); rotations by m then n
    compose to m + n; each pair keeps its length."""
    theta = 10000.0
    bad = 0.0
    x = _rng(71).standard_normal((5, 64))
    bad = max(bad, np.abs(mo.rope(x, np.zeros(5)) - x).max())
    for p in (1, 7, 1000, 32767):
        y = mo.rope(np.array([1.0, 0.0]), p, theta)
        bad = max(bad, abs(y[0] - math.cos(p)), abs(y[1] - math.sin(p)))
        y = mo.rope(np.array([0.0, 0.0, 1.0, 0.0]), p, theta)
        a = p * theta ** -0.5
        bad = max(bad, abs(y[0]), abs(y[1]), abs(y[2] - math.cos(a)), abs(y[3] - math.sin(a)))
        y = mo.rope(np.array([0.0, 1.0]), p, theta)
        bad = max(bad, abs(y[0] + math.sin(p)), abs(y[1] - math.cos(p)))
    m, n = np.array([3, 50, 9000]), np.array([11, 4, 123])
    x = _rng(72).standard_normal((3, 64))
    bad = max(bad, np.abs(mo.rope(mo.rope(x, m), n) - mo.rope(x, m + n)).max() / 10.0)
    y = mo.rope(x, m)
    bad = max(bad, np.abs(np.hypot(y[:, 0::2], y[:, 1::2]) - np.hypot(x[:, 0::2], x[:, 1::2])).max())
    return bad


def pin_rope_relative(mo):
    """The defining property of rotary embedding: the dot product of a query
    rotated to position m and a key rotated to position n depends only on
    m - n."""
    r = _rng(73)
    q, k = r.standard_normal((4, 64)), r.standard_normal((4, 64))
    bad = 0.0
    for m, n in ((5, 2), (300, 17), (16000, 15990), (7, 7)):
        a = np.einsum("ij,ij->i", mo.rope(q, np.full(4, m)), mo.rope(k, np.full(4, n)))
        b = np.einsum("ij,ij->i", mo.rope(q, np.full(4, m - n)), k)
        bad = max(bad, np.abs(a - b).max() / 64.0)
    return bad


def pin_cache_append(mo):
    """Appending the new tokens through a paged block table: reading every
    sequence back in logical order by gathering its blocks shows the new
    rows (latent copied, rope part rotated) at their positions and every
    other token unchanged; the same holds for a contiguous cache. The
    absorbed query and rotated query rope part match their definitions."""
    r = _rng(74)
    B, S, H, bs, d_c, d_r, dn = 3, 2, 2, 4, 8, 4, 4
    nb_per = 3
    perm = r.permutation(B * nb_per + 2)  # two spare blocks
    block_table = perm[:B * nb_per].reshape(B, nb_per).astype(np.int32)
    cache = r.standard_normal((perm.size * bs, d_c + d_r))
    T = B * S
    kv_new = r.standard_normal((T, d_c + d_r))
    positions = np.array([5, 6, 0, 1, 10, 11], np.int32)
    q_nope, q_pe = r.standard_normal((T, H, dn)), r.standard_normal((T, H, d_r))
    w_uk = r.standard_normal((H, d_c, dn))
    ql, qr, new = mo.decode_prologue(q_nope, q_pe, w_uk, kv_new, positions, cache,
                                     block_table, bs, 0, B, S, d_c)
    bad = 0.0
    blocks_old = cache.reshape(-1, bs, d_c + d_r)
    blocks_new = new.reshape(-1, bs, d_c + d_r)
    for b in range(B):
        seq_old = blocks_old[block_table[b]].reshape(-1, d_c + d_r)
        seq_new = blocks_new[block_table[b]].reshape(-1, d_c + d_r)
        touched = set()
        for s_ in range(S):
            t = b * S + s_
            p = int(positions[t])
            touched.add(p)
            bad = max(bad, np.abs(seq_new[p, :d_c] - kv_new[t, :d_c]).max())
            want = mo.rope(kv_new[t, d_c:], p)
            bad = max(bad, np.abs(seq_new[p, d_c:] - want).max())
        for p in range(seq_old.shape[0]):
            if p not in touched:
                bad = max(bad, np.abs(seq_new[p] - seq_old[p]).max())
    spare = blocks_new[perm[B * nb_per:]]
    bad = max(bad, np.abs(spare - blocks_old[perm[B * nb_per:]]).max())
    # contiguous cache: sequence b occupies rows [b * stride, (b + 1) * stride)
    stride = 16
    cc = r.standard_normal((B * stride, d_c + d_r))
    _, _, cn = mo.decode_prologue(q_nope, q_pe, w_uk, kv_new, positions, cc, None, 0, stride,
                                  B, S, d_c)
    diff = np.argwhere(np.any(cn != cc, axis=1)).ravel().tolist()
    want_rows = sorted(b * stride + int(positions[b * S + s_]) for b in range(B) for s_ in range(S))
    bad = max(bad, 0.0 if diff == want_rows else 1.0)
    for h in range(H):
        bad = max(bad, np.abs(ql[:, h] - np.einsum("cj,tj->tc", w_uk[h], q_nope[:, h])).max())
    bad = max(bad, np.abs(qr - mo.rope(q_pe, positions[:, None])).max())
    return bad


PINS = {
    "brute_force": (pin_brute_force, 1e-12),
    "sdpa": (pin_sdpa, 1e-12),
    "absorption": (pin_absorption, 1e-12),
    "split_invariance": (pin_split_invariance, 1e-12),
    "closed_forms": (pin_closed_forms, 1e-12),
    "extreme_part": (pin_extreme_part, 1e-12),
    "causal_window": (pin_causal_window, 1e-12),
    "vup_bmm": (pin_vup_bmm, 1e-10),
    "layout_sizes": (pin_layout_sizes, 0.0),
    "rope_closed_forms": (pin_rope_closed_forms, 1e-9),
    "rope_relative": (pin_rope_relative, 1e-9),
    "cache_append": (pin_cache_append, 1e-12),
}
