"""CPU float64 oracle for absorbed split-KV MLA decode.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it. It shares no code with the HIP library or its binding;
the only module both sides use is the seeded input generator, which holds
none of the method's arithmetic.

What it computes is the plain definition of the result, written out:

* MLA keeps one latent row per cached token, c_KV (d_c = 512) plus a
  decoupled rotary key k_R (d_R = 64), shared by every query head; each head
  recovers its own key and value from the latent ("MLA multi-GPU sharding"
  page, section on c_t^KV / k_t^R; "RTPLLM on K3" page, section 2.1, the
  attention layer flow: recover K/V from the latent, QK, softmax, weighted
  sum).  The oracle therefore materialises, per head h,
  K_h = [c_KV . W_UK[h] || k_R] (192 wide) and V_h = c_KV . W_UV[h] (128 wide)
  and runs textbook softmax attention in float64 (`mla_decode_step`).  This is
  the NON-absorbed form; absorption is an exact regrouping of the same sums.
* A partial over one part of the keys returns (output, log-sum-exp); merging
  partials by their LSEs equals one softmax over all keys ("DCP decode
  streams / V-up study" page, background section and the combine step;
  `lse_combine`).
* V-up maps a batch-major latent [T][H][512] through W_UV[h] [512][128] to
  [T][H*128]; it equals bmm(x^T, W_UV)^T (same page, V-up fusion section;
  `v_up`).
* The absorbed query q_lat = W_UK[h] . q_nope (`q_absorb`) and the latent
  partial (`latent_partial`: attention whose keys are [c_KV || k_R] and whose
  values are c_KV itself) are the plain definitions of what the library's
  q-absorb and partial-attention entry points return.
* The decode prologue (`decode_prologue`): the step before the path. Rotary
  position embedding of the query's rope part and of the new token's k_R
  (`rope`: consecutive pairs rotated by pos * theta^(-2i/d_R), theta 10000;
  the pages name the fused RoPE prologue but fix no variant, so the
  original rotary formulation is the reading), q absorption, and the
  append of the new token's [c_KV || rope(k_R)] row at its paged slot
  (`cache_slot`).

Readings where the pages are silent: natural-log LSE of the *scaled* scores;
an empty key set gives output 0 and LSE -inf; the MTP current-window mask is
bottom-right aligned (query s of S sees keys j <= end - S + s of its range);
W_UK[h] is stored [512][128] like W_UV[h].

Pins (tests, CPU): brute-force loops without the max trick on tiny sizes, the
library SDPA routine over the oracle's materialised K/V, the absorbed form
(written only in the tests), split invariance of the combine, closed forms,
extreme shifted parts, the causal-window equivalences, the pages' printed
layout sizes, rotary closed forms and the relative-position identity, the
cache append read back through the block table, and planted-mistake
checks. The rotary frequency schedule itself is the reading above (parity
unpinned by the pages beyond the rotation's structure).  No page prints an attention output
or LSE value, so the numeric values themselves rest on the textbook
definition plus those checks.
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence

import numpy as np

NEG_INF = -math.inf


# ----------------------------------------------------------------------------
# textbook softmax attention
# ----------------------------------------------------------------------------

def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
           visible: Optional[np.ndarray] = None):
    """Softmax attention of n queries over L keys, float64.

    q [n, d], K [L, d], V [L, dv], visible [n, L] bool (None = all).
    Returns out [n, dv] = sum_j softmax_j(scale * q.K_j) V_j and
    lse [n] = ln sum_j exp(scale * q.K_j) (natural log of the scaled
    scores).  A query with no visible key gets out = 0, lse = -inf.
    """
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    n, L = q.shape[0], K.shape[0]
    out = np.zeros((n, V.shape[1]), np.float64)
    lse = np.full(n, NEG_INF, np.float64)
    if L == 0:
        return out, lse
    s = scale * (q @ K.T)                                  # [n, L]
    if visible is not None:
        s = np.where(visible, s, NEG_INF)
    m = s.max(axis=1)                                      # [n]
    has = np.isfinite(m)
    if not has.any():
        return out, lse
    e = np.zeros_like(s)
    e[has] = np.exp(s[has] - m[has, None])
    z = e.sum(axis=1)
    lse[has] = m[has] + np.log(z[has])
    out[has] = (e[has] / z[has, None]) @ V
    return out, lse


def causal_window_visible(n_keys: int, S: int) -> np.ndarray:
    """Bottom-right aligned window: query s of S sees keys j <= n_keys - S + s."""
    j = np.arange(n_keys)[None, :]
    s = np.arange(S)[:, None]
    return j <= (n_keys - S + s)


# ----------------------------------------------------------------------------
# the full decode step, non-absorbed (materialised per-head K and V)
# ----------------------------------------------------------------------------

def materialize_kv(rows: np.ndarray, w_uk_h: np.ndarray, w_uv_h: np.ndarray, d_c: int):
    """rows [L][d_c + d_R] (c_KV || k_R) -> K [L][d_nope + d_R], V [L][d_v]."""
    c = rows[:, :d_c]
    k_r = rows[:, d_c:]
    K = np.concatenate([c @ w_uk_h, k_r], axis=1)
    V = c @ w_uv_h
    return K, V


def mla_decode_step(q_nope: np.ndarray, q_rope: np.ndarray,
                    seq_rows: Callable[[int], np.ndarray],
                    w_uk: np.ndarray, w_uv: np.ndarray, scale: float, S: int,
                    cur_rows: Optional[Callable[[int], np.ndarray]] = None,
                    seqs: Optional[Sequence[int]] = None,
                    heads: Optional[Sequence[int]] = None):
    """One MLA decode step for the selected sequences and heads.

    q_nope [T][H][d_nope], q_rope [T][H][d_R] with t = b*S + s;
    seq_rows(b) -> cached latent rows [L_b][d_c + d_R] in logical order;
    cur_rows(b) -> the current chunk's rows [S][d_c + d_R] (MTP), or None.
    Query s of sequence b sees every cached row plus current rows 0..s.
    Returns out [T][H][d_v] and lse [T][H] (float64, NaN where not computed).
    """
    T, H, _ = q_nope.shape
    B = T // S
    d_c = w_uk.shape[1]
    d_v = w_uv.shape[2]
    out = np.full((T, H, d_v), np.nan)
    lse = np.full((T, H), np.nan)
    seqs = range(B) if seqs is None else seqs
    heads = range(H) if heads is None else heads
    for b in seqs:
        rows = seq_rows(b)
        L = rows.shape[0]
        vis = None
        if cur_rows is not None:
            rows = np.concatenate([rows, cur_rows(b)], axis=0)
            vis = causal_window_visible(rows.shape[0], S)
        for h in heads:
            K, V = materialize_kv(rows, w_uk[h], w_uv[h], d_c)
            q = np.concatenate([q_nope[b * S:(b + 1) * S, h], q_rope[b * S:(b + 1) * S, h]], axis=1)
            o, l = attend(q, K, V, scale, vis)
            out[b * S:(b + 1) * S, h] = o
            lse[b * S:(b + 1) * S, h] = l
    return out, lse


# ----------------------------------------------------------------------------
# the pieces the library exposes, each by its plain definition
# ----------------------------------------------------------------------------

def q_absorb(q_nope: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """q_lat[t,h,c] = sum_j W_UK[h,c,j] * q_nope[t,h,j]  ([T][H][d_c])."""
    T, H, _ = q_nope.shape
    out = np.empty((T, H, w_uk.shape[1]), np.float64)
    for h in range(H):
        out[:, h, :] = q_nope[:, h, :] @ w_uk[h].T
    return out


def latent_partial(q_lat: np.ndarray, q_rope: np.ndarray, rows: np.ndarray,
                   start: int, end: int, scale: float, causal: bool = False):
    """Attention of one sequence's S queries over keys [start, end) of its rows
    with keys [c_KV || k_R] and values c_KV (the latent partial a part emits).

    q_lat [S][H][d_c], q_rope [S][H][d_R], rows [>=end][d_c + d_R].
    causal: bottom-right aligned window over the range (query s sees range
    positions j <= (end - start) - S + s).
    Returns o_lat [S][H][d_c], lse [S][H].
    """
    S, H, d_c = q_lat.shape
    keys = rows[start:end]
    n = keys.shape[0]
    # every (query, head) pair is one query row of the same key set: the S*H
    # rows go through attend together (each row's softmax is its own)
    q = np.concatenate([q_lat, q_rope], axis=2).reshape(S * H, -1)
    vis = np.repeat(causal_window_visible(n, S), H, axis=0) if causal else None
    o, l = attend(q, keys, keys[:, :d_c], scale, vis)
    return o.reshape(S, H, d_c), l.reshape(S, H)


def lse_combine(outs: np.ndarray, lses: np.ndarray):
    """Merge P partial results by their log-sum-exps.

    outs [P][...][D], lses [P][...]. With m = max_i lse_i and
    w_i = exp(lse_i - m): out = sum_i w_i out_i / sum_i w_i,
    lse = m + ln sum_i w_i. Parts with lse = -inf carry weight 0; if every
    part is empty the result is out = 0, lse = -inf.
    """
    outs = np.asarray(outs, np.float64)
    lses = np.asarray(lses, np.float64)
    m = lses.max(axis=0)
    finite = np.isfinite(m)
    msafe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - msafe[None]), 0.0)
    z = w.sum(axis=0)
    zs = np.where(finite, z, 1.0)
    out = np.where(finite[..., None], (w[..., None] * outs).sum(axis=0) / zs[..., None], 0.0)
    lse = np.where(finite, msafe + np.log(zs), NEG_INF)
    return out, lse


def v_up(x: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """out[t,h,:] = x[t,h,:] . W_UV[h]  (x [T][H][d_c], W_UV [H][d_c][d_v]);
    reshaping the result to [T][H*d_v] gives the layer's attention output."""
    T, H, _ = x.shape
    out = np.empty((T, H, w_uv.shape[2]), np.float64)
    for h in range(H):
        out[:, h, :] = x[:, h, :] @ w_uv[h]
    return out


# ----------------------------------------------------------------------------
# layout sizes printed on the pages
# ----------------------------------------------------------------------------

def latent_bytes_per_token(d_c: int, d_r: int, elem_bytes: int) -> int:
    """Bytes one cached token occupies: (d_c + d_R) values."""
    return (d_c + d_r) * elem_bytes


def block_bytes(block_size: int, d_c: int, d_r: int, elem_bytes: int) -> int:
    """Bytes of one paged cache block of `block_size` tokens."""
    return block_size * latent_bytes_per_token(d_c, d_r, elem_bytes)


# ----------------------------------------------------------------------------
# the decode prologue: rotary position embedding, q absorption, cache append
# ----------------------------------------------------------------------------

def rope(x: np.ndarray, pos, theta: float = 10000.0) -> np.ndarray:
    """Rotary position embedding of the decoupled rope part (d_R values on the
    last axis) at integer position(s) `pos` (broadcast against x[..., 0]).

    The "MLA multi-GPU sharding" page calls k_R the small decoupled rotary
    position vector and the "RTPLLM on K3" page (section 4.1) fuses the RoPE
    transform into the attention prologue; neither fixes the variant. The
    reading taken: the original rotary formulation, each consecutive pair
    (x[2i], x[2i+1]) rotated by the angle pos * theta^(-2i/d_R):
        y[2i]   = x[2i] cos(a_i) - x[2i+1] sin(a_i)
        y[2i+1] = x[2i] sin(a_i) + x[2i+1] cos(a_i)
    """
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    i = np.arange(d // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / d)
    ang = np.asarray(pos, np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = xe * c - xo * s
    y[..., 1::2] = xe * s + xo * c
    return y


def cache_slot(b: int, pos: int, block_table: Optional[np.ndarray], block_size: int,
               seq_stride: int) -> int:
    """Cache row of logical token `pos` of sequence b: block_table[b][pos / bs]
    * bs + pos % bs for a paged cache, b * seq_stride + pos for a contiguous
    one (the paged layout of the "MLA multi-GPU sharding" page's block
    sizes)."""
    if block_size > 0:
        return int(block_table[b, pos // block_size]) * block_size + pos % block_size
    return b * seq_stride + pos


def decode_prologue(q_nope: np.ndarray, q_pe: np.ndarray, w_uk: np.ndarray,
                    kv_new: np.ndarray, positions: np.ndarray, cache_rows: np.ndarray,
                    block_table: Optional[np.ndarray], block_size: int, seq_stride: int,
                    B: int, S: int, d_c: int, theta: float = 10000.0):
    """The step before the attention path, written out: for every new token
    t = b * S + s at position positions[t],
      q_lat[t]   = W_UK[h] . q_nope[t]            (absorption, per head)
      q_rope[t]  = rope(q_pe[t], positions[t])    (per head)
      cache row  = [c_KV(t) || rope(k_R(t), positions[t])]  appended at the
                   token's slot (every other row unchanged).
    cache_rows is the cache flattened to [rows][d_c + d_R]; a copy is
    returned. The "RTPLLM on K3" page (sections 2.1 and 4.1): the input
    projection yields the query's latent and rope parts and the compressed
    latent that the cache stores; RoPE is applied in the fused prologue."""
    q_lat = q_absorb(q_nope, w_uk)
    pos = np.asarray(positions, np.int64)
    q_rope = rope(q_pe, pos[:, None], theta)
    new = np.array(cache_rows, np.float64, copy=True)
    for b in range(B):
        for s_ in range(S):
            t = b * S + s_
            r = cache_slot(b, int(pos[t]), block_table, block_size, seq_stride)
            new[r, :d_c] = kv_new[t, :d_c]
            new[r, d_c:] = rope(kv_new[t, d_c:], int(pos[t]), theta)
    return q_lat, q_rope, new
