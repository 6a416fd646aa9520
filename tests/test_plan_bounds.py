"""Bounds of the partial kernel's automatic split plan (host arithmetic, no
GPU). The plan cuts every (part, sequence) range of nt tiles into
max(1, ceil(nt / c)) chunks, with c the one-round size
c0 = max(4, ceil(T S / G)) or, when c0's chunks make between one and two
rounds of G workgroups, the two-round size
c1 = max(4, ceil(2 S T / (4 G - S U)), ceil(S T / (2 G))) if its chunks fit in
two rounds (T = all tiles, U = ranges, S = queries per range, G = 256). The
launch sizes its grid for max(U + ceil(G / S), ceil(2 G / S)) + 1 chunks and
the split workspace for ceil(2 G / S) + 1 slots (chunks of ranges cut in more
than one). This checks by brute force that no range set overflows either."""
import numpy as np

G = 256
MIN_CHUNK = 4


def chunks(nts, c):
    return np.maximum(1, -(-nts // c))


def plan_chunk_tiles(nts, S):
    U, T = len(nts), int(nts.sum())
    c = max(MIN_CHUNK, -(-T * S // G))
    if 4 * G > S * U:
        c1 = max(MIN_CHUNK, -(-2 * S * T // (4 * G - S * U)), -(-S * T // (2 * G)))
        if c1 < c and S * chunks(nts, c).sum() > G and S * chunks(nts, c1).sum() <= 2 * G:
            c = c1
    return c


def test_plan_chunks_fit_the_grid_and_the_workspace():
    rng = np.random.default_rng(2024)
    for trial in range(4000):
        U = int(rng.integers(1, 700))
        S = int(rng.integers(1, 5))
        kind = trial % 4
        if kind == 0:
            nts = rng.integers(0, 5000, U)
        elif kind == 1:
            nts = rng.integers(0, 40, U)
        elif kind == 2:  # a few long ranges among many short ones
            nts = np.where(rng.random(U) < 0.1, rng.integers(1000, 20000, U), rng.integers(0, 8, U))
        else:
            nts = np.full(U, int(rng.integers(0, 3000)))
        c = plan_chunk_tiles(nts, S)
        n = chunks(nts, c)
        assert n.sum() <= max(U + -(-G // S), -(-2 * G // S)) + 1, (U, S, c)
        assert n[n > 1].sum() <= -(-2 * G // S) + 1, (U, S, c)


def test_two_round_size_on_a_ragged_batch():
    """256 ranges whose one-round chunks make 1.5 rounds take the two-round size."""
    nts = np.array([46] * 100 + [20] * 156)   # T = 7720: c0 = 31 -> 356 chunks
    c = plan_chunk_tiles(nts, 1)
    assert c == max(MIN_CHUNK, -(-2 * 7720 // (1024 - 256)), -(-7720 // 512))   # 21
    assert G < chunks(nts, 31).sum() and chunks(nts, c).sum() <= 2 * G


def test_split_hint_matches_the_plan_on_equal_ranges():
    """For equal ranges the host's split_hint gives the chunk count per range
    that the plan's rule gives (or 1 once the ranges alone fill the target)."""
    from mla_split_kv_absorbed_amd.step import TILE, split_hint
    rng = np.random.default_rng(11)
    for _ in range(3000):
        U = int(rng.integers(1, 600))
        S = int(rng.integers(1, 5))
        L = int(rng.integers(1, 40000))
        nt = (L - 1) // TILE + 1
        hint = split_hint(np.zeros(U, np.int32), np.full(U, L, np.int32), S)
        if U * S >= G:
            assert hint == 1
        else:
            c = plan_chunk_tiles(np.full(U, nt), S)
            assert hint == max(1, -(-nt // c)), (U, S, L)
