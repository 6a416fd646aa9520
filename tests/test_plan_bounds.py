"""The split plan of mla_decode_partial, queried through the C ABI
(mla_decode_partial_plan evaluates the same rule the kernel evaluates on the
device; host arithmetic only, no GPU).

The rule cuts every (part, sequence) range of nt tiles into
max(1, ceil(nt / c)) chunks, with c the one-round size
c0 = max(4, ceil(T S / G)) or, when c0's chunks make between one and two
rounds of G = 256 workgroups, the two-round size
c1 = max(4, ceil(2 S T / (4 G - S U)), ceil(S T / (2 G))) if its chunks fit
in two rounds (T = all tiles, U = ranges, S = queries per range). The launch
sizes its grid for max(U + ceil(G / S), ceil(2 G / S)) + 1 chunks and the
split workspace for ceil(2 G / S) + 1 slots; the brute force below checks
that no range set overflows either, and the worked examples pin the chosen
sizes by hand."""
import numpy as np
import torch

from mla_split_kv_absorbed_amd import _lib as L

G = 256
TILE = 32


def plan(starts, ends, S=1, num_splits=0, flags=0):
    """The library's plan for one part of len(starts) sequences over a
    contiguous cache large enough for every range (the argument struct's
    device pointers are never read by the plan query)."""
    starts = np.asarray(starts, np.int32).reshape(1, -1)
    ends = np.asarray(ends, np.int32).reshape(1, -1)
    B = starts.shape[1]
    d = torch.empty(1, dtype=torch.bfloat16)
    lse = torch.empty(1, dtype=torch.float32)
    rs = torch.from_numpy(starts)
    a = L.partial_args(d, d, d, rs, rs, d, lse, B=B, S=S, H=128, scale=0.1,
                       kv_seq_stride=1 << 30, num_splits=num_splits, flags=flags)
    return L.mla_decode_partial_plan(a, starts, ends)


def tiles_to_ranges(nts):
    return np.zeros(len(nts), np.int32), (np.asarray(nts) * TILE).astype(np.int32)


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
        info = plan(*tiles_to_ranges(nts), S=S)
        assert info.matrix_path == 1
        assert info.max_chunks == max(U + -(-G // S), -(-2 * G // S)) + 1
        assert info.max_split_slots == -(-2 * G // S) + 1
        assert info.chunks <= info.max_chunks, (U, S, info.chunk_tiles)
        assert info.split_chunks <= info.max_split_slots, (U, S, info.chunk_tiles)
        # the reported chunk size accounts for every chunk
        n = np.maximum(1, -(-nts // info.chunk_tiles))
        assert info.chunks == n.sum() and info.split_chunks == n[n > 1].sum()
        assert info.split_ranges == (n > 1).sum()
        assert info.chunk_tiles >= 4


def test_two_round_size_on_a_ragged_batch():
    """256 ranges whose one-round chunks make 1.5 rounds take the two-round
    size: T = 100 x 46 + 156 x 20 = 7720 tiles, c0 = ceil(7720 / 256) = 31
    gives 100 x 2 + 156 x 1 = 356 chunks (one round and a short one);
    c1 = max(4, ceil(15440 / 768), ceil(7720 / 512)) = 21 gives
    100 x 3 + 156 = 456 <= 512."""
    info = plan(*tiles_to_ranges([46] * 100 + [20] * 156))
    assert info.chunk_tiles == 21 and info.chunks == 456
    assert info.split_ranges == 100 and info.split_chunks == 300


def test_equal_split_policy():
    """For ranges with equal tile counts the plan reports the chunk count
    per range (1 once the (range, query) units fill the 256 workgroups);
    ragged, empty or invalid ranges report 0."""
    z = np.zeros(256, np.int32)
    assert plan(z, np.full(256, 4096)).equal_splits == 1          # 256 equal units
    # 32 units of 128 tiles: chunks of max(4, 4096 / 256) = 16 tiles -> 8 per range
    assert plan(z[:32], np.full(32, 4096)).equal_splits == 8
    # 4 units of 2 tiles: chunks of at least 4 tiles -> no cut
    assert plan(z[:4], np.full(4, 64)).equal_splits == 1
    # 16 units of 100 tiles x 2 queries: c0 = ceil(3200 / 256) = 13 -> 8 per range
    assert plan(z[:16], np.full(16, 3200), S=2).equal_splits == 8
    en2 = np.full(256, 4096)
    en2[0] = 100
    assert plan(z, en2).equal_splits == 0                          # ragged
    assert plan(z, np.zeros(256)).equal_splits == 0                # empty ranges
    # equal lengths but a start inside a tile: 2 tiles against 3
    assert plan([0, 16], [64, 80]).equal_splits == 0
    assert plan(z[:128], np.full(128, 4096), S=2).equal_splits == 1  # 128 units x 2 queries
    # 40 units of 50 tiles: chunks of 8 make 280 workgroups (one round and a
    # short one); chunks of max(4, ceil(4000 / 984), ceil(2000 / 512)) = 5
    # make 400, two rounds -> 10 per range
    assert plan(z[:40], np.full(40, 1600)).equal_splits == 10
    # x 4 queries: c0 = 32 makes 320 workgroups; c1 = max(ceil(16000 / 864),
    # ceil(8000 / 512)) = 19 makes 4 x 120 = 480 -> 3 per range
    assert plan(z[:40], np.full(40, 1600), S=4).equal_splits == 3
    # x 8 queries: c0 = 63 makes 320 workgroups, c1 = 46 would make 640, more
    # than two rounds: c0 is kept -> 1 per range
    assert plan(z[:40], np.full(40, 1600), S=8).equal_splits == 1
    # a range past the addressable positions is invalid
    assert plan([0, 0], [64, (1 << 30) + 1]).equal_splits == 0


def test_explicit_split_count():
    """num_splits = k cuts every range into exactly k pieces (no chunk size)."""
    info = plan(np.zeros(10), np.full(10, 640), num_splits=3)
    assert info.chunk_tiles == 0 and info.chunks == 30
    assert info.split_ranges == 10 and info.split_chunks == 30
    assert info.max_chunks == 30 and info.max_split_slots == 30
    info = plan(np.zeros(10), np.full(10, 640), num_splits=1)
    assert info.chunks == 10 and info.split_chunks == 0 and info.max_split_slots == 0


def test_plain_kernel_plan():
    """fp32 (or the forced plain kernel) cuts nothing."""
    info = plan(np.zeros(4), np.full(4, 4096), flags=L.MLA_FLAG_FORCE_SIMPLE)
    assert info.matrix_path == 0 and info.chunks == 4 and info.split_chunks == 0
