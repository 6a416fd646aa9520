"""The plan built on the host (mla_decode_partial_make_plan) against the split
rule the header documents, and the validation of the `plan` arguments (host
arithmetic only, no GPU).

For every range of nt tiles cut into n pieces, piece i must cover tiles
[i nt / n, (i + 1) nt / n); every piece must appear exactly once; cut ranges
(n > 1) take consecutive workspace slots, allocated in range order, and one
descriptor each; the automatic plan hands out chunk ids longest first (the
chunk length's bucket, then range order); an explicit count k maps chunk id
c to range c / k, piece c mod k, or, when the range count is a multiple of 8,
keeps a range's pieces on one XCD (c mod 8 = range mod 8)."""
import ctypes

import numpy as np
import pytest
import torch

from mla_split_kv_absorbed_amd import _lib as L
from tests.test_abi_cpu import FAKE, base_args

TILE = 32
MAGIC = 0x4D4C4131
HEADER, ENTRY, DESC = 8, 8, 4


def args_for(B, P, S, num_splits=0):
    """Arguments of P parts of B sequences over a contiguous cache large
    enough for every range (the plan builder reads no device pointer)."""
    d = torch.empty(1, dtype=torch.bfloat16)
    lse = torch.empty(1, dtype=torch.float32)
    rs = torch.zeros((P, 1), dtype=torch.int32)
    return L.partial_args(d, d, d, rs, rs, d, lse, B=B, S=S, H=128, scale=0.1,
                          kv_seq_stride=1 << 30, num_splits=num_splits)


def range_tiles(st, en):
    return (en - 1) // TILE - st // TILE + 1 if en > st else 0


def bucket(length, c):
    if length >= c:
        return 7
    return min(7, length * 8 // (c + 1))


def check_table(starts, ends, P, S, num_splits):
    B = starts.size // P
    a = args_for(B, P, S, num_splits)
    table, info = L.mla_decode_partial_make_plan(a, starts, ends)
    ref = L.mla_decode_partial_plan(a, starts, ends)
    U = P * B
    assert table[0] == MAGIC
    assert (table[1], table[2], table[3]) == (ref.chunks, ref.split_ranges, ref.chunk_tiles)
    assert (table[4], table[5], table[6]) == (U, S, num_splits)
    assert (info.chunks, info.split_ranges) == (ref.chunks, ref.split_ranges)
    n_chunks = int(table[1])
    ent = table[HEADER:HEADER + ENTRY * n_chunks].reshape(n_chunks, ENTRY)
    desc_off = HEADER + ENTRY * ref.max_chunks
    assert table.size == desc_off + DESC * U
    nt = np.array([range_tiles(int(s), int(e)) for s, e in zip(starts.ravel(), ends.ravel())])
    c = ref.chunk_tiles
    want_n = (np.full(U, num_splits) if num_splits > 0
              else np.maximum(1, -(-nt // c)))
    # every range's pieces, in order, tile it exactly once
    pieces = {}
    for cid, (u, tb, te, slot) in enumerate(ent[:, :4]):
        assert 0 <= u < U and 0 <= tb <= te <= max(nt[u], 0)
        pieces.setdefault(int(u), []).append((int(tb), int(te), int(slot), cid))
    assert sorted(pieces) == list(range(U))
    slot_next, splits = 0, []
    for u in range(U):
        p = sorted(pieces[u])
        n = want_n[u]
        assert len(p) == n
        for i, (tb, te, slot, _) in enumerate(p):
            assert tb == i * nt[u] // n and te == (i + 1) * nt[u] // n
        if n > 1:
            # consecutive slots from the next free one, in range order
            assert [q[2] for q in p] == list(range(slot_next, slot_next + n))
            splits.append((u, slot_next, n))
            slot_next += n
        else:
            assert p[0][2] == -1
    assert slot_next == ref.split_chunks and len(splits) == ref.split_ranges
    desc = table[desc_off:desc_off + DESC * len(splits)].reshape(-1, DESC)
    assert [tuple(map(int, d[:3])) for d in desc] == splits
    if num_splits == 0:
        # longest first: (bucket descending, range ascending, piece ascending)
        keys = [(-bucket((nt[u] + want_n[u] - 1) // want_n[u], c), u, tb)
                for u, tb, te, slot in ent[:, :4]]
        assert keys == sorted(keys)
    else:
        k = num_splits
        for cid, (u, tb, te, slot) in enumerate(ent[:, :4]):
            if U % 8 == 0:
                pos = cid >> 3
                assert u == (cid & 7) + 8 * (pos // k)
                i = pos % k
            else:
                assert u == cid // k
                i = cid % k
            assert tb == i * nt[u] // k
    return ref


def test_host_plans_follow_the_rule():
    rng = np.random.default_rng(77)
    for trial in range(600):
        P = int(rng.integers(1, 4))
        B = int(rng.integers(1, 90))
        S = int(rng.integers(1, 4))
        k = [0, 0, 0, 1, 2, 3][trial % 6]
        kind = trial % 5
        if kind == 0:
            lens = rng.integers(0, 40000, P * B)
        elif kind == 1:
            lens = np.exp(rng.uniform(np.log(16), np.log(9000), P * B)).astype(int)
        elif kind == 2:  # a few long ranges among many short ones
            lens = np.where(rng.random(P * B) < 0.1, rng.integers(30000, 200000, P * B),
                            rng.integers(0, 300, P * B))
        else:
            lens = np.full(P * B, int(rng.integers(0, 50000)))
        starts = rng.integers(0, 64, P * B).astype(np.int32)
        ends = (starts + lens).astype(np.int32)
        if trial % 11 == 0:  # an invalid range (end before start)
            ends[0] = starts[0] - 1
        check_table(starts.reshape(P, B), ends.reshape(P, B), P, S, k)


def test_worked_example():
    """Three ranges of 100, 10 and 50 tiles, one query: c0 = 4 (160 tiles
    over 256 workgroups, raised to the minimum), so the ranges take 25, 3
    and 13 chunks; the longest bucket holds every chunk of 4 tiles, the last
    bucket of range 1 (10 tiles in 3 pieces: 3, 3, 4) sits there too."""
    starts = np.zeros((1, 3), np.int32)
    ends = (np.array([[100, 10, 50]]) * TILE).astype(np.int32)
    ref = check_table(starts, ends, 1, 1, 0)
    assert ref.chunk_tiles == 4 and ref.chunks == 25 + 3 + 13 and ref.split_ranges == 3
    a = args_for(3, 1, 1)
    table, _ = L.mla_decode_partial_make_plan(a, starts, ends)
    ent = table[HEADER:HEADER + ENTRY * 41].reshape(41, ENTRY)
    # all pieces are 3 or 4 tiles, so all fall in the top bucket: range order
    assert list(ent[:, 0]) == [0] * 25 + [1] * 3 + [2] * 13
    assert list(ent[:, 3]) == list(range(41))


@pytest.mark.parametrize("over,code", [
    (dict(plan=FAKE + 0x48000000, plan_chunks=0), -4),
    (dict(plan=FAKE + 0x48000000, plan_chunks=1 << 20), -4),
    (dict(plan=FAKE + 0x48000000, plan_chunks=10, plan_split_units=11), -4),
    (dict(plan=FAKE + 0x48000000, plan_chunks=10, plan_split_units=-1), -4),
    (dict(plan=FAKE + 0x48000000 + 4, plan_chunks=10), -4),        # not 16-byte aligned
    (dict(plan=FAKE + 0x50000000, plan_chunks=10), -8),            # overlaps the output
    (dict(plan=FAKE + 0x48000000, plan_chunks=10, flags=L.MLA_FLAG_FORCE_SIMPLE), -6),
])
def test_plan_argument_validation(over, code):
    a = base_args(**over)
    assert L.lib().mla_decode_partial(ctypes.byref(a), None) == code


def test_plan_words_and_buffer_checks():
    a = base_args()
    words = L.mla_decode_partial_plan_words(a)
    U, S = a.P * a.B, a.S
    ref = L.mla_decode_partial_plan(a, np.zeros(U, np.int32), np.full(U, 64, np.int32))
    assert words == HEADER + ENTRY * ref.max_chunks + DESC * U
    # a set plan pointer does not change the size or the plan
    assert L.mla_decode_partial_plan_words(base_args(plan=FAKE, plan_chunks=3)) == words
    assert L.mla_decode_partial_plan_words(base_args(flags=L.MLA_FLAG_FORCE_SIMPLE)) == 0
    assert L.mla_decode_partial_plan_words(base_args(P=0)) == 0
    small = np.zeros(words - 1, np.int32)
    info = L.SplitInfo()
    rs, re_ = np.zeros(U, np.int32), np.full(U, 64, np.int32)
    i32p = lambda x: x.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))  # noqa: E731
    assert L.lib().mla_decode_partial_make_plan(ctypes.byref(a), i32p(rs), i32p(re_), i32p(small),
                                                words - 1, ctypes.byref(info)) == -5
    with pytest.raises(L.MLAError):
        L.mla_decode_partial_make_plan(base_args(flags=L.MLA_FLAG_FORCE_SIMPLE), rs, re_)
