"""Seeded input generator: determinism, rounding, layout."""
import numpy as np
import pytest
import torch

from mla_split_kv_absorbed_amd import workloads as W


def test_same_seed_same_bytes():
    a = W.make_workload(W.spec(3, B=3, lengths=("uniform", 40, 100)))
    b = W.make_workload(W.spec(3, B=3, lengths=("uniform", 40, 100)))
    for name in ("w_uk", "w_uv", "q_nope", "q_rope", "kv", "block_table", "cur_kv",
                 "range_start", "range_end", "lengths"):
        x, y = getattr(a, name), getattr(b, name)
        assert x.tobytes() == y.tobytes(), name


@pytest.mark.parametrize("dtype,tdt", [("bf16", torch.bfloat16), ("f16", torch.float16)])
def test_rounding_matches_torch_on_fp32_inputs(dtype, tdt):
    # fp32 inputs: torch's fp32 -> half conversions are single RNE roundings
    r = np.random.Generator(np.random.PCG64(3))
    x = (r.standard_normal(200000) * np.exp(r.uniform(-20, 8, 200000))).astype(np.float32)
    x = np.concatenate([x, np.float32([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 0.0])])
    ours = W.round_to(x.astype(np.float64), dtype)
    ref = torch.from_numpy(x).to(tdt).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_bf16_storage_roundtrip():
    r = np.random.Generator(np.random.PCG64(4))
    v = W.round_to(r.standard_normal(10000), "bf16")
    assert np.array_equal(W.from_storage(W.to_storage(v, "bf16"), "bf16"), v)


def test_paged_layout_and_poison():
    w = W.make_workload(W.spec(4, B=5, lengths=("loguniform", 70, 300)), extra_blocks=3)
    bs = w.spec.block_size
    nblk = -(-w.lengths // bs)
    used = set()
    for b in range(5):
        ids = w.block_table[b, :nblk[b]]
        assert np.all(ids >= 0) and np.all(w.block_table[b, nblk[b]:] == -1)
        used.update(ids.tolist())
        rows = w.seq_rows64(b)
        assert rows.shape == (w.lengths[b], 576) and np.all(np.isfinite(rows))
        rem = w.lengths[b] % bs
        if rem:
            tail = w.kv[ids[-1], rem:].astype(np.float64)
            assert np.all(np.isnan(tail))
    assert len(used) == int(nblk.sum())
    unused = sorted(set(range(w.kv.shape[0])) - used)
    assert len(unused) == 3 and np.all(np.isnan(w.kv[unused].astype(np.float64)))


def test_part_ranges_block_aligned_and_cover():
    L = np.array([32768, 100, 33, 0, 64])
    st, en = W.part_ranges(L, 8, 32)
    assert st.shape == (8, 5)
    for b in range(5):
        assert st[0, b] == 0 and en[-1, b] == L[b]
        assert np.all(st[1:, b] == en[:-1, b])
        assert np.all(st[:, b] % 32 == 0)
    # 32768 tokens into 8 parts -> 8 x 4096
    assert np.all(en[:, 0] - st[:, 0] == 4096)


def test_full_size_shapes_without_drawing_cache():
    sp = W.SPECS[2]
    assert (sp.B, sp.H, sp.S, sp.block_size, sp.parts) == (32, 128, 1, 32, 8)
    r = np.random.Generator(np.random.PCG64(1003))
    L = W.draw_lengths(r, W.SPECS[3])
    assert L.min() >= 1024 and L.max() <= 16384 and len(L) == 64
    r = np.random.Generator(np.random.PCG64(1004))
    L = W.draw_lengths(r, W.SPECS[4])
    assert L.min() >= 512 and L.max() <= 8192 and len(L) == 128


def test_cut_ranges_tiles_each_range_exactly():
    """The library's range cut (mla_cut_ranges, the pieces num_splits = k
    makes): k pieces per range, in order, disjoint, covering the range, with
    inner boundaries on 32-key tiles, piece i holding tiles
    [i nt / k, (i + 1) nt / k); empty ranges give empty pieces."""
    import numpy as np
    from mla_split_kv_absorbed_amd import _lib as L
    cut_ranges = L.mla_cut_ranges
    rng = np.random.default_rng(5)
    st = rng.integers(0, 300, 64)
    en = st + rng.integers(0, 900, 64)
    st[:2], en[:2] = 100, 100          # empty ranges
    st[2], en[2] = 0, 4096             # aligned
    for k in (1, 2, 3, 8):
        ps, pe = cut_ranges(st, en, k)
        assert ps.shape == (k, 64) and pe.shape == (k, 64)
        for j in range(64):
            a, e = int(st[j]), int(en[j])
            if e <= a:
                assert np.all(ps[:, j] == a) and np.all(pe[:, j] == a)
                continue
            nt = (e - 1) // 32 - a // 32 + 1
            covered = []
            for i in range(k):
                assert ps[i, j] <= pe[i, j]
                tiles = (i + 1) * nt // k - i * nt // k
                if tiles == 0:
                    assert ps[i, j] == pe[i, j]
                    continue
                covered.append((int(ps[i, j]), int(pe[i, j])))
                first_tile = ps[i, j] // 32 if ps[i, j] != a else a // 32
                assert (pe[i, j] - 1) // 32 - first_tile + 1 == tiles
                if ps[i, j] != a:
                    assert ps[i, j] % 32 == 0
            # the non-empty pieces tile [a, e) in order
            assert covered[0][0] == a and covered[-1][1] == e
            for (s0, e0), (s1, e1) in zip(covered, covered[1:]):
                assert e0 == s1


def test_cut_ranges_rejects_invalid_ranges():
    import numpy as np
    import pytest
    from mla_split_kv_absorbed_amd import _lib as L
    with pytest.raises(L.MLAError):
        L.mla_cut_ranges(np.array([5]), np.array([4]), 2)
    with pytest.raises(L.MLAError):
        L.mla_cut_ranges(np.array([-1]), np.array([4]), 2)
