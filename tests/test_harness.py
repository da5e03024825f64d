"""The parity harness's own helpers, on the CPU: the oracle run over disjoint
frame ranges and summed equals one run over all frames, and the hash-table
layout check accepts a table filled by linear probing in any order and
rejects a damaged one."""
import numpy as np
import pytest

import oracle
from hash_table_amd import scenes
from tests import parity


@pytest.fixture(scope="module", autouse=True)
def built_oracle():
    oracle.build()


def test_summed_ranges_equal_one_run():
    wl = scenes.workload("spherewall320x240")
    frames, summed = parity.oracle_ranges("spherewall320x240", 10, workers=3)
    assert [scenes.frame_digest([f]) for f in frames] == [scenes.frame_digest([wl.frame(i)]) for i in range(10)]
    one = parity.oracle_integrate(frames, wl.voxel_size, wl.trunc, wl.pool_capacity)
    assert np.array_equal(summed.block_coords(), one.block_coords())
    a, b = summed.block_sums(one.block_coords()), one.block_sums(one.block_coords())
    assert np.array_equal(a["weight"], b["weight"])
    for k in ("tsdf", "r", "g", "b"):
        assert np.abs(a[k] - b[k]).max() < 1e-9
    t1, t2 = summed.totals(), one.totals()
    for k in ("blocks", "points_valid", "voxel_updates", "frames", "update_misses", "pool_overflow"):
        assert t1[k] == t2[k], k
    missing = summed.block_sums(np.array([[10 ** 5, 0, 0]], np.int32))
    assert np.isnan(missing["weight"]).all()


def _probe_fill(keys, T, rng):
    """A table of T entries filled by linear probing in a random key order."""
    table = np.full((T, 2), np.uint64(0xFFFFFFFFFFFFFFFF), np.uint64)
    home = (parity.fmix64(keys) & np.uint64(T - 1)).astype(np.int64)
    for n, i in enumerate(rng.permutation(len(keys))):
        p = int(home[i])
        while table[p, 0] != np.uint64(0xFFFFFFFFFFFFFFFF):
            p = (p + 1) % T
        table[p, 0] = keys[i]
        table[p, 1] = np.uint64(n)
    return table


def test_table_layout_check():
    rng = np.random.default_rng(5)
    coords = np.unique(rng.integers(-50, 50, size=(700, 3)), axis=0).astype(np.int32)
    keys = parity._pack(coords).astype(np.uint64)
    T = 1024
    for seed in range(3):                         # any insertion order gives the same layout
        table = _probe_fill(keys, T, np.random.default_rng(seed))
        assert parity.table_layout_failures(table, coords, len(coords)) == []
    # a key moved one slot on into a free slot (a probe that skipped a slot)
    table = _probe_fill(keys, T, rng)
    empty = np.nonzero(table[:, 0] == np.uint64(0xFFFFFFFFFFFFFFFF))[0]
    e = int(empty[len(empty) // 2])
    p = (e - 1) % T
    assert table[p, 0] != np.uint64(0xFFFFFFFFFFFFFFFF)
    bad = table.copy()
    bad[e], bad[p] = table[p], table[e]
    assert parity.table_layout_failures(bad, coords, len(coords)) != []
    # a missing key, a duplicated pool index
    bad = table.copy()
    bad[np.nonzero(bad[:, 0] != np.uint64(0xFFFFFFFFFFFFFFFF))[0][0], 0] = np.uint64(0xFFFFFFFFFFFFFFFF)
    assert parity.table_layout_failures(bad, coords, len(coords)) != []
    bad = table.copy()
    occ = np.nonzero(bad[:, 0] != np.uint64(0xFFFFFFFFFFFFFFFF))[0]
    bad[occ[1], 1] = bad[occ[0], 1]
    assert parity.table_layout_failures(bad, coords, len(coords)) != []


def test_fmix64_known_values():
    # MurmurHash3's fmix64: 0 stays 0; values computed by hand from its definition
    assert int(parity.fmix64(np.array([0], np.uint64))[0]) == 0
    k = 1
    k ^= k >> 33
    k = (k * 0xFF51AFD7ED558CCD) & (2 ** 64 - 1)
    k ^= k >> 33
    k = (k * 0xC4CEB9FE1A85EC53) & (2 ** 64 - 1)
    k ^= k >> 33
    assert int(parity.fmix64(np.array([1], np.uint64))[0]) == k
