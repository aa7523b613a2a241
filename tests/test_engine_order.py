"""Host rule of the engine's extend work order (CPU only; the GPU test
shows the order changes the schedule, never the outputs): a permutation;
longest first (ties in batch order) when the kv heads are a multiple of the
8 XCDs; otherwise the sorted requests dealt back and forth over 8 bins, so
each contiguous eighth of the order gets one of the 8 longest and is
itself longest first."""
import numpy as np
import pytest

from prefix_shared_kv_host_amd.engine import RadixKVCache


def order_for(hkv, lens):
    c = RadixKVCache.__new__(RadixKVCache)      # the rule needs no pool
    c.hkv = hkv
    return c.extend_order(np.asarray(lens))


@pytest.mark.parametrize("B", [1, 7, 8, 16, 64, 100])
def test_longest_first_on_whole_heads(B):
    lens = np.random.default_rng(B).integers(1, 50, B)
    for hkv in (8, 16, 32):
        o = order_for(hkv, lens)
        assert sorted(o.tolist()) == list(range(B))
        assert np.all(np.diff(lens[o]) <= 0)
        for i in range(B - 1):                   # ties keep batch order
            if lens[o[i]] == lens[o[i + 1]]:
                assert o[i] < o[i + 1]


@pytest.mark.parametrize("B", [8, 16, 48, 64])
def test_dealt_over_xcds_otherwise(B):
    lens = np.random.default_rng(100 + B).permutation(B) + 1      # distinct lengths 1..B
    for hkv in (1, 2, 4, 12):
        o = order_for(hkv, lens)
        assert sorted(o.tolist()) == list(range(B))
        bins = np.array_split(lens[o], 8)                          # B is a multiple of 8 here
        top8 = set(range(B - 7, B + 1))
        assert sorted(int(b[0]) for b in bins) == sorted(top8)     # one of the 8 longest leads each
        for b in bins:
            assert np.all(np.diff(b) < 0)                          # longest first within it
        sums = [int(b.sum()) for b in bins]
        assert max(sums) - min(sums) <= B                          # the snake keeps the bins even
