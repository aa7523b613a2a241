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


class _Pool:
    def __init__(self, dtype):
        self.dtype = dtype


def splits_for(hq, hkv, lens, dtype="bf16"):
    import torch
    from types import SimpleNamespace
    c = RadixKVCache.__new__(RadixKVCache)
    c.hkv = hkv
    c.k_pool = _Pool(torch.bfloat16 if dtype == "bf16" else torch.float32)
    b = SimpleNamespace(host={"seq_lens": np.asarray(lens, dtype=np.int32)})
    return c.decode_splits(b, hq)


def test_plain_decode_splits_rule():
    """Plain decode keeps 768-key chunks (num_splits 0) unless the grouped-head
    kernel would get fewer than 1024 items; then enough splits for 1024 items,
    never chunks below 256 keys, and only when that is more splits than the
    longest request already has."""
    rng = np.random.default_rng(7)
    long_ = rng.integers(2049, 8193, 64)
    assert splits_for(64, 8, long_) == 0             # 64 x 8 heads: thousands of items already
    assert splits_for(8, 1, long_) == 16             # one GPU's 8/1-head share: 16 splits -> 1024 items
    assert splits_for(32, 32, long_) == 0            # multi-head: the vector kernel
    assert splits_for(8, 1, long_, "f32") == 0       # fp32: the vector kernel
    assert splits_for(8, 1, [300] * 4) == 0          # 256-key chunks would give 2 splits, no more than 768's 1
    assert splits_for(8, 1, [4096] * 4) == 16        # 4 x 16 = 64 items, capped by 4096 / 256 = 16
    ns = splits_for(8, 1, [2000] * 8)
    assert ns == 2000 // 256 and ns > -(-2000 // 768)
    assert splits_for(8, 1, []) == 0


def plan_for(hkv, hq, lens, shared=2048, **kw):
    """The engine's host plan for requests whose first `shared` keys are one
    run of slots and whose other keys are private."""
    from types import SimpleNamespace
    c = RadixKVCache.__new__(RadixKVCache)      # the rule needs no pool
    c.hkv, c.d = hkv, 128
    lens = np.asarray(lens, dtype=np.int32)
    ld = int(lens.max())
    rows = np.zeros((len(lens), ld), dtype=np.int32)
    nxt = shared
    for r, n in enumerate(lens):
        rows[r, :shared] = np.arange(shared)
        rows[r, shared:n] = np.arange(nxt, nxt + n - shared)
        nxt += n - shared
    b = SimpleNamespace(host={"req_to_token": rows, "seq_lens": lens})
    return c.cascade_plan_host(b, hq, **kw), rows, lens


def test_cascade_chunk_rule():
    """The prefix-shared plan cuts shared runs into chunks of the tail chunk
    (768 keys), and into 256-key chunks when the tail chunk is halved for a
    launch of fewer than 1024 grouped-head tail items; chunks given by the
    caller are kept.  The plan is the planner's own for the chosen chunks."""
    from prefix_shared_kv_host_amd import rkv
    lens = np.random.default_rng(7).integers(2049, 8193, 64)
    for hkv, hq, tc, sc in ((8, 64, 768, 768), (1, 8, 384, 256), (32, 32, 768, 768), (1, 1, 768, 768)):
        p, rows, L = plan_for(hkv, hq, lens)
        assert (p.tail_chunk, p.seg_chunk) == (tc, sc), (hkv, hq)
        ref = rkv.cascade_plan(rows, L, sc, tc, 32, rkv.cascade_max_members(hq, hkv, 128))
        for k in ("perm", "rec_indptr", "tail_begin", "jobs"):
            assert np.array_equal(getattr(p, k), getattr(ref, k)), (hkv, hq, k)
        assert p.n_jobs and int((p.jobs[:, 1] - p.jobs[:, 0]).max()) <= sc
        assert np.all(p.tail_begin == 2048)
        q, _, _ = plan_for(hkv, hq, lens, seg_chunk=100)
        assert q.seg_chunk == 100 and q.tail_chunk == tc
        assert np.array_equal(q.tail_begin, p.tail_begin)    # where tails start depends on neither chunk


def test_cascade_tail_order():
    """The prefix-shared plan hands out the requests' tail splits longest
    first (split length as the kernels cut it: the tail in ceil(tail /
    tail_chunk) equal splits rounded up to 64 keys, never above tail_chunk),
    ties in batch order, when each XCD's contiguous range of tail items is
    whole head blocks (64/8 and 32/32 heads); otherwise (one kv head) the
    sorted requests are dealt over the 8 ranges, each longest first and of
    about equal total.  Off on request, for a single request and for
    launches of fewer than 1024 tail items (the 8/1-head share)."""
    lens = np.random.default_rng(11).integers(2049, 8193, 64)
    small, _, _ = plan_for(1, 8, lens)
    assert small.tail_chunk == 384 and small.tail_order is None
    for hkv, hq, whole, B in ((8, 64, True, 64), (1, 8, False, 512), (32, 32, True, 64)):
        lens = np.random.default_rng(11).integers(2049, 8193, B)
        p, _, L = plan_for(hkv, hq, lens)
        o = p.tail_order
        assert o is not None and sorted(o.tolist()) == list(range(len(L)))
        tails = L.astype(np.int64) - p.tail_begin
        n = -(-tails // p.tail_chunk)
        split = np.minimum(np.minimum(-(-(-(-tails // n)) // 64) * 64, p.tail_chunk), tails)
        runs = [o] if whole else np.array_split(o, 8)
        for run in runs:
            for i in range(len(run) - 1):
                a, b = split[run[i]], split[run[i + 1]]
                assert a > b or (a == b and run[i] < run[i + 1])
        if not whole:
            sums = [int(split[run].sum()) for run in runs]
            assert max(sums) - min(sums) <= int(split.max())
        off, _, _ = plan_for(hkv, hq, lens, longest_tails_first=False)
        assert off.tail_order is None
    one, _, _ = plan_for(8, 64, lens[:1])
    assert one.tail_order is None
