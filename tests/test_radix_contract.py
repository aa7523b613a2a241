"""Error paths of the host tree's slot contract (CPU only): insert, commit and
free reject slots the caller does not hold, repeated slots and unlocks the
batch's locks do not cover, and a rejected call leaves the tree, the free
list and the stats exactly as they were."""
import numpy as np
import pytest

from prefix_shared_kv_host_amd import rkv


def snapshot(t):
    return t.radix_serialize(), t.free_list(), t.stats()


def expect_einval(t, fn):
    before = snapshot(t)
    try:
        code = fn()
    except rkv.RkvError as e:
        code = e.code
    assert code == rkv.EINVAL
    assert snapshot(t) == before


def tree_with_one_sequence(pool=16):
    t = rkv.Tree(pool)
    st, sl = t.alloc(4)
    assert st == rkv.OK and t.radix_insert([1, 2, 3, 4], sl) == 0
    return t, sl


def test_insert_rejects_free_slots_before_overrunning_the_fifo():
    # The tree holds 4 slots and the FIFO the other 12.  An insert of the
    # same tokens with slots that are already free would push each of them
    # to the FIFO again: 16 entries into a 16-slot ring that holds 12.
    t, sl = tree_with_one_sequence()
    foreign = t.free_list()[:4]
    expect_einval(t, lambda: t.radix_insert([1, 2, 3, 4], foreign))
    # the tree's own slots at their own positions are fine (nothing pushed)
    assert t.radix_insert([1, 2, 3, 4], sl) == 4
    assert len(t.free_list()) == 12


def test_insert_rejects_repeated_or_misplaced_slots():
    t, sl = tree_with_one_sequence()
    st, mine = t.alloc(2)
    assert st == rkv.OK
    expect_einval(t, lambda: t.radix_insert([7, 8], [mine[0], mine[0]]))   # a caller slot twice
    expect_einval(t, lambda: t.radix_insert([7, 8], [mine[0], sl[0]]))     # a tree slot elsewhere
    expect_einval(t, lambda: t.radix_insert([1, 2, 9], [sl[1], sl[0], mine[0]]))   # tree slots swapped
    assert t.radix_insert([1, 2, 9], [sl[0], mine[0], mine[1]]) == 2       # a differing duplicate goes back
    assert t.free_list()[-1] == mine[0]


def test_free_rejects_slots_the_caller_does_not_hold():
    t, sl = tree_with_one_sequence()
    st, mine = t.alloc(2)
    expect_einval(t, lambda: t.free([sl[0]]))               # owned by the tree
    expect_einval(t, lambda: t.free([t.free_list()[0]]))    # already free
    expect_einval(t, lambda: t.free([mine[0], mine[0]]))    # repeated
    assert t.free(mine) == rkv.OK
    assert t.free_list()[-2:] == mine


def prepared(t, seqs):
    code, tb = t.batch_prepare(seqs)
    assert code == rkv.OK
    return tb


def test_commit_checks_locks_before_inserting_anything():
    t = rkv.Tree(64)
    tb0 = prepared(t, [[5, 6, 7, 8]])
    assert t.batch_commit([[5, 6, 7, 8]], tb0["req_to_token"], tb0["nodes"]) == rkv.OK
    seqs = [[1, 2, 3], [5, 6, 7, 9]]
    tb = prepared(t, seqs)
    assert tb["nodes"][1] != 0
    # request 1's lock is dropped by hand: the commit must fail before it
    # inserts request 0 (the old code inserted request 0 first)
    assert t.radix_unlock(int(tb["nodes"][1])) == rkv.OK
    expect_einval(t, lambda: t.batch_commit(seqs, tb["req_to_token"], tb["nodes"]))
    assert t.radix_lock(int(tb["nodes"][1])) == rkv.OK
    assert t.batch_commit(seqs, tb["req_to_token"], tb["nodes"]) == rkv.OK


def test_commit_counts_unlocks_per_node_across_the_batch():
    t = rkv.Tree(64)
    tb0 = prepared(t, [[5, 6, 7, 8]])
    assert t.batch_commit([[5, 6, 7, 8]], tb0["req_to_token"], tb0["nodes"]) == rkv.OK
    seqs = [[5, 6, 7, 1], [5, 6, 7, 2]]
    tb = prepared(t, seqs)
    node = int(tb["nodes"][0])
    assert node == int(tb["nodes"][1]) and node != 0       # both locked the same path once each
    # naming the node a third time asks for one unlock more than its count
    r2t = np.vstack([tb["req_to_token"], tb["req_to_token"][:1]])
    nodes = np.array([node, node, node], dtype=np.int64)
    expect_einval(t, lambda: t.batch_commit(seqs + [seqs[0]], r2t, nodes))
    assert t.batch_commit(seqs, tb["req_to_token"], tb["nodes"]) == rkv.OK
    assert t.stats()[3] == 0                                # nothing left locked


def test_commit_rejects_foreign_and_repeated_slots():
    t = rkv.Tree(64)
    seqs = [[1, 2, 3, 4], [1, 2, 3, 5]]
    tb = prepared(t, seqs)
    free_slot = t.free_list()[0]
    bad = tb["req_to_token"].copy()
    bad[1, 3] = free_slot                                   # not the caller's
    expect_einval(t, lambda: t.batch_commit(seqs, bad, tb["nodes"]))
    bad = tb["req_to_token"].copy()
    bad[1, 3] = bad[0, 3]                                   # one new slot in two requests
    expect_einval(t, lambda: t.batch_commit(seqs, bad, tb["nodes"]))
    # the good commit: request 1 matches request 0's new slots for its first
    # three positions and hands its own three back
    own = tb["req_to_token"][1, :3].tolist()
    assert t.batch_commit(seqs, tb["req_to_token"], tb["nodes"]) == rkv.OK
    assert t.free_list()[-3:] == own


def test_commit_after_append_rejects_stale_sequences():
    """A decode loop's appended slots enter the tree only through a commit
    of the grown sequences; the engine refuses the prepared ones."""
    from prefix_shared_kv_host_amd.engine import Batch, RadixKVCache
    t = rkv.Tree(64)
    seqs = [[1, 2, 3], [4, 5]]
    code, tb = t.batch_prepare(seqs, ld=8)
    assert t.batch_append(tb["req_to_token"], tb["seq_lens"])[0] == rkv.OK
    cache = RadixKVCache.__new__(RadixKVCache)
    cache.tree = t
    batch = Batch(seqs=rkv.TokenBatch(seqs), host=tb, req_to_token=None, qo_indptr=None, prefix_lens=None,
                  seq_lens=None, new_slots=None, max_new=1, max_len=4, total_new=2)
    with pytest.raises(ValueError):
        cache.commit(batch)
    cache.commit(batch, [s + [9] for s in seqs])
    st = t.stats()
    assert st[0] + st[1] == 64                              # every slot cached or free: nothing leaked
