"""Native radix tree + allocator vs the oracle, bit-exact: op-for-op on
seeded random streams (outputs, free-list order and canonical dumps after
every op), the walkthrough, and whole workload traces through
batch_prepare / batch_commit.  CPU only (host code of librkv)."""
import numpy as np
import pytest

from inputs import configs
from oracle.radix import OracleTree
from tests import radix_ops, walkthrough
from tests.native_tree import NativeTree


@pytest.mark.parametrize("seed,vocab", [(1, 2), (2, 3), (3, 4), (4, 2), (5, 3)])
def test_native_matches_oracle_op_by_op(seed, vocab):
    P = 48
    perm = np.random.default_rng(100 + seed).permutation(P).tolist()
    c = radix_ops.drive([OracleTree(P, perm), NativeTree(P, perm)], seed, 20000, P, vocab, 12)
    assert c["split"] > 50 and c["evicted_nodes"] > 200


def test_native_walkthrough():
    walkthrough.run(lambda P: NativeTree(P))


def _replay(name, limit=None):
    shape, phases = configs.build(name)
    perm = configs.free_list(shape.pool, shape.seed)
    trees = [OracleTree(shape.pool, perm), NativeTree(shape.pool, perm)]
    for i, ph in enumerate(phases[:limit]):
        res = [t.batch_prepare(ph.seqs) for t in trees]
        assert res[0][0] == res[1][0] == 0, (name, i)
        a, b = res[0][1], res[1][1]
        for key in ("prefix_lens", "seq_lens", "qo_indptr", "new_slots", "nodes"):
            assert list(a[key]) == list(b[key]), (name, i, key)
        for r in range(len(ph.seqs)):
            assert list(a["req_to_token"][r]) == list(b["req_to_token"][r]), (name, i, r)
        for t, (_, tb) in zip(trees, res):
            assert t.batch_commit(ph.seqs, tb["req_to_token"], tb["nodes"]) == 0
        assert trees[0].stats() == trees[1].stats(), (name, i)
        assert trees[0].free_list() == trees[1].free_list(), (name, i)
    assert trees[0].serialize() == trees[1].serialize()
    return trees[0]


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c3ns", "c4"])
def test_workload_tables_bit_exact(name):
    _replay(name)


@pytest.mark.parametrize("name", ["c5", "c5e"])
def test_chat_trace_tables_bit_exact(name):
    t = _replay(name)
    s = t.stats()
    if name == "c5e":
        assert s[7] > 100000      # the 2^19 pool really evicts
    else:
        assert s[7] == 0          # the 2^21 pool never binds


def test_token_batch_equals_lists():
    """Token ids given as an rkv.TokenBatch (one int32 array and offsets)
    produce the same tables, tree and free list as the same ids as lists."""
    import numpy as np
    from inputs import configs
    from prefix_shared_kv_host_amd import rkv
    s, phases = configs.build("c2")
    a = rkv.Tree(4096 * 64, None)
    b = rkv.Tree(4096 * 64, None)
    for ph in phases:
        seqs = [x[:200] for x in ph.seqs[:16]]
        tk = rkv.TokenBatch(seqs)
        assert len(tk) == len(seqs) and tk.flat.dtype == np.int32
        ca, ta = a.batch_prepare(seqs)
        cb, tbb = b.batch_prepare(tk)
        assert ca == cb == rkv.OK
        for key in ("req_to_token", "prefix_lens", "seq_lens", "qo_indptr", "new_slots"):
            assert np.array_equal(ta[key], tbb[key]), key
        a.batch_commit(seqs, ta["req_to_token"], ta["nodes"])
        b.batch_commit(tk, tbb["req_to_token"], tbb["nodes"])
        assert a.radix_serialize() == b.radix_serialize()


@pytest.mark.parametrize("nreq", [0, 1, 5, 16])
def test_prepare_into_caller_buffer(nreq):
    """batch_prepare(out=...) writes every int32 table into one caller buffer
    of exactly table_words words, in the documented order, and nothing past
    it (a guard word after the buffer keeps its value); the tables equal
    those of a call that allocates its own."""
    from prefix_shared_kv_host_amd import rkv
    s, phases = configs.build("c2")
    a = rkv.Tree(4096 * 64, None)
    b = rkv.Tree(4096 * 64, None)
    for ph in phases:
        seqs = [x[:150] for x in ph.seqs[:nreq]]
        B = len(seqs)
        ld = max((len(x) for x in seqs), default=1)
        cap = sum(len(x) for x in seqs)
        n = rkv.Tree.table_words(max(B, 1), ld, max(cap, 1))
        store = np.full(n + 1, -7, dtype=np.int32)
        ca, ta = a.batch_prepare(seqs)
        cb, tb = b.batch_prepare(rkv.TokenBatch(seqs), ld=ld, out=store[:n])
        assert ca == cb == rkv.OK
        assert store[n] == -7
        for key in ("req_to_token", "prefix_lens", "seq_lens", "qo_indptr", "new_slots"):
            assert np.array_equal(ta[key], tb[key]), key
        Bx = max(B, 1)
        T = int(tb["qo_indptr"][B])
        flat = np.concatenate([store[:Bx * ld].reshape(Bx, ld)[:B].ravel(), store[Bx * ld:Bx * ld + Bx][:B],
                               store[Bx * ld + Bx:Bx * ld + 2 * Bx][:B],
                               store[Bx * ld + 2 * Bx:Bx * ld + 3 * Bx + 1][:B + 1],
                               store[Bx * ld + 3 * Bx + 1:][:T]])
        ref = np.concatenate([ta["req_to_token"].ravel(), ta["prefix_lens"], ta["seq_lens"],
                              ta["qo_indptr"], ta["new_slots"]])
        assert np.array_equal(flat, ref)
        a.batch_commit(seqs, ta["req_to_token"], ta["nodes"])
        b.batch_commit(seqs, tb["req_to_token"], tb["nodes"])
        assert a.radix_serialize() == b.radix_serialize()
    with pytest.raises(rkv.RkvError):
        b.batch_prepare([[1, 2, 3]], out=np.zeros(2, dtype=np.int32))
