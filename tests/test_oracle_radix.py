"""Pins for the oracle radix tree: brute-force longest common prefix, the LRU
rule checked on every eviction, structure and slot conservation.  CPU only."""
import numpy as np
import pytest

from oracle.radix import EBUSY, EINVAL, ENOSPC, OK, OracleTree
from tests import radix_ops


@pytest.mark.parametrize("seed,vocab", [(1, 2), (2, 3), (3, 4), (4, 2), (5, 3)])
def test_oracle_tree_vs_brute_force(seed, vocab):
    P = 48
    perm = np.random.default_rng(seed).permutation(P).tolist()
    c = radix_ops.drive([OracleTree(P, perm)], seed, 20000, P, vocab, 12)
    # the stream really exercised splits and multi-node evictions
    assert c["split"] > 50 and c["evicted_nodes"] > 200 and c["insert"] > 1000


def test_error_paths():
    t = OracleTree(8)
    assert t.alloc(9)[0] == ENOSPC and len(t.free_list()) == 8
    assert t.unlock(0) == OK            # the root carries no lock
    st, sl = t.alloc(4)
    assert t.insert([1, 2, 3, 4], sl) == 0
    m, _, nid = t.match([1, 2, 3, 4])
    assert t.unlock(nid) == EINVAL      # lock count would go negative
    assert t.lock(nid) == OK
    st, freed = t.evict(1)
    assert st == EBUSY and freed == 0   # the only leaf is locked
    assert t.lock(12345) == EINVAL
    assert t.insert([1, 2], [0]) == EINVAL
    assert t.batch_prepare([[]])[0] == EINVAL


def test_planted_tie_break_mistake_is_caught(monkeypatch):
    """An eviction that picks the most recent leaf must fail the LRU check."""
    def mru_evict(self, want):
        freed = 0
        while freed < want:
            cands = [n for n in self.nodes.values()
                     if n is not self.root and not n.children and n.lock == 0]
            if not cands:
                return EBUSY, freed
            best = max(cands, key=lambda n: (n.last_access, n.id))
            self.fifo.extend(best.slots)
            freed += len(best.slots)
            best.parent.children.remove(best)
            del self.nodes[best.id]
        return OK, freed
    monkeypatch.setattr(OracleTree, "evict", mru_evict)
    with pytest.raises(AssertionError):
        radix_ops.drive([OracleTree(48)], 3, 3000, 48, 3, 12)


def test_planted_duplicate_slot_mistake_is_caught(monkeypatch):
    """An insert that overwrites cached slots with the caller's must fail."""
    real = OracleTree.insert

    def bad(self, tok, slots):
        m = real(self, tok, slots)
        node, mm, _, path = self._walk(list(tok))
        pos = 0
        for n in path[1:]:
            n.slots = list(slots[pos:pos + len(n.label)])
            pos += len(n.label)
        return m
    monkeypatch.setattr(OracleTree, "insert", bad)
    with pytest.raises(AssertionError):
        radix_ops.drive([OracleTree(48)], 4, 3000, 48, 2, 12)
