"""Adapter giving the native tree (through the ctypes binding) the same
Python API as the oracle tree, for lockstep comparisons."""
import numpy as np

from prefix_shared_kv_host_amd import rkv


class NativeTree:
    def __init__(self, pool_slots, initial_free=None):
        self.t = rkv.Tree(pool_slots, initial_free)

    def match(self, tok):
        return self.t.radix_match(tok)

    def lock(self, nid):
        return self.t.radix_lock(nid)

    def unlock(self, nid):
        return self.t.radix_unlock(nid)

    def insert(self, tok, slots):
        return self.t.radix_insert(tok, slots)

    def evict(self, want):
        return self.t.radix_evict(want)

    def alloc(self, n):
        return self.t.alloc(n)

    def free(self, slots):
        return self.t.free(slots)

    def serialize(self):
        return self.t.radix_serialize()

    def stats(self):
        return self.t.stats()

    def free_list(self):
        return self.t.free_list()

    def batch_prepare(self, seqs, ld=None):
        code, tb = self.t.batch_prepare(seqs, ld)
        if tb is None:
            return code, None
        out = dict(req_to_token=tb["req_to_token"].tolist(), prefix_lens=tb["prefix_lens"].tolist(),
                   seq_lens=tb["seq_lens"].tolist(), qo_indptr=tb["qo_indptr"].tolist(),
                   new_slots=tb["new_slots"].tolist(), nodes=tb["nodes"].tolist())
        return code, out

    def batch_commit(self, seqs, req_to_token, nodes):
        return self.t.batch_commit(seqs, req_to_token, nodes)

    def batch_append(self, req_to_token, seq_lens):
        """Same in-place list semantics as the oracle's batch_append."""
        r2t = np.ascontiguousarray(np.asarray(req_to_token, dtype=np.int32))
        sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
        try:
            code, ns = self.t.batch_append(r2t, sl)
        except rkv.RkvError as e:
            return e.code, None
        if ns is None:
            return code, None
        for r in range(len(seq_lens)):
            req_to_token[r][:] = r2t[r].tolist()
            seq_lens[r] = int(sl[r])
        return code, ns.tolist()
