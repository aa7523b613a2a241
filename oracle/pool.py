"""Oracle token-slot KV pool and scatter.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the native library and never imports it.

The pool holds one K row and one V row per token slot, each [Hkv, D].
RadixAttention keeps the KV of cached prefixes in such a pool so that later
requests can read it instead of recomputing it (unite.ai, "SGLang: Efficient
Execution of Structured Language Model Programs", section "Introduccion a
SGLang", RadixAttention bullet).  Scatter is the plain definition
pool[slots[i]] = new[i]; every other slot keeps what it held, and a slot
never written reads as NaN (poison), so a wrong gather surfaces as NaN.

Storage keeps each scattered block as given (float32 or bfloat16 CPU
tensors) and an index slot -> (block, row); gather converts the rows it
returns to float64 exactly.
"""
from __future__ import annotations

import numpy as np
import torch


class OraclePool:
    def __init__(self, pool_slots: int, hkv: int, d: int):
        self.P, self.hkv, self.d = int(pool_slots), hkv, d
        self.blk = np.full(self.P, -1, dtype=np.int64)
        self.row = np.zeros(self.P, dtype=np.int64)
        self.blocks = []

    def gather(self, slots):
        """(K, V) float64 arrays [len(slots), Hkv, D]; NaN for unwritten slots."""
        slots = np.asarray(slots, dtype=np.int64)
        K = np.full((slots.shape[0], self.hkv, self.d), np.nan)
        V = np.full((slots.shape[0], self.hkv, self.d), np.nan)
        if slots.shape[0] == 0:
            return K, V
        b = self.blk[slots]
        for bi in np.unique(b):
            if bi < 0:
                continue
            sel = np.nonzero(b == bi)[0]
            rows = torch.from_numpy(self.row[slots[sel]])
            kb, vb = self.blocks[bi]
            K[sel] = kb[rows].to(torch.float64).numpy()
            V[sel] = vb[rows].to(torch.float64).numpy()
        return K, V


def scatter(pool: OraclePool, slots, k_new, v_new):
    """pool[slots[i]] = (k_new[i], v_new[i]) for every i."""
    slots = np.asarray(slots, dtype=np.int64)
    k_new = torch.as_tensor(k_new).detach().cpu()
    v_new = torch.as_tensor(v_new).detach().cpu()
    assert k_new.shape[0] == slots.shape[0] == v_new.shape[0]
    if slots.shape[0] == 0:
        return
    pool.blocks.append((k_new, v_new))
    pool.blk[slots] = len(pool.blocks) - 1
    pool.row[slots] = np.arange(slots.shape[0])
