"""Run a synthetic workload through the oracle tree, pool and attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.

For each batch: prepare (match capped at length-1, lock, evict if short,
allocate, fill index tables), scatter the new tokens' K/V into the oracle
pool, attend (extend or decode), commit (insert + unlock).  This is the
request flow of RadixAttention's walkthrough (unite.ai, "SGLang: Efficient
Execution of Structured Language Model Programs", section "SGLang: Modelo de
programacion y metodologia", Steps 2-9): a request reuses its cached prefix,
its new tokens are computed, and the finished sequence goes into the tree.

Content rows come from the shared input generator (`inputs.content`).
"""
from __future__ import annotations

import numpy as np

from inputs import configs as _cfg
from inputs import content as _content

from .attention import decode, extend
from .pool import OraclePool, scatter
from .radix import OK, OracleTree


def run(shape, phases, attend=True, requests_of=None, device="cpu", keep=None):
    """Returns a list with one dict per phase: the tables, and for extend /
    decode phases the float64 outputs o, lse (NaN rows for requests not
    selected by requests_of(phase_index, B) when that is given)."""
    tree = OracleTree(shape.pool, _cfg.free_list(shape.pool, shape.seed))
    pool = OraclePool(shape.pool, shape.hkv, shape.d)
    dt = _content.torch_dtype(shape.dtype)
    out = []
    for i, ph in enumerate(phases):
        st, tb = tree.batch_prepare(ph.seqs)
        if st != OK:
            raise RuntimeError(f"oracle batch_prepare failed with {st} at phase {i}")
        need_q = attend and ph.kind in ("extend", "decode")
        q, k, v = _content.batch_rows(shape.seed, ph.seqs, tb["prefix_lens"], shape.hq,
                                      shape.hkv, shape.d, dt, device, shape.q_scale, need_q)
        scatter(pool, tb["new_slots"], k, v)
        res = dict(kind=ph.kind, tables=tb, stats=tree.stats())
        if need_q:
            req = None if requests_of is None else requests_of(i, len(ph.seqs))
            qn = q.float().cpu().numpy()
            if ph.kind == "extend":
                res["o"], res["lse"] = extend(qn, pool, tb["req_to_token"], tb["qo_indptr"],
                                              tb["prefix_lens"], shape.hq, shape.hkv, requests=req)
            else:
                res["o"], res["lse"] = decode(qn, pool, tb["req_to_token"], tb["seq_lens"],
                                              shape.hq, shape.hkv, requests=req)
        tree.batch_commit(ph.seqs, tb["req_to_token"], tb["nodes"])
        res["evicted_total"] = tree.evicted_total
        out.append(res)
    if keep is not None:
        keep["tree"], keep["pool"] = tree, pool
    return out
