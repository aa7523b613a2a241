"""Runs a workload through the native path on the GPU and through the oracle
on the CPU, side by side.

Both sides get the same seeded input rows (from `inputs.content`) and nothing
else: the oracle builds its own tree, tables and pool (and the tables are
asserted bit-exact against the library's), and computes attention in float64.
"""
from __future__ import annotations

import inspect
import math
import sys
import time

import numpy as np
import torch

from inputs import configs, content
from oracle import attention as oatt
from oracle.pool import OraclePool, scatter as oscatter
from oracle.radix import OracleTree

TOL = {"f32": 1e-5, "bf16": 2e-2}
# lse bounds.  fp32 paths, and the vector-unit decode, keep fp32 softmax
# weights: 1e-5 / 1e-4.  bf16 extend, and bf16 decode with >= 4 query heads
# per kv head (both on matrix cores), normalize by the sum of the same
# bf16-rounded weights that PV multiplies.  Each weight then carries a
# relative error of at most u = 2^-8 (bf16 unit roundoff, round to nearest
# even), so the sum lies in [l(1 - u), l(1 + u)] and its log within
# -ln(1 - 2^-8) = 3.9139e-3 of ln l.  The fp32 part adds at most
# n * 2^-24 relative for the sum of n weights (6.9e-5 at 1152 keys; far
# less in practice, which the 120k-key tests show) plus |lse| * 2^-23 for
# forming m + log2(l) in fp32: 1e-4 covers both at the benchmark sizes.
LSE_BF16_ROUNDING = -math.log1p(-2.0 ** -8)
LSE_TOL = {"f32": 1e-5, "bf16": LSE_BF16_ROUNDING + 1e-4}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _pick(select, i, B, tables):
    """Requests of phase i to check: select(i, B) or, for selectors that
    take a third argument, select(i, B, tables) with the oracle's tables of
    that batch (None = all)."""
    if len(inspect.signature(select).parameters) >= 3:
        return select(i, B, tables)
    return select(i, B)


def needed_slots(shape, phases, select):
    """Dry run of the oracle tree: slots the selected requests will read."""
    t = OracleTree(shape.pool, configs.free_list(shape.pool, shape.seed))
    need = set()
    for i, ph in enumerate(phases):
        st, tb = t.batch_prepare(ph.seqs)
        assert st == 0
        reqs = _pick(select, i, len(ph.seqs), tb) if ph.kind in ("extend", "decode") else []
        if reqs is None:
            reqs = range(len(ph.seqs))
        for r in reqs:
            need.update(tb["req_to_token"][r][: tb["seq_lens"][r]])
        t.batch_commit(ph.seqs, tb["req_to_token"], tb["nodes"])
    return need


ORACLE_CHUNK = 8   # requests per oracle call, each followed by a progress line


def run(shape, phases, select=lambda i, B: None, num_splits=None, content_device="cuda",
        with_lse=True, sparse=False, cascade=None, phase_source=None):
    """Returns a list of per-checked-phase dicts with GPU and oracle outputs
    restricted to the selected requests' rows.  cascade: None for plain
    decode, else a dict of cascade_plan arguments for prefix-shared decode
    (the native plan is then asserted equal to the oracle's).
    phase_source: instead of a fixed `phases` list, a callable
    (cache, oracle_tree) -> iterator of phases, advanced after each phase is
    committed on both trees (a serving loop that decides the next batch
    from the cache's state); not with sparse=True."""
    from prefix_shared_kv_host_amd.engine import RadixKVCache

    dt = content.torch_dtype(shape.dtype)
    perm = configs.free_list(shape.pool, shape.seed)
    otree = OracleTree(shape.pool, perm)
    opool = OraclePool(shape.pool, shape.hkv, shape.d)
    cache = RadixKVCache(shape.pool, shape.hkv, shape.d, dt, "cuda", perm)
    keep = None
    if sparse:
        assert phase_source is None, "a sparse oracle pool needs the phases up front"
        keep = np.zeros(shape.pool, dtype=bool)
        keep[list(needed_slots(shape, phases, select))] = True
    out = []
    source = phases if phase_source is None else phase_source(cache, otree)
    for i, ph in enumerate(source):
        t0 = time.time()
        st, otb = otree.batch_prepare(ph.seqs)
        assert st == 0
        batch = cache.prepare(ph.seqs)
        for key in ("prefix_lens", "seq_lens", "qo_indptr", "new_slots"):
            assert list(otb[key]) == batch.host[key].tolist(), (shape.name, i, key)
        for r in range(len(ph.seqs)):
            L = otb["seq_lens"][r]
            assert list(otb["req_to_token"][r][:L]) == batch.host["req_to_token"][r][:L].tolist()
        reqs = _pick(select, i, len(ph.seqs), otb) if ph.kind in ("extend", "decode") else []
        attend = reqs is None or len(reqs) > 0
        q, k, v = content.batch_rows(shape.seed, ph.seqs, otb["prefix_lens"], shape.hq, shape.hkv,
                                     shape.d, dt, content_device, shape.q_scale, with_q=attend)
        cache.store(batch, k.to("cuda"), v.to("cuda"))
        slots = np.asarray(otb["new_slots"], dtype=np.int64)
        if keep is not None:
            sel = np.nonzero(keep[slots])[0]
            idx = torch.from_numpy(sel).to(k.device)
            oscatter(opool, slots[sel], k.index_select(0, idx).cpu(), v.index_select(0, idx).cpu())
        else:
            oscatter(opool, slots, k.cpu(), v.cpu())
        if attend:
            qd = q.to("cuda")
            rows = qd.shape[0]
            lse = torch.full((rows, shape.hq), float("nan"), device="cuda") if with_lse else None
            if ph.kind == "extend":
                o = cache.extend(batch, qd, lse=lse)
            elif cascade is not None:
                plan = cache.cascade_plan(batch, shape.hq, **cascade)
                check_plan(plan, otb, **cascade, hkv=shape.hkv, G=shape.hq // shape.hkv)
                o = cache.decode_cascade(batch, qd, plan=plan, lse=lse)
            else:
                o = cache.decode(batch, qd, lse=lse, num_splits=num_splits)
            torch.cuda.synchronize()
            B = len(ph.seqs)
            rq = list(range(B)) if reqs is None else list(reqs)
            qn = q.float().cpu().numpy()
            if ph.kind == "extend":
                o_ref = np.full((rows, shape.hq, shape.d), np.nan)
                lse_ref = np.full((rows, shape.hq), np.nan)
                for c in range(0, len(rq), ORACLE_CHUNK):
                    part = rq[c:c + ORACLE_CHUNK]
                    t1 = time.time()
                    o_p, l_p = oatt.extend(qn, opool, otb["req_to_token"], otb["qo_indptr"],
                                           otb["prefix_lens"], shape.hq, shape.hkv, requests=part)
                    pr = np.concatenate([np.arange(otb["qo_indptr"][r], otb["qo_indptr"][r + 1]) for r in part])
                    o_ref[pr], lse_ref[pr] = o_p[pr], l_p[pr]
                    if len(rq) > ORACLE_CHUNK:
                        log(f"  oracle: requests {c}..{c + len(part) - 1} of {len(rq)} ({time.time() - t1:.1f}s)")
                row_idx = np.concatenate([np.arange(otb["qo_indptr"][r], otb["qo_indptr"][r + 1]) for r in rq])
            else:
                o_ref, lse_ref = oatt.decode(qn, opool, otb["req_to_token"], otb["seq_lens"],
                                             shape.hq, shape.hkv, requests=rq)
                row_idx = np.array(rq, dtype=np.int64)
            og = o.float().cpu().numpy()[row_idx]
            lg = lse.cpu().numpy()[row_idx] if with_lse else None
            out.append(dict(phase=i, kind=ph.kind, requests=rq, o=og, o_ref=o_ref[row_idx], lse=lg,
                            lse_ref=lse_ref[row_idx], o_full=o, batch=batch))
            log(f"[{shape.name}] phase {i} {ph.kind} B={B} checked={len(rq)} "
                f"({time.time() - t0:.1f}s)")
        otree.batch_commit(ph.seqs, otb["req_to_token"], otb["nodes"])
        cache.commit(batch)
    return out, cache


def check_plan(plan, otb, seg_chunk=None, tail_chunk=None, min_keys=32, max_members=None, hkv=None, G=None):
    """The native prefix-shared plan equals the oracle's, array by array.
    tail_chunk None: the engine's default rule, 768 keys, or 384 when the
    grouped-head tails (G >= 4) would give fewer than 1024 items at 768.
    seg_chunk None: the tail chunk, or 256 keys when the rule halved it."""
    from oracle import cascade as ocas
    L = otb["seq_lens"]
    sc = seg_chunk
    if tail_chunk is None:
        tail_chunk = 768
        if G is not None and G >= 4:
            rows = [row[: int(L[r])] for r, row in enumerate(otb["req_to_token"])]
            first = ocas.plan(rows, L, 768, 768, min_keys, plan.max_members)
            tails = np.asarray(L, dtype=np.int64) - np.asarray(first["tail_begin"], dtype=np.int64)
            items = int(((tails + 767) // 768).sum()) * hkv
            if 0 < items < 1024:
                tail_chunk = 384
                sc = 256 if seg_chunk is None else seg_chunk
        assert plan.tail_chunk == tail_chunk, (plan.tail_chunk, tail_chunk)
    seg_chunk = tail_chunk if sc is None else sc
    if plan.seg_chunk is not None:
        assert plan.seg_chunk == seg_chunk, (plan.seg_chunk, seg_chunk)
    ref = ocas.plan([row[: int(L[r])] for r, row in enumerate(otb["req_to_token"])], L, seg_chunk,
                    tail_chunk, min_keys, plan.max_members)
    assert plan.perm.tolist() == ref["perm"]
    assert plan.rec_indptr.tolist() == ref["rec_indptr"]
    assert plan.tail_begin.tolist() == ref["tail_begin"]
    assert [tuple(j) for j in plan.jobs.tolist()] == ref["jobs"]
    assert plan.tail_splits == ref["tail_splits"]
    log(f"  plan: {plan.n_jobs} jobs, {plan.n_records} records, tail splits {plan.tail_splits}")


def check(res, dtype, name=""):
    """Asserts the tolerance on every compared element; returns a report."""
    rep = []
    for r in res:
        err = np.abs(r["o"] - r["o_ref"])
        nan = int(np.isnan(r["o"]).sum())
        mx = float(np.nanmax(err)) if err.size else 0.0
        rel = mx / max(float(np.abs(r["o_ref"]).max()), 1e-30)
        line = dict(phase=r["phase"], max_abs=mx, rel=rel, mean_abs=float(err.mean()), nan=nan)
        if r["lse"] is not None:
            line["lse_max_abs"] = float(np.abs(r["lse"] - r["lse_ref"]).max())
        log(f"  {name} {line}")
        rep.append(line)
        assert nan == 0, (name, line)
        assert mx <= TOL[dtype], (name, line)
        if r["lse"] is not None:
            assert line["lse_max_abs"] <= LSE_TOL[dtype], (name, line)
    return rep


def sample(seed, k):
    """Seeded selector: k requests per checked phase (all when B <= k)."""
    def f(i, B):
        if B <= k:
            return None
        rng = np.random.default_rng(seed * 1000 + i)
        return sorted(rng.choice(B, size=k, replace=False).tolist())
    return f


def sm_scale(d):
    return 1.0 / math.sqrt(d)
