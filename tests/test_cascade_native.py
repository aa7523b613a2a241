"""The native prefix-shared decode planner (rkv_cascade_plan) against the
oracle's plan: every array equal, on random prefix-tree tables and on the
decode batches of the radix-tree decode workload (256 requests, 4-ary tree),
its no-share control and the grouped-head workload (64 decode requests under
one 2048-token prefix).  Host code only; no GPU needed."""
import numpy as np
import pytest

from inputs import configs
from oracle import cascade as ocas
from prefix_shared_kv_host_amd import rkv
from tests.test_cascade_oracle import _table


def _same(plan, ref):
    assert plan.perm.tolist() == ref["perm"]
    assert plan.rec_indptr.tolist() == ref["rec_indptr"]
    assert plan.tail_begin.tolist() == ref["tail_begin"]
    assert [tuple(j) for j in plan.jobs.tolist()] == ref["jobs"]
    assert plan.tail_splits == ref["tail_splits"]
    assert plan.n_records == ref["rec_indptr"][-1]


@pytest.mark.parametrize("seed", range(20))
@pytest.mark.parametrize("params", [(1000, 1000, 1, 1000), (4, 5, 3, 2), (64, 3, 8, 3), (1, 1, 1, 1), (7, 768, 2, 32)])
def test_native_plan_equals_oracle(seed, params):
    seg_chunk, tail_chunk, min_keys, mm = params
    r2t, L = _table(500 + seed, B=int(np.random.default_rng(seed).integers(1, 40)))
    plan = rkv.cascade_plan(r2t.astype(np.int32), L, seg_chunk, tail_chunk, min_keys, mm)
    _same(plan, ocas.plan(r2t, L, seg_chunk, tail_chunk, min_keys, mm))


def _decode_tables(name):
    shape, phases = configs.build(name)
    t = rkv.Tree(shape.pool, configs.free_list(shape.pool, shape.seed))
    for ph in phases:
        code, tb = t.batch_prepare(ph.seqs)
        assert code == rkv.OK
        if ph.kind == "decode":
            return shape, tb
        t.batch_commit(ph.seqs, tb["req_to_token"], tb["nodes"])
    raise AssertionError("no decode phase")


@pytest.mark.parametrize("name", ["c3", "c3ns", "c4"])
def test_native_plan_equals_oracle_on_workloads(name):
    shape, tb = _decode_tables(name)
    L = tb["seq_lens"]
    mm = rkv.cascade_max_members(shape.hq, shape.hkv, shape.d)
    plan = rkv.cascade_plan(tb["req_to_token"], L, 256, 768, 32, mm)
    rows = [row[: int(L[r])] for r, row in enumerate(tb["req_to_token"])]
    _same(plan, ocas.plan(rows, L, 256, 768, 32, mm))
    if name == "c3ns":
        assert plan.n_jobs == 0
    else:
        assert plan.n_jobs > 0


def test_plan_argument_errors_and_sizing():
    r2t = np.array([[1, 2, 3], [1, 2, 4]], dtype=np.int32)
    L = np.array([3, 3], dtype=np.int32)
    lib = rkv.lib()
    import ctypes
    perm = np.zeros(2, np.int32)
    rec = np.zeros(3, np.int32)
    tb = np.zeros(2, np.int32)
    n, ts = ctypes.c_int64(-1), ctypes.c_int32(-1)
    p = lambda a: a.ctypes.data_as(rkv.c_i32p)

    def call(L_, ld=3, seg=4, tail=4, mk=1, mm=4, jobs=None, cap=0):
        return lib.rkv_cascade_plan(p(r2t), ld, p(L_), 2, seg, tail, mk, mm, p(perm), p(rec), p(tb),
                                    jobs, cap, ctypes.byref(n), ctypes.byref(ts))

    assert call(L) == rkv.ENOSPC and n.value == 1           # sizing: one job needed
    jobs = np.zeros(5, np.int32)
    assert call(L, jobs=p(jobs), cap=1) == rkv.OK
    assert jobs.tolist() == [0, 2, 0, 2, 0] and tb.tolist() == [2, 2] and rec.tolist() == [0, 2, 4]
    assert call(np.array([0, 3], np.int32)) == rkv.EINVAL   # L < 1
    assert call(np.array([4, 3], np.int32)) == rkv.EINVAL   # L > ld
    for kw in ({"seg": 0}, {"tail": 0}, {"mk": 0}, {"mm": 0}):
        assert call(L, **kw) == rkv.EINVAL
    # an empty batch plans nothing
    plan = rkv.cascade_plan(np.zeros((0, 4), np.int32), np.zeros(0, np.int32))
    assert plan.n_jobs == 0 and plan.rec_indptr.tolist() == [0] and plan.tail_splits == 0


def test_native_plan_on_gpu_test_workloads():
    """The tree-shaped decode batches the GPU cascade tests use: the native
    plan equals the oracle's and the batches do share at several levels."""
    from tests.test_gpu_cascade import CASES, tree_decode_workload
    for hq, hkv, d, params in CASES:
        phases = tree_decode_workload(seed=hq * 100 + d + params["tail_chunk"])
        t = rkv.Tree(1 << 16)
        code, tb = t.batch_prepare(phases[0].seqs)
        assert code == rkv.OK
        t.batch_commit(phases[0].seqs, tb["req_to_token"], tb["nodes"])
        code, tb = t.batch_prepare(phases[1].seqs)
        assert code == rkv.OK
        L = tb["seq_lens"]
        mm = params.get("max_members", rkv.cascade_max_members(hq, hkv, d))
        args = (params["seg_chunk"], params["tail_chunk"], params["min_keys"], mm)
        plan = rkv.cascade_plan(tb["req_to_token"], L, *args)
        _same(plan, ocas.plan([row[: int(L[r])] for r, row in enumerate(tb["req_to_token"])], L, *args))
        assert plan.n_jobs >= 3
        assert len({j[4] for j in plan.jobs.tolist()}) >= 2          # runs nest
        assert min(L) == 1
