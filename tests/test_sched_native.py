"""Native cache-aware scheduling (rkv_radix_peek, rkv_schedule, the package's
run_queue) against the oracle, bit for bit: same matched lengths, same order,
same turns run in the same steps with the same reuse, same final tree."""
import numpy as np
import pytest

from inputs import configs
from oracle import serving as oserving
from oracle.radix import OK, OracleTree
from prefix_shared_kv_host_amd import rkv, serving
from tests.test_sched_oracle import _query, _tiny_trace


def _pair(seed, n_seqs, vocab, pool):
    rng = np.random.default_rng(seed)
    perm = [int(x) for x in rng.permutation(pool)]
    o, n = OracleTree(pool, perm), rkv.Tree(pool, np.asarray(perm, dtype=np.int32))
    seqs = []
    for _ in range(n_seqs):
        if seqs and rng.random() < 0.6:
            base = seqs[int(rng.integers(len(seqs)))]
            seq = base[: int(rng.integers(0, len(base) + 1))] + [int(x) for x in rng.integers(0, vocab, int(rng.integers(1, 8)))]
        else:
            seq = [int(x) for x in rng.integers(0, vocab, int(rng.integers(1, 12)))]
        st, tb = o.batch_prepare([seq])
        code, tbn = n.batch_prepare([seq])
        assert (st == OK) == (code == rkv.OK)
        if st != OK:
            continue
        o.batch_commit([seq], tb["req_to_token"], tb["nodes"])
        n.batch_commit([seq], tbn["req_to_token"], tbn["nodes"])
        seqs.append(seq)
    assert o.serialize() == n.radix_serialize()
    return o, n, seqs, rng


@pytest.mark.parametrize("seed", range(10))
def test_peek_and_schedule_match_oracle(seed):
    o, n, seqs, rng = _pair(seed, 40, 4, pool=48)
    queue = [_query(rng, seqs, 4) for _ in range(40)] + [[], [7]]
    before = n.radix_serialize()
    for q in queue:
        assert n.radix_peek(q) == o.peek(q)
    order, matched = n.schedule(queue)
    oo, om = o.schedule(queue)
    assert order.tolist() == list(oo) and matched.tolist() == list(om)
    assert n.radix_serialize() == before


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("policy", ["fcfs", "cache"])
def test_run_queue_matches_oracle_tiny(seed, policy):
    turns, arrival = _tiny_trace(300 + seed, sessions=6, turns_per=3, seg=(2, 7))
    pool = 40
    perm = [int(x) for x in np.random.default_rng(seed).permutation(pool)]
    a = serving.run_queue(rkv.Tree(pool, np.asarray(perm, dtype=np.int32)), turns, arrival, policy, max_batch=2)
    b = oserving.serve(OracleTree(pool, perm), turns, arrival, policy, max_batch=2)
    assert a["order"] == b["order"] and a["reused"] == b["reused"] and a["steps"] == b["steps"]


@pytest.mark.parametrize("policy", ["fcfs", "cache"])
def test_run_queue_matches_oracle_on_chat_trace_with_eviction(policy):
    s, _ = configs.c5e()
    batches, tags = configs.chat_trace(s.seed)
    turns = {st: seq for b, tg in zip(batches, tags) for seq, st in zip(b, tg)}
    arrival = [st for tg in tags for st in tg]
    perm = configs.free_list(s.pool, s.seed)
    nt, ot = rkv.Tree(s.pool, perm), OracleTree(s.pool, perm)
    a = serving.run_queue(nt, turns, arrival, policy)
    b = oserving.serve(ot, turns, arrival, policy)
    assert a["order"] == b["order"] and a["reused"] == b["reused"]
    assert nt.radix_serialize() == ot.serialize()
    assert nt.stats()[7] == ot.stats()[7] > 0        # evictions happened


def test_schedule_argument_errors():
    t = rkv.Tree(16, np.arange(16, dtype=np.int32))
    with pytest.raises(rkv.RkvError):
        rkv._check(rkv.lib().rkv_schedule(t._h, -1, None, None, None, None))
    assert rkv.lib().rkv_schedule(t._h, 0, None, None, None, None) == rkv.OK
    bad = np.array([0, 3, 1], dtype=np.int64)      # decreasing offsets
    tok = np.zeros(3, dtype=np.int32)
    order = np.zeros(2, dtype=np.int32)
    matched = np.zeros(2, dtype=np.int64)
    code = rkv.lib().rkv_schedule(t._h, 2, tok.ctypes.data_as(rkv.c_i32p), bad.ctypes.data_as(rkv.c_i64p),
                                  order.ctypes.data_as(rkv.c_i32p), matched.ctypes.data_as(rkv.c_i64p))
    assert code == rkv.EINVAL
