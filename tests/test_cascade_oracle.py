"""Pins for the oracle's prefix-shared decode plan (oracle/cascade.py).

The plan is integer work, checked against what its definition fixes rather
than against a second copy of it:

  * exact cover: the records of every request cover its keys 0 .. L-1 once;
  * sharing is real: every member of a job has the same slots over the job's
    keys, and none of them is its own query key (key_end <= L_m - 1);
  * minimal reads (min_keys = 1, unbounded chunks and groups): the keys the
    plan reads equal the number of distinct prefixes of the truncated rows,
    counted by brute force as a set of tuples, plus one query key per
    request; no plan that reads every distinct prefix once can read fewer;
  * maximal sharing (min_keys = 1): no position of a private tail, other
    than the query key, is shared with another request (brute force);
  * folding (min_keys > 1): every emitted segment is at least min_keys long,
    the cover and sharing pins still hold, and no request shares more than
    the unfolded plan lets it;
  * chunks and groups: no job is longer than seg_chunk or has more members
    than max_members, tail records hold at most tail_chunk keys;
  * arithmetic: the record-by-record decode equals plain decode attention
    (float64, 1e-12), which is the split identity the plan relies on.
"""
import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import cascade
from oracle.pool import OraclePool, scatter


def _table(seed, B, max_len=40, p_share=0.7, p_dup=0.1):
    """Rows built like a prefix tree: each request copies a cut of an earlier
    row (or of nothing) and appends fresh slots; some rows are exact copies
    of earlier ones; lengths from 1 up."""
    rng = np.random.default_rng(seed)
    next_slot = [1000]
    rows = []

    def fresh(n):
        out = list(range(next_slot[0], next_slot[0] + n))
        next_slot[0] += n
        return out

    for _ in range(B):
        if rows and rng.random() < p_dup:
            rows.append(list(rows[int(rng.integers(len(rows)))]))
            continue
        if rows and rng.random() < p_share:
            base = rows[int(rng.integers(len(rows)))]
            cut = int(rng.integers(0, len(base) + 1))
            row = base[:cut] + fresh(int(rng.integers(0 if cut else 1, 12)))
        else:
            row = fresh(int(rng.integers(1, max_len)))
        rows.append(row[:max_len] if row else fresh(1))
    ld = max(len(r) for r in rows) + 3
    r2t = np.full((B, ld), -1, dtype=np.int64)
    for r, row in enumerate(rows):
        r2t[r, :len(row)] = row
    return r2t, np.array([len(r) for r in rows], dtype=np.int64)


def _check_cover_and_sharing(p, r2t, L, seg_chunk, tail_chunk, max_members):
    B = len(L)
    counts = [np.zeros(int(L[r]), dtype=np.int64) for r in range(B)]
    seen = set()
    for kb, ke, first, count, rec_off in p["jobs"]:
        assert 0 <= kb < ke and ke - kb <= seg_chunk
        assert 1 <= count <= max_members
        ms = p["perm"][first:first + count]
        assert len(ms) == count
        for m in ms:
            assert ke <= L[m] - 1
            assert list(r2t[m, kb:ke]) == list(r2t[ms[0], kb:ke])
            assert 0 <= rec_off < p["rec_indptr"][m + 1] - p["rec_indptr"][m]
            assert (m, rec_off) not in seen
            seen.add((m, rec_off))
            counts[m][kb:ke] += 1
    for r in range(B):
        n = p["rec_indptr"][r + 1] - p["rec_indptr"][r]
        tb = p["tail_begin"][r]
        assert 0 <= tb <= L[r] - 1
        ntail = -(-(int(L[r]) - tb) // tail_chunk)
        assert 1 <= ntail <= p["tail_splits"]
        assert {k for (m, k) in seen if m == r} == set(range(n - ntail))
        counts[r][tb:] += 1
        assert (counts[r] == 1).all(), (r, counts[r])
    assert p["rec_indptr"][0] == 0 and all(a <= b for a, b in zip(p["rec_indptr"], p["rec_indptr"][1:]))
    assert sorted(p["perm"]) == list(range(B))


def _distinct_prefixes(r2t, L):
    s = set()
    for r in range(len(L)):
        row = tuple(int(x) for x in r2t[r, :max(int(L[r]) - 1, 0)])
        for t in range(len(row)):
            s.add(row[:t + 1])
    return len(s)


def _keys_read(p, L):
    return sum(ke - kb for kb, ke, *_ in p["jobs"]) + sum(int(L[r]) - p["tail_begin"][r] for r in range(len(L)))


@pytest.mark.parametrize("seed", range(16))
def test_plan_cover_sharing_minimal_maximal(seed):
    r2t, L = _table(seed, B=int(np.random.default_rng(seed).integers(1, 30)))
    big = int(L.max()) + 1
    p = cascade.plan(r2t, L, seg_chunk=big, tail_chunk=big, min_keys=1)
    _check_cover_and_sharing(p, r2t, L, big, big, len(L))
    assert _keys_read(p, L) == _distinct_prefixes(r2t, L) + len(L)
    # maximal: a tail position (before the query key) has no other request
    # with the same prefix up to and including it
    for r in range(len(L)):
        for t in range(p["tail_begin"][r], int(L[r]) - 1):
            pre = list(r2t[r, :t + 1])
            assert not any(o != r and t < L[o] - 1 and list(r2t[o, :t + 1]) == pre for o in range(len(L)))


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("min_keys", [2, 3, 8])
def test_plan_folding(seed, min_keys):
    r2t, L = _table(100 + seed, B=25)
    big = int(L.max()) + 1
    p = cascade.plan(r2t, L, seg_chunk=big, tail_chunk=big, min_keys=min_keys)
    _check_cover_and_sharing(p, r2t, L, big, big, len(L))
    # unbounded chunks and groups: one job per emitted segment
    assert all(ke - kb >= min_keys for kb, ke, *_ in p["jobs"])
    ref = cascade.plan(r2t, L, seg_chunk=big, tail_chunk=big, min_keys=1)
    assert _keys_read(p, L) >= _keys_read(ref, L)
    # folding only moves keys later into segments or into the tail: a request
    # shares at most what the unfolded plan lets it share
    for r in range(len(L)):
        assert p["tail_begin"][r] <= ref["tail_begin"][r]


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("min_keys,seg_chunk,tail_chunk,max_members", [(3, 4, 5, 2), (8, 64, 3, 3), (1, 1, 1, 1)])
def test_plan_chunks_and_groups(seed, min_keys, seg_chunk, tail_chunk, max_members):
    r2t, L = _table(200 + seed, B=25)
    big = int(L.max()) + 1
    p = cascade.plan(r2t, L, seg_chunk=seg_chunk, tail_chunk=tail_chunk, min_keys=min_keys,
                     max_members=max_members)
    _check_cover_and_sharing(p, r2t, L, seg_chunk, tail_chunk, max_members)
    # cutting into chunks and groups changes no request's shared keys
    whole = cascade.plan(r2t, L, seg_chunk=big, tail_chunk=big, min_keys=min_keys)
    assert p["tail_begin"] == whole["tail_begin"]
    assert p["perm"] == whole["perm"]


@pytest.mark.parametrize("seed", range(6))
def test_record_decode_equals_plain_decode(seed):
    rng = np.random.default_rng(seed)
    r2t, L = _table(300 + seed, B=12, max_len=30)
    hq, hkv, D = 4, 2, 16
    slots = sorted({int(x) for x in r2t.ravel() if x >= 0})
    pool = OraclePool(max(slots) + 1, hkv, D)
    scatter(pool, slots, torch.randn(len(slots), hkv, D, dtype=torch.float64, generator=torch.Generator().manual_seed(seed)),
            torch.randn(len(slots), hkv, D, dtype=torch.float64, generator=torch.Generator().manual_seed(seed + 99)))
    q = rng.standard_normal((len(L), hq, D))
    o_ref, lse_ref = oa.decode(q, pool, r2t, L, hq, hkv)
    for mk, sc, tc, mm in ((1, 1000, 1000, None), (2, 3, 4, 2), (5, 7, 2, 1)):
        p = cascade.plan(r2t, L, seg_chunk=sc, tail_chunk=tc, min_keys=mk, max_members=mm)
        o, lse = cascade.decode(q, pool, r2t, L, hq, hkv, p, tc)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_plan_small_worked_example():
    """Rows A=[1,2,3,9], B=[1,2,4,8], C=[5,6]: A and B share slots 1,2 (keys
    0-1); their third keys differ; C shares nothing; every query key is
    private."""
    r2t = np.array([[1, 2, 3, 9], [1, 2, 4, 8], [5, 6, -1, -1]])
    p = cascade.plan(r2t, [4, 4, 2], seg_chunk=8, tail_chunk=8)
    assert p["perm"] == [0, 1, 2]
    assert p["jobs"] == [(0, 2, 0, 2, 0)]
    assert p["tail_begin"] == [2, 2, 0]
    assert p["rec_indptr"] == [0, 2, 4, 5]
    # identical rows share all but the query key; a row that is a proper
    # prefix of another shares its keys before its own query key
    r2t = np.array([[7, 8, 9], [7, 8, 9], [7, 8, -1]])
    p = cascade.plan(r2t, [3, 3, 2], seg_chunk=8, tail_chunk=8)
    assert p["perm"] == [2, 0, 1]
    assert p["jobs"] == [(0, 1, 0, 3, 0), (1, 2, 1, 2, 1)]
    assert p["tail_begin"] == [2, 2, 1]


def test_pins_catch_planted_mistakes(monkeypatch):
    """A plan that shares the query key, and one that forgets to carry a
    folded run into the next, each fail the pins above."""
    real = cascade.plan

    def shares_query_key(req_to_token, seq_lens, *a, **k):
        return real(req_to_token, [int(x) + 1 for x in seq_lens], *a, **k)

    def drops_folded(req_to_token, seq_lens, seg_chunk, tail_chunk, min_keys=1, max_members=None):
        p = real(req_to_token, seq_lens, seg_chunk, tail_chunk, min_keys, max_members)
        p["jobs"] = [(kb + 1 if kb > 0 else kb, ke, f, c, ro) for kb, ke, f, c, ro in p["jobs"]]
        return p

    for fn, check in ((shares_query_key, test_plan_cover_sharing_minimal_maximal),
                      (drops_folded, test_plan_cover_sharing_minimal_maximal)):
        with monkeypatch.context() as m:
            m.setattr(cascade, "plan", fn)
            with pytest.raises(AssertionError):
                for s in range(16):
                    check(s)
