"""Pins for the oracle's read-only match (peek), its cache-aware queue order
(schedule) and its serving loop, against brute force and closed forms.

  * peek(q) = longest common prefix of q with any cached root path (the paths
    are read from the canonical dump), and peek leaves the dump unchanged;
  * schedule: matched[q] = that brute-force length on the first L-1 tokens;
    the order is a permutation, non-increasing in matched, ties in queue order;
  * serving: with an unbounded pool every turn reuses exactly its session's
    previous turn (closed form), under either order; on tiny traces an
    exhaustive search over every order that respects the sessions' turn order
    bounds both orders from above, and re-evaluating each order's own run
    from scratch gives back the reuse the loop reported.
"""
import itertools

import numpy as np
import pytest

from oracle import serving
from oracle.radix import OK, OracleTree
from tests.radix_ops import parse_dump, paths


def _lcp(a, b):
    n = 0
    while n < len(a) and n < len(b) and a[n] == b[n]:
        n += 1
    return n


def _random_tree(seed, n_seqs, vocab, pool):
    rng = np.random.default_rng(seed)
    t = OracleTree(pool, [int(x) for x in rng.permutation(pool)])
    seqs = []
    for _ in range(n_seqs):
        if seqs and rng.random() < 0.6:
            base = seqs[int(rng.integers(len(seqs)))]
            cut = int(rng.integers(0, len(base) + 1))
            seq = base[:cut] + [int(x) for x in rng.integers(0, vocab, int(rng.integers(1, 8)))]
        else:
            seq = [int(x) for x in rng.integers(0, vocab, int(rng.integers(1, 12)))]
        st, tb = t.batch_prepare([seq])
        if st != OK:
            continue
        t.batch_commit([seq], tb["req_to_token"], tb["nodes"])
        seqs.append(seq)
    return t, seqs, rng


def _query(rng, seqs, vocab):
    base = seqs[int(rng.integers(len(seqs)))] if seqs else []
    cut = int(rng.integers(0, len(base) + 1))
    return base[:cut] + [int(x) for x in rng.integers(0, vocab, int(rng.integers(0, 5)))]


def _cached_paths(t):
    return [p for p, _ in paths(parse_dump(t.serialize())).values()]


@pytest.mark.parametrize("seed", range(12))
def test_peek_is_longest_cached_prefix_and_read_only(seed):
    t, seqs, rng = _random_tree(seed, 40, 4, pool=48)     # small pool: evictions happen
    cached = _cached_paths(t)
    for _ in range(60):
        q = _query(rng, seqs, 4)
        before = t.serialize()
        assert t.peek(q) == max([_lcp(q, p) for p in cached], default=0)
        assert t.serialize() == before


@pytest.mark.parametrize("seed", range(8))
def test_schedule_ranks_by_capped_reuse(seed):
    t, seqs, rng = _random_tree(100 + seed, 30, 3, pool=64)
    cached = _cached_paths(t)
    queue = [_query(rng, seqs, 3) for _ in range(25)] + [[]]
    before = t.serialize()
    order, matched = t.schedule(queue)
    assert t.serialize() == before
    for q, m in zip(queue, matched):
        capped = q[: max(len(q) - 1, 0)]
        assert m == max([_lcp(capped, p) for p in cached], default=0)
    assert sorted(order) == list(range(len(queue)))
    for a, b in zip(order, order[1:]):
        assert matched[a] > matched[b] or (matched[a] == matched[b] and a < b)


def _tiny_trace(seed, sessions, turns_per, seg=(2, 5), vocab=50):
    rng = np.random.default_rng(seed)
    turns, arrival = {}, []
    for s in range(sessions):
        hist = []
        for t in range(turns_per):
            segment = [int(x) for x in rng.integers(1, vocab, int(rng.integers(seg[0], seg[1] + 1)))]
            if t == 0:
                segment[0] = 1000 + s          # sessions never share a prefix
            hist = hist + segment
            turns[(s, t)] = list(hist)
    keys = list(turns)
    for i in rng.permutation(len(keys)):
        arrival.append(keys[int(i)])
    return turns, arrival


def _reuse_of_order(turns, order, pool, free):
    """Runs the turns one per batch in the given order on a fresh tree."""
    t = OracleTree(pool, list(free))
    total = 0
    for st in order:
        status, tb = t.batch_prepare([turns[st]])
        if status != OK:
            return None
        t.batch_commit([turns[st]], tb["req_to_token"], tb["nodes"])
        total += int(tb["prefix_lens"][0])
    return total


def _valid_orders(turns):
    keys = sorted(turns)
    for perm in itertools.permutations(keys):
        seen = set()
        ok = True
        for st in perm:
            if st[1] > 0 and (st[0], st[1] - 1) not in seen:
                ok = False
                break
            seen.add(st)
        if ok:
            yield perm


@pytest.mark.parametrize("seed", range(4))
def test_unbounded_pool_reuses_exactly_the_history(seed):
    turns, arrival = _tiny_trace(seed, sessions=5, turns_per=4)
    expect = sum(len(turns[(s, t - 1)]) for (s, t) in turns if t > 0)
    for policy in ("fcfs", "cache"):
        tree = OracleTree(4096, list(range(4096)))
        r = serving.serve(tree, turns, arrival, policy, max_batch=3)
        assert r["reused_tokens"] == expect
        assert sorted(r["order"]) == sorted(turns)


@pytest.mark.parametrize("seed", range(6))
def test_exhaustive_optimum_bounds_both_orders(seed):
    turns, arrival = _tiny_trace(200 + seed, sessions=3, turns_per=2, seg=(3, 6))
    pool = max(len(v) for v in turns.values()) + 4          # eviction binds
    free = [int(x) for x in np.random.default_rng(seed).permutation(pool)]
    best = max(v for v in (_reuse_of_order(turns, o, pool, free) for o in _valid_orders(turns)) if v is not None)
    # closed-form pin of the exhaustive evaluator: an unbounded pool makes
    # every valid order reuse exactly the history
    hist = sum(len(turns[(s, t - 1)]) for (s, t) in turns if t > 0)
    assert {_reuse_of_order(turns, o, 4096, range(4096)) for o in _valid_orders(turns)} == {hist}
    for policy in ("fcfs", "cache"):
        r = serving.serve(OracleTree(pool, list(free)), turns, arrival, policy, max_batch=1)
        assert r["reused_tokens"] == _reuse_of_order(turns, r["order"], pool, free)
        assert r["reused_tokens"] <= best


def test_pins_catch_planted_mistakes(monkeypatch):
    """A peek that drops the partial edge, and a schedule without the L-1
    cap, each fail the pins above."""
    def partial_edge_peek(self, tok):
        tok = [int(t) for t in tok]
        node, m = self.root, 0
        while m < len(tok):
            c = self._child(node, tok[m])
            if c is None:
                break
            k = 0
            while k < len(c.label) and m + k < len(tok) and c.label[k] == tok[m + k]:
                k += 1
            if k < len(c.label):
                break
            m += k
            node = c
        return m

    def uncapped_schedule(self, seqs):
        matched = [self.peek(list(s)) for s in seqs]
        return sorted(range(len(seqs)), key=lambda q: (-matched[q], q)), matched

    for name, fn, check in (("peek", partial_edge_peek, test_peek_is_longest_cached_prefix_and_read_only),
                            ("schedule", uncapped_schedule, test_schedule_ranks_by_capped_reuse)):
        with monkeypatch.context() as m:
            m.setattr(OracleTree, name, fn)
            with pytest.raises(AssertionError):
                for s in range(8):
                    check(s)
