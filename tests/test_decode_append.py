"""Decode continuation of a prepared batch (batch_append): one new slot per
request per step, no re-match, the generated tokens inserted at the commit.
CPU only: the oracle pinned against the per-step prepare/commit path it must
reproduce, its error paths, and the native tree bit-exact against it (tables,
new slots, free list, tree dump) through steps that evict."""
import numpy as np
import pytest

from oracle.radix import EBUSY, EINVAL, OK, OracleTree
from tests.native_tree import NativeTree


def histories(seed, B, max_len, vocab=32000):
    """Cached histories with shared prefixes at several depths and a few
    identical ones; the decode token of request i is unique to it."""
    rng = np.random.default_rng(seed)
    hist = []
    for i in range(B):
        if i >= 2 and i % 7 == 0:
            h = list(hist[int(rng.integers(len(hist)))])
        elif hist and rng.random() < 0.7:
            base = hist[int(rng.integers(len(hist)))]
            cut = int(rng.integers(1, len(base) + 1))
            h = base[:cut] + [int(x) for x in rng.integers(0, vocab, int(rng.integers(1, max_len // 2)))]
        else:
            h = [int(x) for x in rng.integers(0, vocab, int(rng.integers(2, max_len)))]
        hist.append(h[:max_len])
    return hist


def decode_tokens(step, B):
    return [100000 + 1000 * step + i for i in range(B)]


def run_append(tree, hist, steps, ld):
    """Setup commit, one prepare of history + first token, `steps` appends,
    one commit.  Returns the tables after every step and the final sequences."""
    B = len(hist)
    st, tb = tree.batch_prepare(hist)
    assert st == OK
    tree.batch_commit(hist, tb["req_to_token"], tb["nodes"])
    seqs = [h + [t] for h, t in zip(hist, decode_tokens(0, B))]
    st, tb = tree.batch_prepare(seqs, ld)
    assert st == OK
    r2t, lens = tb["req_to_token"], list(tb["seq_lens"])
    trace = [([list(x) for x in r2t], list(lens), list(tb["new_slots"]))]
    for k in range(1, steps + 1):
        st, new = tree.batch_append(r2t, lens)
        assert st == OK
        seqs = [s + [t] for s, t in zip(seqs, decode_tokens(k, B))]
        trace.append(([list(x) for x in r2t], list(lens), list(new)))
    assert tree.batch_commit(seqs, r2t, tb["nodes"]) == OK
    return trace, seqs


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_oracle_append_equals_per_step_commit(seed):
    """Appending k positions then committing once gives, step by step, the
    same token tables and new slots as matching the whole history again each
    step (prepare + commit per step), and at the end the same slots for every
    full sequence and the same free list."""
    hist = histories(seed, B=12, max_len=60)
    steps, ld = 6, 80
    a = OracleTree(4096)
    trace, seqs = run_append(a, hist, steps, ld)

    b = OracleTree(4096)
    B = len(hist)
    st, tb = b.batch_prepare(hist)
    b.batch_commit(hist, tb["req_to_token"], tb["nodes"])
    cur = [h + [t] for h, t in zip(hist, decode_tokens(0, B))]
    for k in range(steps + 1):
        st, tb = b.batch_prepare(cur, ld)
        assert st == OK
        r2t, lens, new = trace[k]
        assert tb["req_to_token"] == r2t, k
        assert tb["seq_lens"] == lens, k
        assert tb["new_slots"] == new, k
        assert all(p == L - 1 for p, L in zip(tb["prefix_lens"], tb["seq_lens"]))
        b.batch_commit(cur, tb["req_to_token"], tb["nodes"])
        if k < steps:
            cur = [s + [t] for s, t in zip(cur, decode_tokens(k + 1, B))]
    assert cur == seqs
    for s in seqs:
        ma, sa, _ = a.match(s)
        mb, sb, _ = b.match(s)
        assert ma == mb == len(s) and sa == sb
    assert a.free_list() == b.free_list()
    assert a.stats()[3] == b.stats()[3] == 0          # nothing stays locked


def test_oracle_append_error_paths():
    t = OracleTree(8)
    st, tb = t.batch_prepare([[1, 2, 3]], ld=4)
    assert st == OK and t.stats()[1] == 5
    r2t, lens = tb["req_to_token"], list(tb["seq_lens"])
    assert t.batch_append(r2t, lens)[0] == OK and lens == [4]
    snap = ([list(x) for x in r2t], list(lens), t.free_list())
    assert t.batch_append(r2t, lens)[0] == EINVAL          # the row is full
    assert ([list(x) for x in r2t], list(lens), t.free_list()) == snap
    assert t.batch_append([], [])[0] == OK
    # no free slot and nothing evictable (the batch's path is locked)
    u = OracleTree(4)
    st, tb = u.batch_prepare([[5, 6, 7, 8]], ld=6)
    r2t, lens = tb["req_to_token"], list(tb["seq_lens"])
    assert u.batch_append(r2t, lens) == (EBUSY, None)
    assert lens == [4] and r2t[0][4] == -1


def test_oracle_append_evicts_lru_leaf():
    """With the free list empty, a step evicts the least recently used
    unlocked leaf and takes its first freed slot."""
    t = OracleTree(10)
    st, tb = t.batch_prepare([[1, 2, 3], [9, 8, 7]])
    t.batch_commit([[1, 2, 3], [9, 8, 7]], tb["req_to_token"], tb["nodes"])
    old = tb["req_to_token"][0]
    st, tb = t.batch_prepare([[9, 8, 7, 6]], ld=8)       # touches [9, 8, 7]; 3 free left
    r2t, lens = tb["req_to_token"], list(tb["seq_lens"])
    for _ in range(3):
        assert t.batch_append(r2t, lens)[0] == OK
    assert t.stats()[1] == 0
    st, new = t.batch_append(r2t, lens)
    assert st == OK and new == [old[0]]                  # [1, 2, 3] was evicted
    assert t.match([1, 2, 3])[0] == 0


@pytest.mark.parametrize("seed,pool", [(3, 1 << 14), (4, 600), (5, 500)])
def test_native_append_matches_oracle(seed, pool):
    """Native tree against the oracle through appends, including pools small
    enough that the steps evict (600 slots) or run out (500: EBUSY with the
    batch's own paths locked): tables, new slots, free list and tree dump
    identical after every step."""
    hist = histories(seed, B=10, max_len=50)
    steps, ld = 40, 100
    o, n = OracleTree(pool), NativeTree(pool)
    for t in (o, n):
        st, tb = t.batch_prepare(hist)
        assert st == OK
        t.batch_commit(hist, tb["req_to_token"], tb["nodes"])
    # unrelated cached sequences that the steps can evict
    extra = [[200000 + 100 * j + x for x in range(30)] for j in range(8)]
    for t in (o, n):
        st, tb = t.batch_prepare(extra)
        t.batch_commit(extra, tb["req_to_token"], tb["nodes"])
    seqs = [h + [t] for h, t in zip(hist, decode_tokens(0, len(hist)))]
    (so, to), (sn, tn) = o.batch_prepare(seqs, ld), n.batch_prepare(seqs, ld)
    assert so == sn == OK and to == tn
    ro, lo = to["req_to_token"], list(to["seq_lens"])
    rn, ln = [list(x) for x in tn["req_to_token"]], list(tn["seq_lens"])
    busy = False
    for k in range(1, steps + 1):
        (co, no), (cn, nn) = o.batch_append(ro, lo), n.batch_append(rn, ln)
        assert co == cn and no == nn, k
        assert ro == rn and lo == ln, k
        assert o.free_list() == n.free_list(), k
        assert o.serialize() == n.serialize(), k
        if co == EBUSY:
            busy = True
            break
        seqs = [s + [t] for s, t in zip(seqs, decode_tokens(k, len(seqs)))]
    if not busy:
        assert o.batch_commit(seqs, ro, to["nodes"]) == n.batch_commit(seqs, rn, tn["nodes"]) == OK
        assert o.serialize() == n.serialize()
        assert o.free_list() == n.free_list()
    if pool < 1000:
        assert o.stats()[7] > 0                            # these pools really evict
    assert busy == (pool == 500)
