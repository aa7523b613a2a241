"""Seeded random operation streams over a radix tree + allocator, and
structural checks on the canonical dump.  Shared by the oracle pins and the
native-vs-oracle parity tests (it holds no tree logic of its own)."""
import numpy as np


def parse_dump(buf):
    """Canonical DFS dump -> list of node dicts in DFS order."""
    out, i = [], 0
    while i < len(buf):
        nid, par, la, lock, n = buf[i:i + 5]
        label = list(buf[i + 5:i + 5 + n])
        slots = list(buf[i + 5 + n:i + 5 + 2 * n])
        out.append(dict(id=nid, parent=par, last_access=la, lock=lock, label=label, slots=slots))
        i += 5 + 2 * n
    return out


def check_structure(nodes):
    """No two children share a first token; non-root labels non-empty;
    locks >= 0; children appear in ascending first-token order."""
    kids = {}
    for nd in nodes:
        if nd["id"] != 0:
            assert len(nd["label"]) > 0, nd
        assert nd["lock"] >= 0, nd
        kids.setdefault(nd["parent"], []).append(nd["label"][0] if nd["label"] else None)
    for par, firsts in kids.items():
        if par == -1:
            continue
        assert len(firsts) == len(set(firsts)), (par, firsts)
        assert firsts == sorted(firsts)


def paths(nodes):
    """node id -> (full token path from the root, start depth)."""
    by = {nd["id"]: nd for nd in nodes}
    memo = {0: []}

    def get(i):
        if i not in memo:
            nd = by[i]
            memo[i] = get(nd["parent"]) + nd["label"]
        return memo[i]
    return {nd["id"]: (get(nd["id"]), len(get(nd["id"])) - len(nd["label"])) for nd in nodes}


def expected_victim(nodes):
    """Brute-force LRU pick: unlocked non-root leaf with min (last_access, id)."""
    parents = {nd["parent"] for nd in nodes}
    cands = [nd for nd in nodes if nd["id"] != 0 and nd["lock"] == 0 and nd["id"] not in parents]
    if not cands:
        return None
    return min(cands, key=lambda nd: (nd["last_access"], nd["id"]))


class BruteCache:
    """The set of cached prefixes: tuple(tok[:k]) -> slot of position k-1."""

    def __init__(self):
        self.c = {}

    def match(self, tok):
        m = 0
        for k in range(1, len(tok) + 1):
            if tuple(tok[:k]) in self.c:
                m = k
            else:
                break
        return m, [self.c[tuple(tok[:k])] for k in range(1, m + 1)]

    def insert(self, tok, slots):
        dup = []
        for k in range(1, len(tok) + 1):
            key = tuple(tok[:k])
            if key in self.c:
                if self.c[key] != slots[k - 1]:
                    dup.append(slots[k - 1])
            else:
                self.c[key] = slots[k - 1]
        return dup

    def drop_path(self, full, start):
        for k in range(start + 1, len(full) + 1):
            del self.c[tuple(full[:k])]


def op_stream(seed, n_ops, vocab, max_len):
    """Yields (op, args) tuples; the driver supplies slots and node ids."""
    rng = np.random.default_rng(seed)
    for _ in range(n_ops):
        r = rng.random()
        L = int(rng.integers(1, max_len + 1))
        tok = rng.integers(0, vocab, size=L).tolist()
        if r < 0.30:
            yield "match", tok, bool(rng.random() < 0.5)
        elif r < 0.65:
            yield "insert", tok, None
        elif r < 0.75:
            yield "unlock", None, int(rng.integers(0, 1 << 30))
        elif r < 0.85:
            yield "evict", None, int(rng.integers(1, 8))
        elif r < 0.92:
            yield "alloc", None, int(rng.integers(0, 6))
        else:
            yield "free", None, int(rng.integers(0, 1 << 30))


OK, EINVAL, ENOSPC, EBUSY = 0, -1, -2, -3


def simulate_evict(nodes, want):
    """Brute-force eviction on a parsed dump: repeatedly drop the LRU
    unlocked leaf until `want` tokens are freed.  Returns (status, victims)."""
    nodes = [dict(nd) for nd in nodes]
    freed, victims = 0, []
    while freed < want:
        v = expected_victim(nodes)
        if v is None:
            return EBUSY, victims
        victims.append(v)
        freed += len(v["slots"])
        nodes = [nd for nd in nodes if nd["id"] != v["id"]]
    return OK, victims


def drive(trees, seed, n_ops, pool, vocab, max_len):
    """Apply one seeded op stream to every tree in `trees` (objects with the
    Python tree API), checking each against a brute-force model of the cached
    prefix set, the LRU rule, slot conservation and structure, and all trees
    against each other (outputs and canonical dumps) after every op."""
    brute = BruteCache()
    held_nodes, held_slots = [], []
    rng = np.random.default_rng(seed + 1)
    counts = dict(match=0, insert=0, evict=0, evicted_nodes=0, split=0)

    def same(vals):
        for v in vals[1:]:
            assert v == vals[0], (vals[0], v)
        return vals[0]

    def evict_checked(want):
        before = parse_dump(trees[0].serialize())
        fifo0 = trees[0].free_list()
        st_exp, victims = simulate_evict(before, want)
        res = same([t.evict(want) for t in trees])
        assert res[0] == st_exp
        assert res[1] == sum(len(v["slots"]) for v in victims)
        tail = [s for v in victims for s in v["slots"]]
        assert trees[0].free_list() == fifo0 + tail
        pth = paths(before)
        for v in victims:
            brute.drop_path(*pth[v["id"]])
        counts["evict"] += 1
        counts["evicted_nodes"] += len(victims)
        return res

    for op, tok, arg in op_stream(seed, n_ops, vocab, max_len):
        if op == "match":
            n_before = len(parse_dump(trees[0].serialize()))
            m, slots, nid = same([t.match(tok) for t in trees])
            assert (m, slots) == brute.match(tok)
            counts["split"] += len(parse_dump(trees[0].serialize())) - n_before
            counts["match"] += 1
            if arg and nid != 0:
                assert same([t.lock(nid) for t in trees]) == OK
                held_nodes.append(nid)
        elif op == "insert":
            n = len(tok)
            st, sl = same([t.alloc(n) for t in trees])
            if st == ENOSPC:
                assert len(trees[0].free_list()) < n
                evict_checked(n - len(trees[0].free_list()))
                st, sl = same([t.alloc(n) for t in trees])
                if st != OK:
                    continue
            fifo0 = trees[0].free_list()
            m_b, _ = brute.match(tok)
            dup = brute.insert(tok, sl)
            m = same([t.insert(tok, sl) for t in trees])
            assert m == m_b
            assert trees[0].free_list() == fifo0 + dup
            counts["insert"] += 1
        elif op == "unlock":
            if held_nodes:
                nid = held_nodes.pop(arg % len(held_nodes))
                assert same([t.unlock(nid) for t in trees]) == OK
        elif op == "evict":
            evict_checked(arg)
        elif op == "alloc":
            free_before = len(trees[0].free_list())
            st, sl = same([t.alloc(arg) for t in trees])
            assert (st == OK) == (free_before >= arg)
            held_slots += sl
        elif op == "free":
            if held_slots:
                k = arg % (len(held_slots) + 1)
                give = [held_slots.pop(int(rng.integers(0, len(held_slots)))) for _ in range(min(k, len(held_slots)))]
                assert same([t.free(give) for t in trees]) == OK
        dumps = same([list(t.serialize()) for t in trees])
        nodes = parse_dump(dumps)
        check_structure(nodes)
        owned = [s for nd in nodes for s in nd["slots"]]
        assert sorted(owned + trees[0].free_list() + held_slots) == list(range(pool))
        st = same([list(t.stats()) for t in trees])
        # the first five stats are sums over the dump and the free list
        non_root = [nd for nd in nodes if nd["id"] != 0]
        assert st[:5] == [sum(len(nd["label"]) for nd in non_root), len(trees[0].free_list()),
                          sum(len(nd["label"]) for nd in non_root if nd["lock"] == 0),
                          sum(len(nd["label"]) for nd in non_root if nd["lock"] > 0), len(non_root)], st
    return counts
