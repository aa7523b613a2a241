"""Oracle radix tree + token-slot allocator (naive, pure Python).

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the native library and never imports it.

What the pages fix (unite.ai, "SGLang: Efficient Execution of Structured
Language Model Programs", Spanish edition):
  * section "Introduccion a SGLang", RadixAttention bullet: the runtime keeps
    an LRU cache of KV inside a radix tree and uses the tree for matching,
    insertion and eviction;
  * section "SGLang: Modelo de programacion y metodologia", nine-step
    walkthrough: every edge is labelled with a token sequence (intro to the
    steps); a new prompt reuses the KV of its longest cached prefix and its new
    turn becomes a new node (Step 3); a node is split so that two sequences
    share their common part (Steps 4 and 7); under a memory limit whole nodes
    are evicted, least recently used first (Steps 5, 8 and 9).

Everything else below is a reading of those statements, chosen so that two
implementations can agree bit for bit:

  * a global tick, +1 at the start of every match and every insert;
  * match walks from the root, splits an edge where the query ends or diverges
    inside it, stamps every node on the root path with the tick, and returns
    the matched length, the matched slots and the stop node;
  * insert walks the same way, keeps the tree's slots for positions already
    cached, hands the caller's differing duplicates back to the free list in
    position order, and hangs the rest as a new leaf;
  * a split keeps the lower node's id; the new upper node copies the lower
    node's tick and lock count;
  * lock/unlock add +-1 on every node from the given node up to (not
    including) the root;
  * evict frees whole unlocked leaves, smallest (last_access, id) first,
    appending their slots to the free-list tail in label order, until at least
    the wanted number of tokens is freed (EBUSY if it runs out of candidates);
  * the allocator is a FIFO of slot ids; alloc pops from the head, free
    appends to the tail;
  * batch_prepare matches each request capped at its length minus one (so
    every request computes at least its last token), locks the stop node,
    evicts if the free list is short, pops all new slots and fills the index
    tables; batch_commit inserts each full sequence and unlocks;
  * batch_append continues a prepared, uncommitted batch by one decode
    position per request without matching again: a finished turn, answer
    included, becomes one node (Step 3), so generated tokens reach the tree
    only at the commit.  It evicts if fewer slots than requests are free
    (EBUSY if it cannot), pops one slot per request in request order, writes
    it after the row's last entry and extends the length.

The implementation is deliberately naive: children are a Python list scanned
linearly, the LRU leaf is found by scanning every node.
"""
from __future__ import annotations

from collections import deque

OK, EINVAL, ENOSPC, EBUSY = 0, -1, -2, -3


class _Node:
    __slots__ = ("id", "label", "slots", "parent", "children", "last_access", "lock")

    def __init__(self, nid, label, slots, parent, last_access, lock):
        self.id = nid
        self.label = list(label)
        self.slots = list(slots)
        self.parent = parent          # _Node or None for the root
        self.children = []            # list of _Node, unordered
        self.last_access = last_access
        self.lock = lock


class OracleTree:
    """Radix tree over token sequences plus a FIFO slot allocator."""

    def __init__(self, pool_slots: int, initial_free=None):
        self.pool_slots = int(pool_slots)
        order = range(self.pool_slots) if initial_free is None else [int(s) for s in initial_free]
        self.fifo = deque(order)
        self.root = _Node(0, [], [], None, 0, 0)
        self.nodes = {0: self.root}
        self.next_id = 1
        self.tick = 0
        self.matched_total = 0
        self.prompt_total = 0
        self.evicted_total = 0
        self.evicted_ids = []          # every evicted node id, in eviction order

    # ------------------------------------------------------------------ helpers
    def _child(self, node, first_token):
        for c in node.children:
            if c.label[0] == first_token:
                return c
        return None

    def _split(self, x, k):
        """Cut x's edge after k tokens; the new upper node takes x's place."""
        parent = x.parent
        up = _Node(self.next_id, x.label[:k], x.slots[:k], parent, x.last_access, x.lock)
        self.next_id += 1
        self.nodes[up.id] = up
        parent.children[parent.children.index(x)] = up
        x.label = x.label[k:]
        x.slots = x.slots[k:]
        x.parent = up
        up.children.append(x)
        return up

    def _walk(self, tok):
        """Descend along tok, splitting where it ends or diverges inside an
        edge.  Returns (stop node, matched length, matched slots, path)."""
        node, m, slots, path = self.root, 0, [], [self.root]
        while m < len(tok):
            c = self._child(node, tok[m])
            if c is None:
                break
            k = 0
            while k < len(c.label) and m + k < len(tok) and c.label[k] == tok[m + k]:
                k += 1
            if k < len(c.label):
                c = self._split(c, k)
            # c now spans exactly the k matched tokens; the next lookup finds
            # no child when the query diverged or ended inside the old edge
            slots.extend(c.slots)
            m += k
            node = c
            path.append(c)
        return node, m, slots, path

    # ------------------------------------------------------------------ core ops
    def peek(self, tok):
        """Length of the longest cached prefix of tok, leaving the tree
        untouched (no split, no tick): what a scheduler ranks requests by."""
        tok = [int(t) for t in tok]
        node, m = self.root, 0
        while m < len(tok):
            c = self._child(node, tok[m])
            if c is None:
                break
            k = 0
            while k < len(c.label) and m + k < len(tok) and c.label[k] == tok[m + k]:
                k += 1
            m += k
            if k < len(c.label):
                break
            node = c
        return m

    def schedule(self, seqs):
        """Cache-aware order of a waiting queue (the article, section "SGLang:
        Evaluacion y resultados": cache-aware scheduling approaches the optimal
        hit rate; its rule is not given).  Reading: rank by the prefix a batch
        would reuse now (peek of the first L-1 tokens, as batch_prepare caps
        its match), longest first, ties in queue order.  Returns (order,
        matched)."""
        matched = [self.peek(list(s)[: len(s) - 1]) if len(s) > 0 else 0 for s in seqs]
        order = sorted(range(len(seqs)), key=lambda q: (-matched[q], q))
        return order, matched

    def match(self, tok):
        """Longest cached prefix of tok: (matched length, slots, stop node id)."""
        tok = [int(t) for t in tok]
        self.tick += 1
        node, m, slots, path = self._walk(tok)
        for n in path:
            n.last_access = self.tick
        return m, slots, (node.id if m > 0 else 0)

    def lock(self, nid):
        if nid not in self.nodes:
            return EINVAL
        n = self.nodes[nid]
        while n is not self.root:
            n.lock += 1
            n = n.parent
        return OK

    def unlock(self, nid):
        if nid not in self.nodes:
            return EINVAL
        n = self.nodes[nid]
        p = n
        while p is not self.root:
            if p.lock <= 0:
                return EINVAL
            p = p.parent
        while n is not self.root:
            n.lock -= 1
            n = n.parent
        return OK

    def insert(self, tok, slots):
        """Insert tok with the caller's slots; returns the already-cached length."""
        tok = [int(t) for t in tok]
        slots = [int(s) for s in slots]
        if len(tok) != len(slots):
            return EINVAL
        self.tick += 1
        node, m, tree_slots, path = self._walk(tok)
        for i in range(m):
            if slots[i] != tree_slots[i]:
                self.fifo.append(slots[i])
        if m < len(tok):
            leaf = _Node(self.next_id, tok[m:], slots[m:], node, self.tick, 0)
            self.next_id += 1
            self.nodes[leaf.id] = leaf
            node.children.append(leaf)
            path.append(leaf)
        for n in path:
            n.last_access = self.tick
        return m

    def evict(self, want):
        """Free whole unlocked leaves, LRU first, until >= want tokens freed.
        Returns (status, freed)."""
        freed = 0
        while freed < want:
            best = None
            for n in self.nodes.values():
                if n is self.root or n.children or n.lock != 0:
                    continue
                if best is None or (n.last_access, n.id) < (best.last_access, best.id):
                    best = n
            if best is None:
                return EBUSY, freed
            self.fifo.extend(best.slots)
            freed += len(best.slots)
            self.evicted_total += len(best.slots)
            self.evicted_ids.append(best.id)
            best.parent.children.remove(best)
            del self.nodes[best.id]
        return OK, freed

    def alloc(self, n):
        if n < 0:
            return EINVAL, []
        if len(self.fifo) < n:
            return ENOSPC, []
        return OK, [self.fifo.popleft() for _ in range(n)]

    def free(self, slots):
        self.fifo.extend(int(s) for s in slots)
        return OK

    # ------------------------------------------------------------------ batches
    def batch_prepare(self, seqs, ld=None):
        """Match (capped at L-1), lock, evict if short, alloc, fill tables.

        Returns (status, tables) where tables holds req_to_token [B][ld] (-1
        past each length), prefix_lens, seq_lens, qo_indptr, new_slots, nodes.
        """
        B = len(seqs)
        lens = [len(s) for s in seqs]
        if ld is None:
            ld = max(lens) if lens else 0
        if any(L < 1 or L > ld for L in lens):
            return EINVAL, None
        pref, nodes, mslots = [], [], []
        for s in seqs:
            m, sl, nid = self.match(s[: len(s) - 1])
            self.lock(nid)
            pref.append(m); nodes.append(nid); mslots.append(sl)
        T = sum(L - p for L, p in zip(lens, pref))
        if len(self.fifo) < T:
            st, _ = self.evict(T - len(self.fifo))
            if st != OK:
                for nid in nodes:
                    self.unlock(nid)
                return EBUSY, None
        st, new = self.alloc(T)
        assert st == OK
        r2t = [[-1] * ld for _ in range(B)]
        indptr = [0]
        pos = 0
        for r in range(B):
            n = lens[r] - pref[r]
            row = mslots[r] + new[pos:pos + n]
            r2t[r][: lens[r]] = row
            pos += n
            indptr.append(pos)
            self.matched_total += pref[r]
            self.prompt_total += lens[r]
        return OK, dict(req_to_token=r2t, prefix_lens=pref, seq_lens=lens,
                        qo_indptr=indptr, new_slots=new, nodes=nodes)

    def batch_append(self, req_to_token, seq_lens):
        """One more position per request of a prepared batch; req_to_token
        (rows of length ld) and seq_lens are updated in place.  Returns
        (status, new_slots)."""
        B = len(seq_lens)
        if B == 0:
            return OK, []
        ld = len(req_to_token[0])
        if any(L < 1 or L >= ld for L in seq_lens):
            return EINVAL, None
        if len(self.fifo) < B:
            st, _ = self.evict(B - len(self.fifo))
            if st != OK:
                return EBUSY, None
        st, new = self.alloc(B)
        assert st == OK
        for r in range(B):
            req_to_token[r][seq_lens[r]] = new[r]
            seq_lens[r] += 1
        return OK, new

    def batch_commit(self, seqs, req_to_token, nodes):
        for r, s in enumerate(seqs):
            self.insert(s, req_to_token[r][: len(s)])
            st = self.unlock(nodes[r])
            if st != OK:
                return st
        return OK

    # ------------------------------------------------------------------ views
    def serialize(self):
        """DFS from the root, children by ascending first token; per node
        (id, parent id, last_access, lock, len, label..., slots...)."""
        out = []

        def visit(n):
            out.extend([n.id, -1 if n.parent is None else n.parent.id,
                        n.last_access, n.lock, len(n.label)])
            out.extend(n.label)
            out.extend(n.slots)
            for c in sorted(n.children, key=lambda c: c.label[0]):
                visit(c)

        visit(self.root)
        return out

    def stats(self):
        """[cached, free, evictable, locked, nodes, matched_total,
        prompt_total, evicted_total] (token counts except nodes)."""
        cached = evictable = locked = 0
        for n in self.nodes.values():
            if n is self.root:
                continue
            cached += len(n.label)
            if n.lock == 0:
                evictable += len(n.label)
            else:
                locked += len(n.label)
        return [cached, len(self.fifo), evictable, locked, len(self.nodes) - 1,
                self.matched_total, self.prompt_total, self.evicted_total]

    def tree_slots(self):
        out = []
        for n in self.nodes.values():
            out.extend(n.slots)
        return out

    def free_list(self):
        return list(self.fifo)
