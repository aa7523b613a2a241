"""Oracle of prefix-shared ("cascade") decode: the plan and its split arithmetic.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the native library and never imports it.

Why this exists.  RadixAttention keeps a shared prompt prefix once in the KV
pool, so requests whose table rows begin with the same slots read the same
K/V there (unite.ai, "SGLang: Efficient Execution of Structured Language
Model Programs", section "Introduccion a SGLang", RadixAttention bullet).
The pages stop at reusing the cache; reading each shared run once per decode
batch is an extension taken here.  It rests on one identity: softmax
attention over a union of disjoint key ranges equals the combination of the
per-range states (m, l, acc), each rescaled to the common maximum.

The plan, as defined here (every step integer and deterministic):

  * row r counts only its first L_r - 1 keys as shareable: the decode
    query's own key (position L_r - 1) is always private;
  * perm = request ids sorted by that truncated row, compared slot by slot
    as a sequence (a proper prefix sorts first), ties by request id;
  * walking request r's positions t = 0 .. L_r - 2, the member set of t is
    every request whose truncated row has the same first t + 1 slots.  A
    run is a maximal stretch of positions with one member set of size >= 2;
    the member sets only shrink along a row;
  * folding: along each row, a run is emitted as a segment
    [eff_start, run_end) when run_end - eff_start >= min_keys, where
    eff_start is the end of the last emitted segment (0 at the start);
    otherwise its keys are carried into the next run.  The private tail of
    r is [eff_start, L_r) after its last emitted segment (never empty);
  * a segment's members form one contiguous block of perm; segments are
    ordered by (first position in perm, key_begin), which is a preorder of
    the prefix tree.  Each is cut into chunks of seg_chunk keys, and each
    chunk into member groups of at most max_members (perm order); a job is
    (key_begin, key_end, perm_first, count, rec_off);
  * records of r: one per chunk of each of its segments, in path order, then
    one per tail_chunk keys of its tail.  rec_indptr is their exclusive
    prefix sum over r; rec_off of a job is the index, within each member's
    list, of that chunk's record (the same for every member);
  * tail_splits = the largest number of tail records of any request.
"""
from __future__ import annotations

import math

import numpy as np

from oracle.attention import merge_states, partial_state


def _ceil_div(a, b):
    return -(-a // b)


def plan(req_to_token, seq_lens, seg_chunk, tail_chunk, min_keys=1, max_members=None):
    """Builds the plan from the host table.  Returns a dict with perm,
    rec_indptr, tail_begin, jobs (list of 5-tuples), tail_splits."""
    B = len(seq_lens)
    L = [int(x) for x in seq_lens]
    rows = [tuple(int(s) for s in req_to_token[r][: max(L[r] - 1, 0)]) for r in range(B)]
    if max_members is None:
        max_members = max(B, 1)
    perm = sorted(range(B), key=lambda r: (rows[r], r))
    pos = {r: i for i, r in enumerate(perm)}

    # explicit, uncompressed prefix tree: one node per distinct prefix of a
    # truncated row, with the requests that pass through it
    child = [dict()]
    members = [[]]
    node_path = []
    for r in range(B):
        node, nodes = 0, []
        for s in rows[r]:
            nxt = child[node].get(s)
            if nxt is None:
                nxt = len(child)
                child[node][s] = nxt
                child.append(dict())
                members.append([])
            members[nxt].append(r)
            node = nxt
            nodes.append(node)
        node_path.append(nodes)

    segments = {}                 # (key_begin, key_end, perm_first) -> members in perm order
    tail_begin = [0] * B
    path = [[] for _ in range(B)]
    for r in range(B):
        eff = 0
        t = 0
        n = len(rows[r])
        nodes = node_path[r]
        while t < n:
            # member sets only shrink along a row, so equal size = equal set
            size = len(members[nodes[t]])
            end = t
            while end < n and len(members[nodes[end]]) == size:
                end += 1
            if size >= 2 and end - eff >= min_keys:
                ms = members[nodes[end - 1]]
                first = min(pos[m] for m in ms)
                segments[(eff, end, first)] = sorted(ms, key=lambda m: pos[m])
                path[r].append((eff, end, first))
                eff = end
            t = end
        tail_begin[r] = eff

    # records: segment chunks in path order, then the tail chunks
    nrec = []
    rec_of = {}                   # (segment, r) -> record index of its first chunk within r
    for r in range(B):
        k = 0
        for seg in path[r]:
            rec_of[(seg, r)] = k
            k += _ceil_div(seg[1] - seg[0], seg_chunk)
        nrec.append(k + _ceil_div(L[r] - tail_begin[r], tail_chunk))
    rec_indptr = [0]
    for r in range(B):
        rec_indptr.append(rec_indptr[-1] + nrec[r])

    jobs = []
    for seg in sorted(segments, key=lambda s: (s[2], s[0])):
        ms = segments[seg]
        base = rec_of[(seg, ms[0])]
        assert all(rec_of[(seg, m)] == base for m in ms)
        kb, ke, first = seg
        assert [pos[m] for m in ms] == list(range(first, first + len(ms)))
        for c in range(_ceil_div(ke - kb, seg_chunk)):
            b0 = kb + c * seg_chunk
            b1 = min(ke, b0 + seg_chunk)
            for g0 in range(0, len(ms), max_members):
                jobs.append((b0, b1, first + g0, min(max_members, len(ms) - g0), base + c))
    tail_splits = max([_ceil_div(L[r] - tail_begin[r], tail_chunk) for r in range(B)], default=0)
    return {"perm": perm, "rec_indptr": rec_indptr, "tail_begin": tail_begin, "jobs": jobs,
            "tail_splits": tail_splits}


def record_ranges(p, seq_lens, tail_chunk):
    """Key range of every record: {(r, record index within r): (begin, end)}.
    The keys of a shared record are read from the members' common slots."""
    out = {}
    for kb, ke, first, count, rec_off in p["jobs"]:
        for m in p["perm"][first:first + count]:
            assert (m, rec_off) not in out
            out[(m, rec_off)] = (kb, ke)
    for r, L in enumerate(seq_lens):
        L = int(L)
        n = p["rec_indptr"][r + 1] - p["rec_indptr"][r]
        ntail = _ceil_div(L - p["tail_begin"][r], tail_chunk)
        for s in range(ntail):
            b0 = p["tail_begin"][r] + s * tail_chunk
            out[(r, n - ntail + s)] = (b0, min(L, b0 + tail_chunk))
    return out


def decode(q, pool, req_to_token, seq_lens, hq, hkv, p, tail_chunk, scale=None, requests=None):
    """Decode attention evaluated record by record: each record's (m, l, acc)
    over its key range in float64, merged per (request, q head) in record
    order.  Equals attention.decode up to rounding when the plan covers
    every key of every request exactly once."""
    q = np.asarray(q, dtype=np.float64)
    B, _, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    group = hq // hkv
    ranges = record_ranges(p, seq_lens, tail_chunk)
    o = np.full((B, hq, D), np.nan)
    lse = np.full((B, hq), np.nan)
    for r in (range(B) if requests is None else requests):
        n = p["rec_indptr"][r + 1] - p["rec_indptr"][r]
        K, V = pool.gather(req_to_token[r][: int(seq_lens[r])])
        for h in range(hq):
            g = h // group
            states = []
            for k in range(n):
                b0, b1 = ranges[(r, k)]
                states.append(partial_state(q[r, h, :], K[b0:b1, g, :], V[b0:b1, g, :], scale))
            o[r, h, :], lse[r, h] = merge_states(states)
    return o, lse
