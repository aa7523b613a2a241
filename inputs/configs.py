"""Seeded synthetic workloads: token sequences, shapes and pool sizes.

Each workload is a list of phases.  A phase is one batch of token sequences
that goes through the same host path (prepare, scatter the new tokens' K/V,
attend, commit).  "setup" phases only fill the cache; "extend" and "decode"
phases are the ones whose attention is checked and timed.

The shapes follow the prefix-sharing patterns the SGLang article describes for
RadixAttention (few-shot batches sharing examples, fork/self-consistency trees,
multi-turn chat sessions; unite.ai "SGLang: Efficient Execution of Structured
Language Model Programs", section "SGLang: Modelo de programacion y
metodologia", the nine-step RadixAttention walkthrough).  The pages print no
token data; every token id here is drawn uniformly from [0, 32000).

Nothing in this module computes attention or walks a radix tree.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

VOCAB = 32000


@dataclass
class Shape:
    name: str
    hq: int
    hkv: int
    d: int
    dtype: str          # "f32" or "bf16"
    pool: int           # token slots in the KV pool
    seed: int           # seeds tokens, content and the free-list permutation
    q_scale: float = 1.0


@dataclass
class Phase:
    kind: str                       # "setup" | "extend" | "decode"
    seqs: list = field(default_factory=list)


def free_list(pool: int, seed: int) -> np.ndarray:
    """Initial free-slot order: a seeded permutation of [0, pool)."""
    rng = np.random.Generator(np.random.PCG64(seed ^ 0x5EED_F1F0))
    return rng.permutation(pool).astype(np.int32)


def _fresh(rng, n):
    return rng.integers(0, VOCAB, size=n, dtype=np.int64).astype(np.int32).tolist()


def _distinct_first(rng, count, lengths, avoid=()):
    """`count` fresh segments whose first tokens are pairwise distinct."""
    firsts = set(avoid)
    out = []
    for i in range(count):
        seg = _fresh(rng, lengths[i])
        if lengths[i] > 0:
            while seg[0] in firsts:
                seg[0] = int(rng.integers(0, VOCAB))
            firsts.add(seg[0])
        out.append(seg)
    return out


def c1():
    """Tiny fp32 extend: 4 requests share a cached 64-token prefix, +16 each."""
    s = Shape("c1", 4, 4, 64, "f32", 512, 1)
    rng = np.random.Generator(np.random.PCG64(s.seed))
    prefix = _fresh(rng, 64)
    tails = _distinct_first(rng, 4, [16] * 4)
    return s, [Phase("setup", [prefix]), Phase("extend", [prefix + t for t in tails])]


def c2(q_scale=1.0, name="c2"):
    """Llama-7B-shaped few-shot extend: 64 requests share a 1024-token prefix,
    each extends 128 fresh tokens; 32 q/kv heads, D=128, bf16, 2^20 slots."""
    s = Shape(name, 32, 32, 128, "bf16", 1 << 20, 2, q_scale)
    rng = np.random.Generator(np.random.PCG64(s.seed))
    prefix = _fresh(rng, 1024)
    tails = _distinct_first(rng, 64, [128] * 64)
    return s, [Phase("setup", [prefix]), Phase("extend", [prefix + t for t in tails])]


def c2s():
    """c2 with Q scaled by 8: peaked softmax, |o| ~ 1 (parity only)."""
    return c2(8.0, "c2s")


def _c3_lengths(rng):
    """The 4-ary depth-3 shared tree of the decode workload: edge lengths and
    per-request context lengths."""
    e1 = rng.integers(64, 513, size=4)
    e2 = rng.integers(64, 513, size=16)
    e3 = rng.integers(64, 513, size=64)
    shared = np.array([e1[r // 64] + e2[r // 16] + e3[r // 4] for r in range(256)])
    want = rng.integers(512, 4097, size=256)
    L = np.maximum(want, shared + 1)
    return e1, e2, e3, shared, L


def c3():
    """Llama-7B-shaped decode: 256 requests under a 4-ary radix tree of depth 3
    (edges U{64..512}) with private tails, contexts U{512..4096}, one new
    token each; 32/32 heads, D=128, bf16, 2^20 slots."""
    s = Shape("c3", 32, 32, 128, "bf16", 1 << 20, 3)
    rng = np.random.Generator(np.random.PCG64(s.seed))
    e1, e2, e3, shared, L = _c3_lengths(rng)
    lvl1 = _distinct_first(rng, 4, e1)
    lvl2 = []
    for a in range(4):
        lvl2 += _distinct_first(rng, 4, e2[4 * a:4 * a + 4])
    lvl3 = []
    for b in range(16):
        lvl3 += _distinct_first(rng, 4, e3[4 * b:4 * b + 4])
    p1 = [lvl1[a] for a in range(4)]
    p2 = [p1[b // 4] + lvl2[b] for b in range(16)]
    p3 = [p2[c // 4] + lvl3[c] for c in range(64)]
    full = []
    for c in range(64):
        tails = _distinct_first(rng, 4, [int(L[4 * c + i] - shared[4 * c + i]) for i in range(4)])
        full += [p3[c] + t for t in tails]
    hist = [seq[:-1] for seq in full]
    return s, [Phase("setup", p1), Phase("setup", p2), Phase("setup", p3),
               Phase("setup", hist), Phase("decode", full)]


def c3ns():
    """No-share control: c3's context lengths, every context private."""
    s = Shape("c3ns", 32, 32, 128, "bf16", 1 << 20, 3)
    rng = np.random.Generator(np.random.PCG64(s.seed))
    _, _, _, _, L = _c3_lengths(rng)
    full = _distinct_first(rng, 256, [int(x) for x in L])
    return s, [Phase("setup", [q[:-1] for q in full]), Phase("decode", full)]


def c4():
    """Llama-70B-shaped GQA: 64 q / 8 kv heads, D=128, bf16.  128 requests
    share a 2048-token prefix; requests 0-63 extend 256 tokens (contexts
    U{2304..8192}), requests 64-127 decode one token (U{2049..8192})."""
    s = Shape("c4", 64, 8, 128, "bf16", 1 << 20, 4)
    rng = np.random.Generator(np.random.PCG64(s.seed))
    prefix = _fresh(rng, 2048)
    n = [256] * 64 + [1] * 64
    L = np.concatenate([rng.integers(2304, 8193, size=64), rng.integers(2049, 8193, size=64)])
    after = _distinct_first(rng, 128, [int(L[r] - 2048) for r in range(128)])
    full = [prefix + after[r] for r in range(128)]
    hist = [full[r][: len(full[r]) - n[r]] for r in range(128)]
    return s, [Phase("setup", [prefix]), Phase("setup", hist),
               Phase("extend", full[:64]), Phase("decode", full[64:])]


def chat_trace(seed: int, sessions: int = 512, max_batch: int = 64):
    """Multi-turn chat: session s has U{1..8} turns; turn t appends a fresh
    segment of U{32..512} tokens and asks for segments 1..t.  Turns are
    interleaved in a seeded random order that keeps each session's order,
    then cut into batches of at most `max_batch` with no session twice in a
    batch.  Returns (batches, turn_of) where batches hold sequences and
    turn_of holds matching (session, turn) pairs."""
    rng = np.random.Generator(np.random.PCG64(seed))
    turns = rng.integers(1, 9, size=sessions)
    segs = []
    firsts = set()
    for sidx in range(sessions):
        lens = rng.integers(32, 513, size=int(turns[sidx]))
        ss = [_fresh(rng, int(x)) for x in lens]
        while ss[0][0] in firsts:
            ss[0][0] = int(rng.integers(0, VOCAB))
        firsts.add(ss[0][0])
        segs.append(ss)
    order = np.repeat(np.arange(sessions), turns)
    rng.shuffle(order)
    nxt = np.zeros(sessions, dtype=np.int64)
    batches, tags = [], []
    cur, cur_tags, in_batch = [], [], set()
    for sidx in order.tolist():
        if len(cur) == max_batch or sidx in in_batch:
            batches.append(cur); tags.append(cur_tags)
            cur, cur_tags, in_batch = [], [], set()
        t = int(nxt[sidx]); nxt[sidx] += 1
        seq = [tok for seg in segs[sidx][: t + 1] for tok in seg]
        cur.append(seq); cur_tags.append((sidx, t)); in_batch.add(sidx)
    if cur:
        batches.append(cur); tags.append(cur_tags)
    return batches, tags


def c5(pool=1 << 21, name="c5"):
    """Mixtral-8x7B-shaped multi-turn chat: 32 q / 8 kv heads, D=128, bf16,
    512 sessions; LRU eviction and reinsertion under the pool limit."""
    s = Shape(name, 32, 8, 128, "bf16", pool, 5)
    batches, _ = chat_trace(s.seed)
    return s, [Phase("extend", b) for b in batches]


def c5e():
    """c5's trace under a 2^19-slot pool, so eviction binds."""
    return c5(1 << 19, "c5e")


def c4tp8():
    """One GPU's share of c4 under 8-way tensor parallelism over heads: the
    same requests, with this GPU's 8 q heads and 1 kv head."""
    s, phases = c4()
    return Shape("c4tp8", 8, 1, s.d, s.dtype, s.pool, s.seed), phases


def c5tp8():
    """One GPU's share of c5 under 8-way tensor parallelism: 4 q heads and 1
    kv head per GPU, the same chat trace."""
    s, phases = c5()
    return Shape("c5tp8", 4, 1, s.d, s.dtype, s.pool, s.seed), phases


def mm_trace(seed: int = 9, images: int = 24, questions: int = 5, image_bytes: int = 4096,
             system: int = 35, max_batch: int = 16):
    """LLaVA-style visual question answering: every request is a shared
    system prompt, one image and a question of U{8..48} fresh text tokens;
    each image is asked `questions` questions.  Images are seeded random
    bytes (their content, which the runtime hashes); requests come in a
    seeded interleaved order, cut into batches of at most `max_batch` with no
    image twice in a batch.  Returns (system tokens, image bytes list,
    batches of (image index, question tokens))."""
    rng = np.random.Generator(np.random.PCG64(seed))
    sys_tokens = _fresh(rng, system)
    blobs = [rng.integers(0, 256, size=image_bytes, dtype=np.uint8).tobytes() for _ in range(images)]
    order = np.repeat(np.arange(images), questions)
    rng.shuffle(order)
    batches, cur, in_batch = [], [], set()
    for img in order.tolist():
        if len(cur) == max_batch or img in in_batch:
            batches.append(cur)
            cur, in_batch = [], set()
        cur.append((img, _fresh(rng, int(rng.integers(8, 49)))))
        in_batch.add(img)
    if cur:
        batches.append(cur)
    return sys_tokens, blobs, batches


def mm():
    """LLaVA-v1.5-7B-shaped: 32 q / 32 kv heads, D=128, bf16; 576 image
    positions per image (a 336-pixel image in 14-pixel patches); the
    mm_trace requests.  Returns (shape, trace, image positions)."""
    s = Shape("mm", 32, 32, 128, "bf16", 1 << 20, 9)
    return s, mm_trace(s.seed), 576


CONFIGS = {"c1": c1, "c2": c2, "c2s": c2s, "c3": c3, "c3ns": c3ns, "c4": c4, "c5": c5, "c5e": c5e,
           "c4tp8": c4tp8, "c5tp8": c5tp8}


def build(name: str):
    return CONFIGS[name]()


def tiny(seed: int, hq=4, hkv=2, d=64, dtype="f32", pool=4096, n_req=5, prefix=70,
         new=(1, 37, 64, 3, 129)):
    """A small ragged workload for parity tests: a shared prefix, ragged new
    lengths that cross tile boundaries, and one request with no prefix."""
    s = Shape(f"tiny{seed}", hq, hkv, d, dtype, pool, seed)
    rng = np.random.Generator(np.random.PCG64(seed))
    pre = _fresh(rng, prefix)
    tails = _distinct_first(rng, n_req, list(new[:n_req]), avoid=(pre[0],))
    seqs = [pre + t for t in tails[:-1]] + [tails[-1]]
    return s, [Phase("setup", [pre]), Phase("extend", seqs)]
