"""Queue order for a RadixAttention cache: first come first served, or
cache-aware (the article, unite.ai, "SGLang: Efficient Execution of Structured
Language Model Programs", section "SGLang: Evaluacion y resultados": SGLang's
cache-aware scheduling keeps the cache hit rate near the optimum).

`run_queue` drives a native tree (rkv.Tree) through a multi-turn workload: a
session's turn t becomes runnable once its turn t-1 has run (its prompt holds
that history); every step takes at most `max_batch` runnable turns, in
arrival order or by rkv_schedule (longest reusable prefix first, ties in
arrival order), and runs them as one batch (batch_prepare + batch_commit).
The ranking runs in librkv; this module only keeps the queue.
"""
from __future__ import annotations

from . import rkv


def run_queue(tree, turns, arrival, policy, max_batch=64):
    """turns: {(session, t): token list}; arrival: the turns in arrival order.
    Returns dict(steps, prompt_tokens, reused_tokens, hit_rate, order, reused)
    with the turns in the order they ran and the cached prefix each reused."""
    if policy not in ("fcfs", "cache"):
        raise ValueError(f"unknown policy {policy!r}")
    pos = {st: i for i, st in enumerate(arrival)}
    finished = set()
    pending = sorted(arrival, key=pos.__getitem__)
    order, reused = [], []
    steps = 0
    while pending:
        ready = [st for st in pending if st[1] == 0 or (st[0], st[1] - 1) in finished]
        if policy == "cache":
            rank, _ = tree.schedule([turns[st] for st in ready])
            batch = [ready[int(i)] for i in rank[:max_batch]]
        else:
            batch = ready[:max_batch]
        seqs = [turns[st] for st in batch]
        code, tb = tree.batch_prepare(seqs)
        if code != rkv.OK:
            raise rkv.RkvError(code, "batch_prepare: eviction cannot free enough slots")
        tree.batch_commit(seqs, tb["req_to_token"], tb["nodes"])
        order += batch
        reused += [int(x) for x in tb["prefix_lens"]]
        finished.update(batch)
        taken = set(batch)
        pending = [st for st in pending if st not in taken]
        steps += 1
    prompt = sum(len(turns[st]) for st in order)
    return dict(steps=steps, prompt_tokens=prompt, reused_tokens=sum(reused),
                hit_rate=sum(reused) / max(prompt, 1), order=order, reused=reused)
