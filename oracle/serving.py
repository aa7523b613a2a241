"""Oracle serving loop for comparing queue orders (pure Python).

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the native library and never imports it.

The article (unite.ai, "SGLang: Efficient Execution of Structured Language
Model Programs", section "SGLang: Evaluacion y resultados") reports that its
cache-aware scheduling reaches about 96 % of the optimal cache hit rate; it
gives neither the rule nor the queue model.  Readings used here:

  * a trace is a set of turns (session, t); turn t of a session can run only
    after its turn t-1 has run (its prompt contains that history); all turns
    wait from the start, in a given arrival order;
  * each step takes at most `max_batch` runnable turns, in arrival order
    ("fcfs") or by OracleTree.schedule ("cache": longest reusable prefix
    first, ties in arrival order), and runs them as one batch
    (batch_prepare, then batch_commit);
  * hit rate = tokens whose KV was reused / all prompt tokens.
"""
from __future__ import annotations

from .radix import OK


def serve(tree, turns, arrival, policy, max_batch=64):
    """turns: {(session, t): token list}; arrival: list of (session, t).
    Returns dict(steps, prompt_tokens, reused_tokens, hit_rate, order) where
    order lists the turns in the order they ran and reused[i] their reuse."""
    done = set()
    waiting = list(arrival)              # arrival order
    ran, reused = [], []
    steps = 0
    while waiting:
        runnable = [st for st in waiting if st[1] == 0 or (st[0], st[1] - 1) in done]
        if policy == "fcfs":
            pick = runnable[:max_batch]
        elif policy == "cache":
            order, _ = tree.schedule([turns[st] for st in runnable])
            pick = [runnable[i] for i in order[:max_batch]]
        else:
            raise ValueError(policy)
        seqs = [turns[st] for st in pick]
        status, tb = tree.batch_prepare(seqs)
        if status != OK:
            raise RuntimeError(f"batch_prepare failed with {status}")
        tree.batch_commit(seqs, tb["req_to_token"], tb["nodes"])
        ran.extend(pick)
        reused.extend(int(x) for x in tb["prefix_lens"])
        for st in pick:
            done.add(st)
        picked = set(pick)
        waiting = [st for st in waiting if st not in picked]
        steps += 1
    prompt = sum(len(turns[st]) for st in ran)
    return dict(steps=steps, prompt_tokens=prompt, reused_tokens=sum(reused),
                hit_rate=sum(reused) / max(prompt, 1), order=ran, reused=reused)
