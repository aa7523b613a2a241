"""Decode steps captured into a HIP graph (engine.StepGraph) and replayed.

A replay runs the same kernels on the same buffers as the eager calls, so its
outputs must equal the eager outputs bit for bit (the kernels accumulate in a
fixed order).  Every replay is checked, with eager work of the program
between replays; new query rows copied into the captured buffer must give
the eager result for those rows; and the eager path must still match the
float64 oracle on the batch (tests/gpu_runner)."""
import numpy as np
import pytest
import torch

from inputs import configs, content
from tests import gpu_runner as G

pytestmark = pytest.mark.gpu


def _setup(hq, hkv, d, lens, seed):
    from prefix_shared_kv_host_amd.engine import RadixKVCache
    rng = np.random.default_rng(seed)
    shared = [int(x) for x in rng.integers(0, 32000, 300)]
    seqs = []
    for i, L in enumerate(lens):
        tail = [int(x) for x in rng.integers(0, 32000, L)]
        tail[0] = 40000 + i
        seqs.append(shared + tail if i % 3 else tail)
    pool = 1 << 15
    cache = RadixKVCache(pool, hkv, d, torch.bfloat16, "cuda", configs.free_list(pool, seed))
    hseqs = [s[:-1] for s in seqs if len(s) > 1]
    hist = cache.prepare(hseqs)
    _, k, v = content.batch_rows(seed, hseqs, hist.host["prefix_lens"], hq, hkv, d, torch.bfloat16, "cuda", 1.0,
                                 with_q=False)
    cache.store(hist, k, v)
    cache.commit(hist)
    batch = cache.prepare(seqs)
    q, k, v = content.batch_rows(seed + 1, seqs, batch.host["prefix_lens"], hq, hkv, d, torch.bfloat16, "cuda",
                                 1.0, with_q=True)
    cache.store(batch, k, v)
    torch.cuda.synchronize()
    return cache, batch, q


@pytest.mark.parametrize("hq,hkv,d,cascade", [(8, 1, 128, False), (8, 1, 128, True), (32, 32, 128, False),
                                              (32, 32, 128, True), (16, 2, 64, True)])
def test_decode_graph_replays_equal_eager(hq, hkv, d, cascade):
    from prefix_shared_kv_host_amd.engine import StepGraph
    lens = [1, 5, 33, 64, 65, 200, 700, 1500, 3000] * 3
    cache, batch, q = _setup(hq, hkv, d, lens, seed=hq + d)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[0], hq, dtype=torch.float32, device="cuda")
    plan = cache.cascade_plan(batch, hq, seg_chunk=64, tail_chunk=256, min_keys=8) if cascade else None

    def step():
        if cascade:
            cache.decode_cascade(batch, q, plan=plan, o=o, lse=lse)
        else:
            cache.decode(batch, q, o=o, lse=lse)

    step()
    torch.cuda.synchronize()
    o_ref, lse_ref = o.clone(), lse.clone()
    g = StepGraph(step)
    q2 = torch.randn_like(q.float()).to(q.dtype)
    scratch = torch.zeros(1 << 20, device="cuda")
    for rep in range(4):
        o.fill_(0)
        lse.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), rep
        scratch.add_(1.0)                     # the program's own eager work between replays
        torch.cuda.synchronize()
    # new query rows in the captured buffer
    q_saved = q.clone()
    q.copy_(q2)
    g.replay()
    torch.cuda.synchronize()
    o_g, lse_g = o.clone(), lse.clone()
    step()
    torch.cuda.synchronize()
    assert torch.equal(o_g, o) and torch.equal(lse_g, lse)
    q.copy_(q_saved)
    G.log(f"graph decode {hq}/{hkv} d{d} cascade={cascade}: 5 replays equal the eager results")


def test_decode_graph_eager_path_matches_oracle():
    """The step the graph captures is the checked decode: the same batch
    shape through the oracle comparison of tests/gpu_runner."""
    shape = configs.Shape("graph-8-1-128", 8, 1, 128, "bf16", 1 << 15, 5)
    rng = np.random.default_rng(5)
    full = [[int(x) for x in rng.integers(0, 32000, L)] for L in (2, 65, 700, 1500)]
    for i, f in enumerate(full):
        f[0] = 50000 + i
    phases = [configs.Phase("setup", [f[:-1] for f in full]), configs.Phase("decode", full)]
    res, _ = G.run(shape, phases, content_device="cpu")
    G.check(res, "bf16", "graph batch, eager")


def test_full_step_graph_replays_equal_eager():
    """A whole serving step in one graph: kv_scatter + attn_extend for an
    extend batch, kv_scatter + prefix-shared decode for a decode batch (the
    step bench.py times), replayed with the pool rows rewritten each time."""
    from prefix_shared_kv_host_amd.engine import RadixKVCache, StepGraph
    hq, hkv, d, seed = 8, 2, 128, 91
    rng = np.random.default_rng(seed)
    pool = 1 << 16
    cache = RadixKVCache(pool, hkv, d, torch.bfloat16, "cuda", configs.free_list(pool, seed))
    shared = [int(x) for x in rng.integers(0, 32000, 500)]
    ext_seqs = [shared + [int(x) for x in rng.integers(0, 32000, n)] for n in (1, 17, 64, 130)]
    dec_full = [shared + [int(x) for x in rng.integers(0, 32000, n)] + [7] for n in (3, 40, 900)]
    setup = cache.prepare([s_[:-1] for s_ in dec_full])
    _, k, v = content.batch_rows(seed, [s_[:-1] for s_ in dec_full], setup.host["prefix_lens"], hq, hkv, d,
                                 torch.bfloat16, "cuda", 1.0, with_q=False)
    cache.store(setup, k, v)
    cache.commit(setup)
    eb = cache.prepare(ext_seqs)
    eq, ek, ev = content.batch_rows(seed + 1, ext_seqs, eb.host["prefix_lens"], hq, hkv, d, torch.bfloat16,
                                    "cuda", 1.0)
    db = cache.prepare(dec_full)
    dq, dk, dv = content.batch_rows(seed + 2, dec_full, db.host["prefix_lens"], hq, hkv, d, torch.bfloat16,
                                    "cuda", 1.0)
    plan = cache.cascade_plan(db, hq, seg_chunk=64, tail_chunk=128, min_keys=8)
    eo, do = torch.empty_like(eq), torch.empty_like(dq)
    else_ = torch.empty(eq.shape[0], hq, dtype=torch.float32, device="cuda")
    dlse = torch.empty(dq.shape[0], hq, dtype=torch.float32, device="cuda")

    def step():
        cache.store(eb, ek, ev)
        cache.extend(eb, eq, o=eo, lse=else_)
        cache.store(db, dk, dv)
        cache.decode_cascade(db, dq, plan=plan, o=do, lse=dlse)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (eo, else_, do, dlse)]
    g = StepGraph(step)
    for rep in range(4):
        for t in (eo, else_, do, dlse):
            t.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip((eo, else_, do, dlse), ref):
            assert torch.equal(t, r), rep
    G.log("graph full step: 4 replays equal the eager step")
