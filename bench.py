"""Benchmark: RadixAttention prefix-shared KV attention on one MI355X.

One step = one pass of the device hot path over the two Llama-7B-shaped
batches (32 q / 32 kv heads, head_dim 128, bf16):

  extend  64 requests share a cached 1024-token prefix and extend 128 new
          tokens each: kv_scatter of the 8192 new tokens' K/V, then
          attn_extend (bf16 MFMA);
  decode  256 requests under a 4-ary, depth-3 radix tree with private tails
          (contexts 512..4096), one new token each: kv_scatter, then
          prefix-shared decode (attn_decode_cascade: each run of keys the
          tree shares is read once for all requests under it, merged with
          each request's private tail); plain split-KV attn_decode on the
          same batch is reported beside it.

Index tables come from the native radix tree (batch_prepare, untimed), the
prefix-shared plan from the native planner (rkv_cascade_plan, untimed, its
host time reported), and both are resident in HBM when the timed region
starts.  value = tokens per second of
the whole step (8192 + 256 tokens).  Extend TFLOP/s and decode KV GB/s are
reported against the MI355X peaks (2516.6 TFLOP/s dense bf16, 8 TB/s HBM),
per kernel from HIP events on the launch stream.  The host radix operations
are timed separately (ns per token).  The float64 oracle is timed on a
the host cores on the step's whole batches (rank 0 only).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "extend attn TFLOP/s + decode KV GB/s (frac of peak); tokens/s, 1 MI355X"
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0


def extend_flops(prefix_lens, seq_lens, hq, d):
    p = np.asarray(prefix_lens, dtype=np.float64)
    n = np.asarray(seq_lens, dtype=np.float64) - p
    return float(4.0 * d * hq * np.sum(n * p + n * (n + 1) / 2))


def decode_bytes(seq_lens, hq, hkv, d, b, unique_slots=None):
    L = np.asarray(seq_lens, dtype=np.float64)
    B = L.shape[0]
    kv_tokens = L.sum() if unique_slots is None else float(unique_slots)
    return float(kv_tokens * hkv * d * 2 * b + 4 * L.sum() + 2 * B * hq * d * b)


def scatter_bytes(T, hkv, d, b):
    return float(4 * T * hkv * d * b + 4 * T)


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    record (profiles/hbm_traffic.json), or None when the record is missing or
    was taken on kernel sources that have changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(path))["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    m = hashlib.sha256()
    for src in rec["sources"]:
        try:
            m.update(open(os.path.join(ROOT, src), "rb").read())
        except OSError:
            return None
    return float(rec["bytes_per_launch"]) if m.hexdigest() == rec["sources_sha256"] else None


class Phase:
    """A prepared batch whose tables and new-token K/V/Q sit in HBM."""

    def __init__(self, name, cfg_fn, kind_index):
        import torch
        from inputs import configs, content
        from prefix_shared_kv_host_amd.engine import RadixKVCache

        self.shape, phases = cfg_fn()
        s = self.shape
        dt = content.torch_dtype(s.dtype)
        perm = configs.free_list(s.pool, s.seed)
        self.cache = RadixKVCache(s.pool, s.hkv, s.d, dt, "cuda", perm)
        self.radix_ns = []
        for i, ph in enumerate(phases):
            t0 = time.perf_counter()
            batch = self.cache.prepare(ph.seqs)
            t1 = time.perf_counter()
            q, k, v = content.batch_rows(s.seed, ph.seqs, batch.host["prefix_lens"], s.hq, s.hkv, s.d,
                                         dt, "cuda", s.q_scale, with_q=(i == kind_index))
            self.cache.store(batch, k, v)
            if i == kind_index:
                self.batch, self.q, self.k, self.v = batch, q, k, v
                self.kind = ph.kind
                self.prepare_s = t1 - t0
                self.tokens_in_batch = int(batch.host["seq_lens"].sum())
                break
            t2 = time.perf_counter()
            self.cache.commit(batch)
            self.radix_ns.append((t1 - t0 + time.perf_counter() - t2) * 1e9 / max(1, sum(map(len, ph.seqs))))
        torch.cuda.synchronize()
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[0], s.hq, dtype=torch.float32, device="cuda")
        if self.kind == "decode":
            B, hq, _ = self.q.shape
            self.cache.workspace(B, hq, self.batch.max_len)
        self.name = name

        self.plan = None

    def use_cascade(self, **plan_args):
        """Decode through the prefix-shared plan (host planning timed here,
        outside the GPU step, like the tables themselves)."""
        import torch
        B, hq, _ = self.q.shape
        t0 = time.perf_counter()
        self.plan = self.cache.cascade_plan(self.batch, hq, **plan_args)
        torch.cuda.synchronize()
        self.plan_ms = (time.perf_counter() - t0) * 1e3
        self.plan_args = plan_args

    def plan_bytes(self):
        """Bytes the prefix-shared plan reads: K and V rows of every job's
        keys and every private tail key, their slot indices, q and o."""
        s, tb, pl = self.shape, self.batch.host, self.plan
        j = pl.jobs.astype(np.int64)
        shared_keys = int((j[:, 1] - j[:, 0]).sum()) if pl.n_jobs else 0
        tail_keys = int((tb["seq_lens"].astype(np.int64) - pl.tail_begin).sum())
        keys = shared_keys + tail_keys
        B = len(tb["seq_lens"])
        return float(keys * s.hkv * s.d * 2 * 2 + 4 * keys + 2 * B * s.hq * s.d * 2)

    def scatter(self):
        self.cache.store(self.batch, self.k, self.v)

    def attend(self):
        if self.kind == "extend":
            self.cache.extend(self.batch, self.q, self.o, self.lse)
        elif self.plan is not None:
            self.cache.decode_cascade(self.batch, self.q, plan=self.plan, o=self.o, lse=self.lse)
        else:
            self.cache.decode(self.batch, self.q, self.o, self.lse)

    def attend_plain(self):
        self.cache.decode(self.batch, self.q, self.o, self.lse)


def gqa_halves(steps, warmup, cfg=None):
    """Llama-70B-shaped GQA (c4: 64 q / 8 kv heads, D=128, bf16, a shared
    2048-token prefix): the extend half (64 requests x 256 new tokens) and the
    decode half (64 requests x 1 token), each kv_scatter + attention;
    reported separately and summed.  An attention's `us`: calls back to back
    from a HIP graph of 10 calls, wall clock (graph_b2b_us); `us_events`:
    calls issued back to back with HIP events between them; `us_synced`:
    one call at a time, synchronized after each (adds the launch latency).
    cfg: another config with c4's phases (its heads may differ)."""
    import torch
    from inputs import configs
    cfg = configs.c4 if cfg is None else cfg
    stream = torch.cuda.current_stream()
    out = {}
    for name, idx in (("extend", 2), ("decode", 3)):
        ph = Phase("c4-" + name, cfg, idx)
        for _ in range(warmup):
            ph.scatter()
            ph.attend()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        sc, at = [], []
        for _ in range(steps):
            ev[0].record(stream); ph.scatter(); ev[1].record(stream); ph.attend(); ev[2].record(stream)
            torch.cuda.synchronize()
            sc.append(ev[0].elapsed_time(ev[1])); at.append(ev[1].elapsed_time(ev[2]))
        tb, s_ = ph.batch.host, ph.shape
        sus, us_ev = back_to_back_us([ph.scatter, ph.attend], steps)
        us = graph_b2b_us(ph.attend, max(2, steps // 5))
        synced = dict(us_events=us_ev, us_synced=float(np.mean(at)) * 1e3,
                      scatter_us_synced=float(np.mean(sc)) * 1e3)
        T = int(tb["qo_indptr"][-1])
        if name == "extend":
            F = extend_flops(tb["prefix_lens"], tb["seq_lens"], s_.hq, s_.d)
            out[name] = dict(kernel="attn_extend", us=us, scatter_us=sus, flop=F, tflops=F / (us * 1e-6) / 1e12,
                             frac_of_peak=F / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
                             tokens_per_s=T / ((us + sus) * 1e-6), **synced)
        else:
            Bl = decode_bytes(tb["seq_lens"], s_.hq, s_.hkv, s_.d, 2)
            uniq = len(np.unique(np.concatenate([tb["req_to_token"][r][: tb["seq_lens"][r]]
                                                 for r in range(len(tb["seq_lens"]))])))
            Bu = decode_bytes(tb["seq_lens"], s_.hq, s_.hkv, s_.d, 2, unique_slots=uniq)
            out[name] = dict(kernel="attn_decode", us=us, scatter_us=sus, bytes_logical=Bl, bytes_unique=Bu,
                             logical_equiv_gbs=Bl / (us * 1e-6) / 1e9, gbs_unique=Bu / (us * 1e-6) / 1e9,
                             frac_of_peak_unique=Bu / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                             tokens_per_s=T / ((us + sus) * 1e-6), **synced)
            # the same batch through the prefix-shared path (64 requests under
            # one 2048-token prefix)
            ph.use_cascade()
            for _ in range(warmup):
                ph.attend()
            cas = []
            for _ in range(steps):
                ev[1].record(stream); ph.attend(); ev[2].record(stream)
                torch.cuda.synchronize()
                cas.append(ev[1].elapsed_time(ev[2]))
            (cus_ev,) = back_to_back_us([ph.attend], steps)
            cus = graph_b2b_us(ph.attend, max(2, steps // 5))
            out[name]["cascade"] = dict(kernel="attn_decode_cascade", us=cus, us_events=cus_ev,
                                        us_synced=float(np.mean(cas)) * 1e3,
                                        bytes_plan=ph.plan_bytes(),
                                        gbs_plan=ph.plan_bytes() / (cus * 1e-6) / 1e9,
                                        frac_of_peak=ph.plan_bytes() / (cus * 1e-6) / 1e9 / PEAK_HBM_GBS,
                                        jobs=ph.plan.n_jobs, seg_chunk=ph.plan.seg_chunk,
                                        tail_chunk=ph.plan.tail_chunk, host_plan_ms=ph.plan_ms)
            # both decode paths captured into a HIP graph and replayed: the
            # same kernels without the host side of each call
            out[name]["graph_us"] = graph_replay_us(ph.attend_plain, steps, warmup)
            out[name]["cascade"]["graph_us"] = graph_replay_us(ph.attend, steps, warmup)
        del ph
        torch.cuda.empty_cache()
    tot = out["extend"]["us"] + out["extend"]["scatter_us"] + out["decode"]["us"] + out["decode"]["scatter_us"]
    out["summed"] = dict(us=tot, tokens=64 * 256 + 64, tokens_per_s=(64 * 256 + 64) / (tot * 1e-6))
    out["workload"] = ("llama70b-gqa: 128 requests share a 2048-token prefix; 64 extend 256 tokens (contexts "
                       "2304-8192), 64 decode 1 token (contexts 2049-8192); 64/8 heads, D=128, bf16, 2^20 slots")
    return out


def back_to_back_us(fns, steps):
    """Mean device time of each of `fns` when the sequence is issued `steps`
    times back to back with no synchronization in between (as the timed step
    loop issues its calls): HIP events on the launch stream between the
    calls, one synchronization at the end.  A call whose host side is slower
    than the kernels before it shows that host time too."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps * len(fns) + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    i = 0
    for _ in range(steps):
        for f in fns:
            f()
            i += 1
            ev[i].record(stream)
    torch.cuda.synchronize()
    t = np.array([ev[j].elapsed_time(ev[j + 1]) for j in range(i)]).reshape(steps, len(fns))
    return [float(x) * 1e3 for x in t.mean(axis=0)]


def graph_b2b_us(fn, reps, inner=10):
    """Device time per call of `fn`: `inner` calls captured into one HIP
    graph (engine.StepGraph) and the graph replayed `reps` times back to
    back, wall clock over the replays.  No events sit between the calls, and
    the host side of each call is out of the loop, so short kernels are
    timed as the device runs them back to back."""
    import torch
    from prefix_shared_kv_host_amd.engine import StepGraph
    g = StepGraph(lambda: [fn() for _ in range(inner)])
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / (reps * inner)
    del g
    return us


def graph_replay_us(fn, steps, warmup):
    """Mean time of one replay of `fn` captured into a HIP graph
    (engine.StepGraph), timed like the eager calls: HIP events around each
    replay on the launch stream, synchronized after each."""
    import torch
    from prefix_shared_kv_host_amd.engine import StepGraph
    g = StepGraph(fn)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t = []
    for _ in range(steps):
        ev[0].record(stream); g.replay(); ev[1].record(stream)
        torch.cuda.synchronize()
        t.append(ev[0].elapsed_time(ev[1]))
    return float(np.mean(t)) * 1e3


def step_graph(step, tokens, steps, warmup):
    """The whole step (both scatters, extend, prefix-shared decode) captured
    into one HIP graph and replayed, timed like the eager step that `value`
    reports: wall clock over `steps` replays, synchronized after each, plus
    HIP events on the launch stream."""
    import torch
    from prefix_shared_kv_host_amd.engine import StepGraph
    g = StepGraph(step)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t = []
    t0 = time.perf_counter()
    for _ in range(steps):
        ev[0].record(stream); g.replay(); ev[1].record(stream)
        torch.cuda.synchronize()
        t.append(ev[0].elapsed_time(ev[1]))
    ms = (time.perf_counter() - t0) * 1e3 / steps
    return dict(ms_per_step=ms, ms_events=float(np.mean(t)), tokens_per_s=tokens / (ms * 1e-3),
                note="the same step replayed from a HIP graph (engine.StepGraph); `value` is the eager step")


def tp8_share(steps, warmup):
    """One GPU's share of 8-way tensor parallelism over heads, at real shape:
    c4 with 8 q / 1 kv heads per GPU (both halves), c5 with 4 q / 1 kv heads
    (the chat replay).  The all-reduce after the attention projection is
    outside this path and not modelled."""
    from inputs import configs
    c4s = gqa_halves(steps, warmup, configs.c4tp8)
    c4s["workload"] = ("llama70b-gqa, one GPU of 8-way tensor parallelism: 8 q / 1 kv heads, the c4 requests "
                       "(64 extend 256 tokens, 64 decode 1 token, 2048-token shared prefix)")
    s, phases = configs.c5tp8()
    replay(s, phases[:4])
    c5s = replay(s, phases)
    c5s["workload"] = "c5 chat replay, one GPU of 8-way tensor parallelism: 4 q / 1 kv heads, 2^21 slots"
    return {"c4tp8": c4s, "c5tp8": c5s}


def chat_pipeline(name):
    """Multi-turn chat replay (c5: 512 sessions, 89 batches; c5e: the same
    trace on a 2^19-slot pool, where LRU eviction and recompute bind), timed
    end to end: host radix prepare/commit, table upload, kv_scatter and
    attn_extend for every batch.  The new tokens' q/k/v stand for the model's
    projections and are generated before the timed region."""
    import torch
    from inputs import configs, content
    from prefix_shared_kv_host_amd import rkv
    from prefix_shared_kv_host_amd.engine import RadixKVCache

    s, phases = configs.build(name)
    out = replay(s, phases)
    out["workload"] = (f"{name}: Mixtral-8x7B-shaped multi-turn chat, 512 sessions, 32/8 heads, D=128, "
                       f"2^{int(np.log2(s.pool))} slots")
    return out


def decode_loop_host(steps=16):
    """Per-step cost outside the kernels of a decode loop over the radix-tree
    decode batch (256 requests of 512-4096 tokens): matching every history
    again each step (prepare + commit of the grown batch, the whole token
    table uploaded) against continuing the prepared batch (append: one slot
    per request on the host, B slot ids uploaded, the device table grown in
    place by rkv_table_append; one commit at the end, counted).  No attention
    runs: this is the host tree and table traffic a step adds."""
    import torch
    from inputs import configs
    from prefix_shared_kv_host_amd import rkv
    from prefix_shared_kv_host_amd.engine import RadixKVCache

    s, phases = configs.build("c3")
    dec = phases[-1]
    B = len(dec.seqs)
    ld = max(len(x) for x in dec.seqs) + steps + 1
    grown = [[list(x) for x in dec.seqs]]
    for k in range(steps):
        grown.append([x + [1_000_000 + 1000 * k + i] for i, x in enumerate(grown[-1])])
    toks = [rkv.TokenBatch(g) for g in grown]           # token arrays, as a server holds them
    out = dict(requests=B, steps=steps, ld=ld)
    for mode in ("rematch", "append"):
        # the tables do not depend on the head shape: one 64-wide kv head keeps the pool small
        cache = RadixKVCache(s.pool, 1, 64, torch.bfloat16, "cuda", configs.free_list(s.pool, s.seed),
                             poison=False)
        for ph in phases[:-1]:
            cache.commit(cache.prepare(ph.seqs))
        b = cache.prepare(toks[0], ld)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if mode == "rematch":
            cache.commit(b)
            for k in range(1, steps + 1):
                b = cache.prepare(toks[k], ld)
                cache.commit(b)
        else:
            for k in range(1, steps + 1):
                cache.append(b)
            cache.commit(b, toks[steps])
        torch.cuda.synchronize()
        out[f"{mode}_ms_per_step"] = (time.perf_counter() - t0) * 1e3 / steps
        del cache, b
        torch.cuda.empty_cache()
    out["rematch_upload_bytes_per_step"] = 4 * (B * ld + 3 * B + 1 + B)
    out["append_upload_bytes_per_step"] = 4 * B
    return out


def decode_loop(steps=33):
    """End-to-end decode loop over the radix-tree decode batch (256 requests
    of 512-4096 tokens, 32 heads, D=128, bf16): each step grows the batch by
    append, plans prefix-shared decode on the host, stores the step's new K/V
    and runs the prefix-shared decode; nothing waits for the GPU inside the
    loop, so the host work of step k+1 overlaps the kernels of step k.  The
    steps' q/k/v stand for the model's projections and are generated before
    timing; the first step (the prepare's own token) is not timed."""
    import torch
    from inputs import configs, content
    from prefix_shared_kv_host_amd.engine import RadixKVCache

    s, phases = configs.build("c3")
    dt = content.torch_dtype(s.dtype)
    cache = RadixKVCache(s.pool, s.hkv, s.d, dt, "cuda", configs.free_list(s.pool, s.seed), poison=False)
    for ph in phases[:-1]:
        b = cache.prepare(ph.seqs)
        _, k, v = content.batch_rows(s.seed, ph.seqs, b.host["prefix_lens"], s.hq, s.hkv, s.d, dt, "cuda",
                                     with_q=False)
        cache.store(b, k, v)
        cache.commit(b)
        del k, v
    dec = phases[-1]
    B = len(dec.seqs)
    b = cache.prepare(dec.seqs, max(len(x) for x in dec.seqs) + steps + 1)
    g = torch.Generator(device="cuda").manual_seed(s.seed)
    qkv = [tuple(torch.randn(B, h, s.d, device="cuda", generator=g).to(dt) for h in (s.hq, s.hkv, s.hkv))
           for _ in range(steps)]
    o = torch.empty(B, s.hq, s.d, dtype=dt, device="cuda")
    cache.store(b, qkv[0][1], qkv[0][2])
    cache.decode_cascade(b, qkv[0][0], plan=cache.cascade_plan(b, s.hq), o=o)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = []
    t0 = time.perf_counter()
    for k in range(1, steps):
        cache.append(b)
        plan = cache.cascade_plan(b, s.hq)
        q, kn, vn = qkv[k]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        cache.store(b, kn, vn)
        cache.decode_cascade(b, q, plan=plan, o=o)
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n = steps - 1
    dev_ms = sum(a.elapsed_time(c) for a, c in ev) / n
    out = dict(requests=B, steps=n, ms_per_step=wall * 1e3 / n, device_ms_per_step=dev_ms,
               tokens_per_s=B * n / wall, final_max_len=int(b.max_len))
    del cache, b, qkv, o
    torch.cuda.empty_cache()
    return out


def replay(s, phases):
    """Times batches end to end: host radix prepare/commit, table upload,
    kv_scatter and attn_extend for every batch."""
    import torch
    from inputs import configs, content
    from prefix_shared_kv_host_amd import rkv
    from prefix_shared_kv_host_amd.engine import RadixKVCache

    dt = content.torch_dtype(s.dtype)
    perm = configs.free_list(s.pool, s.seed)
    # dry run on a host tree: the timed replay sees the same prefix lengths
    tree = rkv.Tree(s.pool, perm)
    pre, lens = [], []
    for ph in phases:
        code, tb = tree.batch_prepare(ph.seqs)
        assert code == rkv.OK
        pre.append(tb["prefix_lens"].copy())
        lens.append(tb["seq_lens"].copy())
        tree.batch_commit(ph.seqs, tb["req_to_token"], tb["nodes"])
    del tree
    qkv = [content.batch_rows(s.seed, ph.seqs, pre[i], s.hq, s.hkv, s.d, dt, "cuda", s.q_scale, with_q=True)
           for i, ph in enumerate(phases)]
    # token ids as int32 arrays, as a server holds them (converted here, untimed)
    toks = [rkv.TokenBatch(ph.seqs) for ph in phases]
    flop = sum(extend_flops(pre[i], lens[i], s.hq, s.d) for i in range(len(phases)))
    new_tokens = int(sum(int(np.sum(lens[i] - pre[i])) for i in range(len(phases))))
    cache = RadixKVCache(s.pool, s.hkv, s.d, dt, "cuda", perm, poison=False)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = []
    t0 = time.perf_counter()
    for i, ph in enumerate(phases):
        b = cache.prepare(toks[i])
        q, k, v = qkv[i]
        cache.store(b, k, v)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        cache.extend(b, q)
        e1.record(stream)
        ev.append((e0, e1))
        cache.commit(b)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_s = sum(a.elapsed_time(b) for a, b in ev) * 1e-3
    st = cache.tree.stats()
    out = dict(batches=len(phases), new_tokens=new_tokens, seconds=wall,
               pipeline_tokens_per_s=new_tokens / wall, extend_flop=flop, extend_kernel_s=kern_s,
               extend_tflops=flop / kern_s / 1e12, evicted_tokens=int(st[7]),
               prompt_tokens=int(st[6]), hit_rate=float(st[5]) / max(1, int(st[6])))
    del qkv, cache
    torch.cuda.empty_cache()
    return out


def multimodal_replay():
    """LLaVA-v1.5-7B-shaped visual QA (24 images x 5 questions, 576 image
    positions, 35-token system prompt): images enter the tree as their
    content-hash keys, so later questions about an image reuse its KV;
    against the same trace with a fresh key sequence per request (no image
    reuse).  End to end per trace, as the chat replay."""
    from inputs import configs
    from prefix_shared_kv_host_amd import mm
    s, trace, n_img = configs.mm()
    sys_tokens, blobs, batches = trace
    hashed = [configs.Phase("extend", b) for b in mm.trace_batches(trace, n_img)]
    fresh_blobs, fresh = [], []
    for k, b in enumerate(batches):
        seqs = []
        for j, (img, q) in enumerate(b):
            seqs.append(mm.request_tokens(sys_tokens, blobs[img] + bytes(f"/{k}/{j}", "ascii"), n_img, q))
        fresh.append(configs.Phase("extend", seqs))
    # each trace twice, the second timed: the first replay also loads the
    # kernels and grows the pinned host buffers the table uploads reuse
    replay(s, hashed), replay(s, fresh)
    a, b = replay(s, hashed), replay(s, fresh)
    return dict(workload="LLaVA-v1.5-7B-shaped visual QA: 24 images x 5 questions, 576 image positions, "
                         "35-token system prompt, batches of <= 16 requests; 32/32 heads, D=128, bf16",
                hashed_keys=a, no_image_reuse=b, seconds_ratio=b["seconds"] / a["seconds"],
                prompt_tokens_per_s_hashed=a["prompt_tokens"] / a["seconds"],
                prompt_tokens_per_s_no_reuse=b["prompt_tokens"] / b["seconds"])


def sampling_penalties(steps=64, warmup=8):
    """Batched sampling penalties on the decode loop: 256 running requests,
    vocabulary 32000 (Llama-7B), 256-token prompts, with the sampling page's
    "all penalties" benchmark settings (frequency 1.1, presence 1.1,
    repetition 0.1, min_new_tokens 5, EOS id 2).  Each step applies the
    penalties to the fp32 logits [256, 32000] in place and records one
    seeded output token per request; HIP events on the launch stream."""
    import torch
    from prefix_shared_kv_host_amd import rkv
    B, V, P = 256, 32000, 256
    rng = np.random.default_rng(61)
    st = rkv.PenaltyState(B, V, P + warmup + steps + 8)
    rows = torch.arange(B, dtype=torch.int32, device="cuda")
    prompts = (rng.zipf(1.2, (B, P)) % V).astype(np.int32)
    indptr = torch.arange(0, B * P + 1, P, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    pids = torch.from_numpy(prompts.reshape(-1)).cuda()
    st.admit(rows, indptr, pids)                # first launch loads the code object
    torch.cuda.synchronize()
    ev[0].record(stream)
    st.admit(rows, indptr, pids)
    ev[1].record(stream)
    torch.cuda.synchronize()
    admit_us = ev[0].elapsed_time(ev[1]) * 1e3
    # output tokens: half repeat a prompt or earlier token, half fresh
    toks = np.where(rng.random((warmup + steps, B)) < 0.5, prompts[np.arange(B), rng.integers(0, P, (warmup + steps, B))],
                    rng.integers(0, V, (warmup + steps, B))).astype(np.int32)
    toks = torch.from_numpy(toks).cuda()
    f32 = lambda v: torch.full((B,), v, dtype=torch.float32, device="cuda")
    freq, pres, rep = f32(1.1), f32(1.1), f32(0.1)
    min_new = torch.full((B,), 5, dtype=torch.int32, device="cuda")
    stop_indptr = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    stop_ids = torch.full((B,), 2, dtype=torch.int32, device="cuda")
    logits = torch.randn(B, V, device="cuda")
    # decode step = one launch: record the previous token, then penalize
    ap, sep = [], []
    for i in range(warmup + steps):
        ev[0].record(stream)
        st.apply(logits, rows, freq, pres, rep, min_new, stop_indptr, stop_ids, new_tokens=toks[i])
        ev[1].record(stream)
        torch.cuda.synchronize()
        if i >= warmup:
            ap.append(ev[0].elapsed_time(ev[1]))
    seen = int(st.seen_len.sum().item())
    # the same step as two launches (accumulate, then apply), for comparison
    for i in range(warmup + steps):
        ev[0].record(stream)
        st.accumulate(rows, toks[i])
        st.apply(logits, rows, freq, pres, rep, min_new, stop_indptr, stop_ids)
        ev[1].record(stream)
        torch.cuda.synchronize()
        if i >= warmup:
            sep.append(ev[0].elapsed_time(ev[1]))
    step_us, sep_us = float(np.mean(ap)) * 1e3, float(np.mean(sep)) * 1e3
    moved = float(seen * 16 + B * 4 * 10)       # per listed token: list, count, logit read and write
    dense = float(B * V * 12)                   # a full-vocabulary sweep: logits read + write, counts read
    return dict(workload="256 running requests x vocab 32000, 256-token prompts, freq 1.1 / presence 1.1 / "
                         "repetition 0.1 / min_new_tokens 5, fp32 logits",
                step_us=step_us, step_us_two_launches=sep_us, admit_us=admit_us,
                listed_tokens_at_end=seen, step_bytes_at_end=moved,
                dense_sweep_bytes=dense, dense_sweep_us_at_hbm_peak=dense / (PEAK_HBM_GBS * 1e3),
                requests_per_s=B / (step_us * 1e-6))


def queue_orders():
    """Cache hit rate of the multi-turn chat trace under a serving queue (a
    session's next turn is runnable once its previous turn ran; <= 64 turns a
    step), first come first served vs cache-aware (rkv_schedule: longest
    reusable prefix first), on the native tree; host only."""
    from inputs import configs
    from prefix_shared_kv_host_amd import rkv, serving
    out = []
    for name in ("c5", "c5e"):
        s, _ = configs.build(name)
        batches, tags = configs.chat_trace(s.seed)
        turns = {st: seq for b, tg in zip(batches, tags) for seq, st in zip(b, tg)}
        arrival = [st for tg in tags for st in tg]
        row = dict(workload=f"{name}: 512 sessions, 2241 turns, pool 2^{int(np.log2(s.pool))} slots")
        for policy in ("fcfs", "cache"):
            tree = rkv.Tree(s.pool, configs.free_list(s.pool, s.seed))
            t0 = time.perf_counter()
            r = serving.run_queue(tree, turns, arrival, policy)
            row[policy] = dict(hit_rate=r["hit_rate"], reused_tokens=r["reused_tokens"], steps=r["steps"],
                               evicted_tokens=int(tree.stats()[7]), host_s=time.perf_counter() - t0)
        row["prompt_tokens"] = r["prompt_tokens"]
        out.append(row)
    return out


def time_host_radix(phase_obj, reps=3):
    """ns per token of batch_prepare + batch_commit on a fresh native tree
    replaying the same workload (host only; token ids as int32 arrays)."""
    from inputs import configs
    from prefix_shared_kv_host_amd import rkv
    s, phases = phase_obj.cfg
    toks = [rkv.TokenBatch(ph.seqs) for ph in phases]
    best = None
    for _ in range(reps):
        t = rkv.Tree(s.pool, configs.free_list(s.pool, s.seed))
        tot_tok, tot_s = 0, 0.0
        for tk in toks:
            t0 = time.perf_counter()
            code, tb = t.batch_prepare(tk)
            t.batch_commit(tk, tb["req_to_token"], tb["nodes"])
            tot_s += time.perf_counter() - t0
            tot_tok += int(tk.indptr[-1])
        v = tot_s * 1e9 / tot_tok
        best = v if best is None else min(best, v)
    return best


def host_info():
    """The host the oracle runs on: logical CPUs, CPU model, BLAS threads."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas = None
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return dict(cpu_count=os.cpu_count(), cpu_model=model, blas_threads=blas)


def oracle_attention_time(cfg_fn, kind_index, keep=None):
    """Seconds the float64 oracle takes for one batch's attention.  The
    oracle tree, tables and pool are built the way a server fills them
    (every earlier phase prepared, its new tokens' K/V scattered, committed),
    untimed; content rows come from the shared input generator on the GPU.
    keep: the requests of the batch to compute (None = all).  Returns
    (seconds, host tables, shape, requests)."""
    import torch
    from inputs import configs, content
    from oracle import attention as oatt
    from oracle.pool import OraclePool, scatter
    from oracle.radix import OracleTree

    s, phases = cfg_fn()
    tree = OracleTree(s.pool, configs.free_list(s.pool, s.seed))
    pool = OraclePool(s.pool, s.hkv, s.d)
    dt = content.torch_dtype(s.dtype)
    for i, ph in enumerate(phases):
        st, tb = tree.batch_prepare(ph.seqs)
        q, k, v = content.batch_rows(s.seed, ph.seqs, tb["prefix_lens"], s.hq, s.hkv, s.d, dt, "cuda",
                                     s.q_scale, with_q=(i == kind_index))
        scatter(pool, tb["new_slots"], k.cpu(), v.cpu())
        del k, v
        if i == kind_index:
            qn = q.float().cpu().numpy()
            del q
            torch.cuda.empty_cache()
            rq = list(range(len(ph.seqs))) if keep is None else list(keep)
            t0 = time.perf_counter()
            if ph.kind == "extend":
                oatt.extend(qn, pool, tb["req_to_token"], tb["qo_indptr"], tb["prefix_lens"], s.hq, s.hkv,
                            requests=rq)
            else:
                oatt.decode(qn, pool, tb["req_to_token"], tb["seq_lens"], s.hq, s.hkv, requests=rq)
            return time.perf_counter() - t0, tb, s, rq
        tree.batch_commit(ph.seqs, tb["req_to_token"], tb["nodes"])
    raise RuntimeError("no such phase")


def cpu_baseline():
    """The float64 oracle timed on the host cores in the same run: the
    step's whole extend batch (64 requests) and whole decode batch (256
    requests), plus 8 of the 64 extend requests of the 64/8-head batch as a
    sample of that kernel's rate.  value = the step's tokens / the oracle's
    seconds for the step."""
    from inputs import configs
    info = host_info()
    te, tbe, se, _ = oracle_attention_time(configs.c2, 1)
    Fe = extend_flops(tbe["prefix_lens"], tbe["seq_lens"], se.hq, se.d)
    td, tbd, sd, _ = oracle_attention_time(configs.c3, 4)
    Bd = decode_bytes(tbd["seq_lens"], sd.hq, sd.hkv, sd.d, 2)
    keep4 = list(range(0, 64, 8))
    t4, tb4, s4, rq4 = oracle_attention_time(configs.c4, 2, keep4)
    F4 = extend_flops([tb4["prefix_lens"][r] for r in rq4], [tb4["seq_lens"][r] for r in rq4], s4.hq, s4.d)
    Te, Td = int(tbe["qo_indptr"][-1]), int(tbd["qo_indptr"][-1])
    return dict(value=(Te + Td) / (te + td), unit="tokens/s", cores=info["blas_threads"] or info["cpu_count"],
                kind="oracle",
                sample="the whole step: float64 oracle attention over all 64 extend requests (32 heads, 1152 "
                       "keys each) and all 256 decode requests; tree, tables and pool built untimed",
                seconds=te + td, cpu_count=info["cpu_count"], cpu_model=info["cpu_model"],
                blas_threads=info["blas_threads"],
                cores_note="cores = the BLAS threads the oracle's matrix products use; its gathers and "
                           "exponentials run on one thread",
                extend=dict(seconds=te, flop=Fe, gflops=Fe / te / 1e9, tokens_per_s=Te / te),
                decode=dict(seconds=td, bytes_logical=Bd, gbs=Bd / td / 1e9, tokens_per_s=Td / td),
                llama70b_extend_sample=dict(requests=len(rq4), seconds=t4, flop=F4, gflops=F4 / t4 / 1e9,
                                            note="8 of the 64 extend requests of the 64/8-head batch"))


LEGS = {
    # leg: (config, phase index, prefix-shared decode)
    "extend": ("c2", 1, False),
    "decode": ("c3", 4, True),
    "gqa-extend": ("c4", 2, False),
    "gqa-decode": ("c4", 3, False),
    "gqa-decode-cascade": ("c4", 3, True),
}


def one_leg(leg, steps, warmup):
    """One kernel's workload, timed alone with HIP events on the launch
    stream: `steps` launches after `warmup`, each synchronized.  extend and
    decode are the step's two halves; the gqa-* legs are the 64/8-head
    batch's (plain or prefix-shared decode), for counter passes."""
    import torch
    from inputs import configs
    cfg, idx, cascade = LEGS[leg]
    ph = Phase(leg, getattr(configs, cfg), idx)
    if cascade:
        ph.use_cascade()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for _ in range(warmup):
        ph.scatter()
        ph.attend()
    torch.cuda.synchronize()
    sc, at = [], []
    for _ in range(steps):
        ev[0].record(stream); ph.scatter(); ev[1].record(stream); ph.attend(); ev[2].record(stream)
        torch.cuda.synchronize()
        sc.append(ev[0].elapsed_time(ev[1])); at.append(ev[1].elapsed_time(ev[2]))
    tb, s_ = ph.batch.host, ph.shape
    us = float(np.mean(at)) * 1e3
    out = dict(leg=leg, steps=steps, warmup=warmup, attend_us=us, scatter_us=float(np.mean(sc)) * 1e3)
    if ph.kind == "extend":
        F = extend_flops(tb["prefix_lens"], tb["seq_lens"], s_.hq, s_.d)
        out.update(flop=F, tflops=F / (us * 1e-6) / 1e12, frac_of_peak=F / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS)
    elif cascade:
        Bp = ph.plan_bytes()
        out.update(bytes_plan=Bp, gbs_plan=Bp / (us * 1e-6) / 1e9, frac_of_peak=Bp / (us * 1e-6) / 1e9 / PEAK_HBM_GBS)
    else:
        uniq = len(np.unique(np.concatenate([tb["req_to_token"][r][: tb["seq_lens"][r]]
                                             for r in range(len(tb["seq_lens"]))])))
        Bu = decode_bytes(tb["seq_lens"], s_.hq, s_.hkv, s_.d, 2, unique_slots=uniq)
        out.update(bytes_unique=Bu, gbs_unique=Bu / (us * 1e-6) / 1e9,
                   frac_of_peak_unique=Bu / (us * 1e-6) / 1e9 / PEAK_HBM_GBS)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-reps", type=int, default=10)
    ap.add_argument("--leg", choices=sorted(LEGS), default=None,
                    help="time one kernel's workload alone (for counter runs under rocprofv3): "
                         "extend = scatter + attn_extend of the 64 x (1024 + 128) batch, decode = scatter + "
                         "prefix-shared decode of the 256-request tree batch; gqa-extend, gqa-decode, "
                         "gqa-decode-cascade = the 64/8-head batch's extend, plain decode and prefix-shared "
                         "decode; prints one JSON line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this path has no sharding or collectives; "
              "--gpus above 1 is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    from inputs import configs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.leg:
        print(json.dumps(one_leg(args.leg, args.steps, args.warmup)))
        return
    t_setup = time.perf_counter()
    ext = Phase("extend", configs.c2, 1)
    ext.cfg = configs.c2()
    dec = Phase("decode", configs.c3, 4)
    dec.cfg = configs.c3()
    dec.use_cascade()
    print(f"# setup {time.perf_counter() - t_setup:.1f}s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]

    def step(evl=None, dec_ev=None):
        if evl:
            evl[0].record(stream)
        ext.scatter()
        if evl:
            evl[1].record(stream)
        ext.attend()
        if evl:
            evl[2].record(stream)
        dec.scatter()
        if evl:
            evl[3].record(stream)
        if dec_ev:
            dec_ev[0].record(stream)
        dec.attend()
        if evl:
            evl[4].record(stream)
        if dec_ev:
            dec_ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps issued back to back (as a serving loop
    # issues them), synchronized on both sides.  The chip needs more than a
    # few steps to settle, hence the default warm-up of 100 steps.  Only the
    # dominant kernel, the decode, is bracketed by HIP events here: events
    # between every pair of kernels lengthen the step by 2-4 % (measured), so
    # the other kernels' times come from separate passes below.
    dev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(dec_ev=dev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1000 / args.steps
    dec_ms_live = float(np.mean([e0.elapsed_time(e1) for e0, e1 in dev]))
    # the same steps with a synchronization after each: every step then also
    # waits for the host to launch its first kernel
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
        torch.cuda.synchronize()
    ms_per_step_synced = (time.perf_counter() - t0) * 1000 / args.steps
    # per-kernel times: the same steps with HIP events between the calls
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[i])
        torch.cuda.synchronize()
    per = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(4)] for i in range(args.steps)])
    ms_kernels = per.sum(axis=1).mean()
    kern_ms = per.mean(axis=0)   # scatter_e, extend, scatter_d, decode
    # the extend alone, launched back to back: its time depends on what ran
    # before it in the step (after the HBM-heavy decode it runs longer)
    (ext_alone_us,) = back_to_back_us([ext.attend], args.steps)

    # cold: flush L2 / MALL with a 512 MiB write before each launch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = np.zeros((args.cold_reps, 2))
    for i in range(args.cold_reps):
        flush.fill_(i & 0xFF)
        ev[0].record(stream); ext.attend(); ev[1].record(stream)
        flush.fill_((i + 1) & 0xFF)
        ev[2].record(stream); dec.attend(); ev[3].record(stream)
        torch.cuda.synchronize()
        cold[i] = [ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])]
    # the same decode batch through plain split-KV decode (every request
    # reads its whole context), for comparison with the prefix-shared path
    pl_ms = []
    for i in range(args.warmup + args.steps):
        ev[0].record(stream); dec.attend_plain(); ev[1].record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            pl_ms.append(ev[0].elapsed_time(ev[1]))
    pl_cold = []
    for i in range(args.cold_reps):
        flush.fill_(i & 0xFF)
        ev[0].record(stream); dec.attend_plain(); ev[1].record(stream)
        torch.cuda.synchronize()
        pl_cold.append(ev[0].elapsed_time(ev[1]))
    # no-share control: the same context lengths with every context private,
    # so no KV row is read by two requests (honest HBM fraction for decode)
    ns = Phase("decode-noshare", configs.c3ns, 1)
    ns_ms = []
    for i in range(args.warmup + args.steps):
        ev[0].record(stream); ns.attend(); ev[1].record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            ns_ms.append(ev[0].elapsed_time(ev[1]))
    ns_cold = []
    for i in range(args.cold_reps):
        flush.fill_(i & 0xFF)
        ev[0].record(stream); ns.attend(); ev[1].record(stream)
        torch.cuda.synchronize()
        ns_cold.append(ev[0].elapsed_time(ev[1]))
    # the same no-share batch through the prefix-shared entry: its plan has
    # no shared run, so every key is a private tail read with streaming loads
    ns.use_cascade()
    nc_ms = []
    for i in range(args.warmup + args.steps):
        ev[0].record(stream); ns.attend(); ev[1].record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            nc_ms.append(ev[0].elapsed_time(ev[1]))
    del flush
    tb_n = ns.batch.host
    Bn = decode_bytes(tb_n["seq_lens"], ns.shape.hq, ns.shape.hkv, ns.shape.d, 2)
    ns_us = float(np.mean(ns_ms)) * 1e3
    nc_us = float(np.mean(nc_ms)) * 1e3
    noshare_obj = dict(kernel="attn_decode", us=ns_us, us_cold=float(np.mean(ns_cold)) * 1e3, bytes=Bn,
                       gbs=Bn / (ns_us * 1e-6) / 1e9, frac_of_peak=Bn / (ns_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                       cascade_entry=dict(kernel="attn_decode_cascade (no shared run: streaming tails)", us=nc_us,
                                          jobs=ns.plan.n_jobs, gbs=Bn / (nc_us * 1e-6) / 1e9,
                                          frac_of_peak=Bn / (nc_us * 1e-6) / 1e9 / PEAK_HBM_GBS))
    del ns

    s_e, s_d = ext.shape, dec.shape
    tb_e, tb_d = ext.batch.host, dec.batch.host
    F = extend_flops(tb_e["prefix_lens"], tb_e["seq_lens"], s_e.hq, s_e.d)
    uniq = len(np.unique(np.concatenate([tb_d["req_to_token"][r][: tb_d["seq_lens"][r]]
                                         for r in range(len(tb_d["seq_lens"]))])))
    Bl = decode_bytes(tb_d["seq_lens"], s_d.hq, s_d.hkv, s_d.d, 2)
    Bu = decode_bytes(tb_d["seq_lens"], s_d.hq, s_d.hkv, s_d.d, 2, unique_slots=uniq)
    T_e, T_d = int(tb_e["qo_indptr"][-1]), int(tb_d["qo_indptr"][-1])
    ext_tflops = F / (ext_alone_us * 1e-6) / 1e12
    dec_gbs = Bl / (dec_ms_live * 1e-3) / 1e9
    dec_gbs_u = Bu / (dec_ms_live * 1e-3) / 1e9
    tokens = T_e + T_d
    value = tokens / (ms_per_step * 1e-3)

    extend_obj = dict(kernel="attn_extend (bf16 MFMA)", us=ext_alone_us, us_in_step=kern_ms[1] * 1e3,
                      us_cold=cold[:, 0].mean() * 1e3,
                      flop=F, tflops=ext_tflops, frac_of_peak=ext_tflops / PEAK_BF16_TFLOPS,
                      tokens_per_s=T_e / (kern_ms[0] * 1e-3 + ext_alone_us * 1e-6), scatter_us=kern_ms[0] * 1e3,
                      scatter_gbs=scatter_bytes(T_e, s_e.hkv, s_e.d, 2) / (kern_ms[0] * 1e-3) / 1e9,
                      hit_rate=float(np.sum(tb_e["prefix_lens"]) / np.sum(tb_e["seq_lens"])))
    Bp = dec.plan_bytes()
    pl = dec.plan
    # frac_of_peak counts the bytes this kernel's plan reads (each shared run
    # once); the logical bytes (every context read whole per request) are
    # what plain decode would move, so their rate is an equivalent, not a
    # bandwidth, and no fraction of the HBM peak is formed from it
    decode_obj = dict(kernel="attn_decode_cascade (shared runs once + private tails in one launch, LSE merge)",
                      us=dec_ms_live * 1e3, us_in_step_events=kern_ms[3] * 1e3, us_cold=cold[:, 1].mean() * 1e3,
                      bytes_logical=Bl, bytes_unique=Bu,
                      bytes_plan=Bp, logical_equiv_gbs=dec_gbs, gbs_unique=dec_gbs_u,
                      gbs_plan=Bp / (dec_ms_live * 1e-3) / 1e9,
                      frac_of_peak=Bp / (dec_ms_live * 1e-3) / 1e9 / PEAK_HBM_GBS,
                      frac_of_peak_unique=dec_gbs_u / PEAK_HBM_GBS,
                      tokens_per_s=T_d / ((kern_ms[2] + dec_ms_live) * 1e-3), scatter_us=kern_ms[2] * 1e3,
                      plan=dict(jobs=pl.n_jobs, records=pl.n_records, tail_splits=pl.tail_splits,
                                max_members=pl.max_members, tail_chunk=pl.tail_chunk, seg_chunk=pl.seg_chunk,
                                host_ms=dec.plan_ms,
                                settings="the engine's rules: tail_chunk 768 keys (384 for a small grouped-head "
                                         "launch), seg_chunk = tail_chunk (256 when halved), min_keys 32"))
    pl_us = float(np.mean(pl_ms)) * 1e3
    # plain decode reads every context whole, the shared rows partly from
    # L2/MALL: its logical rate is bytes delivered to the kernel, and its HBM
    # fraction is formed on the unique bytes (each slot once)
    decode_plain_obj = dict(kernel="attn_decode (split-KV partial + LSE merge)", us=pl_us,
                            us_cold=float(np.mean(pl_cold)) * 1e3, bytes_logical=Bl, bytes_unique=Bu,
                            logical_equiv_gbs=Bl / (pl_us * 1e-6) / 1e9,
                            frac_of_peak_unique=Bu / (pl_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                            speedup_of_cascade=pl_us / (dec_ms_live * 1e3))
    roof_e = dict(kernel="attn_extend", bound="mfma", achieved=ext_tflops, peak=PEAK_BF16_TFLOPS,
                  unit="TFLOP/s", frac=ext_tflops / PEAK_BF16_TFLOPS, traffic=measured_traffic("attn_extend"))
    # achieved counts the algorithmic bytes of the prefix-shared algorithm:
    # what its plan must read (each shared run once, the private tails, the
    # slot indices, q and o), Bp.  Per request, decode attention would read
    # every context whole (Bl, "logical"); traffic is what the counters saw
    # past L2 for one launch
    gbs_plan = Bp / (dec_ms_live * 1e-3) / 1e9
    roof_d = dict(kernel="attn_decode_cascade", bound="hbm", achieved=gbs_plan, peak=PEAK_HBM_GBS, unit="GB/s",
                  frac=gbs_plan / PEAK_HBM_GBS, traffic=measured_traffic("attn_decode_cascade"),
                  algorithmic_bytes=Bp, logical_bytes=Bl)
    dominant_is_decode = dec_ms_live * 1e3 >= ext_alone_us
    out = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "plan_host_ms": dec.plan_ms,
        "ms_per_step_synced": ms_per_step_synced,
        "value_note": "value: the K steps issued back to back, wall clock, HIP events around the decode "
                      "only (decode.us, the roofline); ms_per_step_synced: the same steps with a "
                      "synchronization after each (each step then also waits for its first launch); "
                      "ms_kernels_per_step and the *_in_step times: a pass with HIP events between all calls "
                      "(they lengthen the step by a few per cent); extend.us: the extend alone, back to back. "
                      "value "
                      "excludes host work done before the timed region: the radix tables and the "
                      "prefix-shared decode plan (plan_host_ms, rebuilt per step by a decode loop, where "
                      "decode_loop shows it hidden behind the kernels)",
        "config": {"workload": "llama7b-fewshot-extend (64 req x (1024 shared + 128 new), 32/32 heads, "
                               "D=128, 2^20 slots) + llama7b-radix-decode (256 req, 4-ary depth-3 tree, "
                               "ctx 512-4096)",
                   "global_batch": 64 + 256, "tokens_per_step": tokens, "parallelism": "single-gpu"},
        "extend": extend_obj, "decode": decode_obj, "decode_plain": decode_plain_obj,
        "decode_noshare_control": noshare_obj,
        "roofline": roof_d if dominant_is_decode else roof_e,
        "roofline_other": roof_e if dominant_is_decode else roof_d,
        "ms_kernels_per_step": ms_kernels,
        "host_radix_ns_per_token": {"extend_workload": time_host_radix(ext),
                                    "decode_workload": time_host_radix(dec)},
        "context": "the pages' up-to-6.4x end-to-end throughput was measured on NVIDIA A10G/A100 "
                   "against other serving systems; it is not comparable to this number",
    }
    out["step_graph"] = step_graph(step, tokens, args.steps, args.warmup)
    del ext, dec
    torch.cuda.empty_cache()
    out["gqa_llama70b"] = gqa_halves(max(5, args.steps // 2), 3)
    out["tp8_share"] = tp8_share(max(5, args.steps // 2), 3)
    out["chat_pipeline"] = [chat_pipeline("c5"), chat_pipeline("c5e")]
    out["decode_loop_host"] = decode_loop_host()
    out["decode_loop"] = decode_loop()
    out["cache_aware_scheduling"] = queue_orders()
    out["sampling_penalties"] = sampling_penalties()
    out["multimodal"] = multimodal_replay()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
