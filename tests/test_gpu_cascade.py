"""GPU parity of prefix-shared ("cascade") decode (rkv_attn_decode_cascade)
against the float64 oracle's plain decode attention, with the native plan
asserted equal to the oracle's plan on every batch.

Workloads: random prefix trees of decode requests (several sharing levels,
identical histories, one-token requests, ragged lengths) over every
query-per-kv-head ratio the MFMA phase handles and both head dims, with plan
settings that exercise folding, short chunks, ragged tails and member groups
of one; then sampled requests of the radix-tree decode batch (256 requests),
its no-share control (no shared run: tails only) and the grouped-head decode
batch (64 requests under one 2048-token prefix).  Tolerances as for plain
decode: max-abs 2e-2 on o, lse within ln(1 + 2^-8) (weights rounded to bf16
on the matrix cores)."""
import numpy as np
import pytest
import torch

from inputs import configs
from tests import gpu_runner as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from prefix_shared_kv_host_amd import rkv
    rkv.lib()
    G.log(f"device: {torch.cuda.get_device_name(0)}")


def tree_decode_workload(seed, B=24, max_len=1400):
    """Histories cached in a setup batch, then one decode batch.  Request i
    copies a cut of an earlier request's history (often at a deep point, so
    runs nest several levels) and appends fresh tokens; a few copy a whole
    history (identical rows but the query key); some are one token long."""
    rng = np.random.default_rng(seed)
    hist = []
    for i in range(B):
        if i >= 2 and i % 11 == 0:
            h = list(hist[int(rng.integers(len(hist)))])
        elif i % 13 == 5:
            h = []
        elif hist and rng.random() < 0.8:
            base = hist[int(rng.integers(len(hist)))]
            cut = int(rng.integers(len(base) // 3, len(base) + 1)) if base else 0
            n = int(rng.integers(1, 400))
            h = base[:cut] + [int(x) for x in rng.integers(0, 32000, n)]
            if cut < len(base):
                h[cut] = 60000 + i                     # branch off at the cut
        else:
            h = [int(x) for x in rng.integers(0, 32000, int(rng.integers(2, max_len)))]
            h[0] = 70000 + i
        hist.append(h[:max_len])
    full = [h + [80000 + i] for i, h in enumerate(hist)]
    return [configs.Phase("setup", [h for h in hist if h]), configs.Phase("decode", full)]


CASES = [
    # hq, hkv, d, plan settings
    (4, 4, 128, dict(seg_chunk=256, tail_chunk=768, min_keys=32)),
    (4, 4, 128, dict(seg_chunk=100, tail_chunk=128, min_keys=1)),
    (8, 4, 64, dict(seg_chunk=64, tail_chunk=200, min_keys=8)),
    (8, 2, 128, dict(seg_chunk=256, tail_chunk=768, min_keys=32)),
    (16, 2, 128, dict(seg_chunk=96, tail_chunk=320, min_keys=1, max_members=1)),
    (16, 1, 64, dict(seg_chunk=256, tail_chunk=512, min_keys=16)),
    (12, 2, 128, dict(seg_chunk=160, tail_chunk=768, min_keys=4)),
    (3, 1, 128, dict(seg_chunk=256, tail_chunk=384, min_keys=32, max_members=3)),
    (2, 2, 64, dict(seg_chunk=32, tail_chunk=64, min_keys=1)),
    # chunks of 33 and 65 keys: every shared and tail item ends inside a
    # 32-key step of the grouped-head walk
    (16, 2, 128, dict(seg_chunk=33, tail_chunk=65, min_keys=1)),
]


@pytest.mark.parametrize("hq,hkv,d,plan", CASES)
def test_cascade_tree_decode(hq, hkv, d, plan):
    shape = configs.Shape(f"cas-{hq}-{hkv}-{d}", hq, hkv, d, "bf16", 1 << 16, 51)
    phases = tree_decode_workload(seed=hq * 100 + d + plan["tail_chunk"])
    res, _ = G.run(shape, phases, content_device="cpu", cascade=plan)
    G.check(res, "bf16", f"cascade {hq}/{hkv} d{d} {plan}")


@pytest.mark.timeout(400)
@pytest.mark.parametrize("d", [64, 128])
def test_cascade_streaming_tails(d):
    """Grouped-head launches with at least 2048 tail slots take the variant
    whose tail V tiles stream in (non-temporal DMA): 64 requests x 8 kv heads
    with tails of up to 4 chunks of 768 keys, on both head dims."""
    shape = configs.Shape(f"cas-stream-{d}", 32, 8, d, "bf16", 1 << 18, 71)
    phases = tree_decode_workload(seed=d + 71, B=64, max_len=3000)
    res, _ = G.run(shape, phases, content_device="cpu", cascade=dict(tail_chunk=768),
                   select=G.sample(3, 12), sparse=True)
    G.check(res, "bf16", f"cascade streaming tails d{d}")


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name", ["c3", "c3ns"])
def test_cascade_c3_sampled(name):
    shape, phases = configs.build(name)
    res, _ = G.run(shape, phases, select=G.sample(5, 24), sparse=True, cascade={})
    G.check(res, "bf16", f"{name} cascade")


@pytest.mark.timeout(400)
def test_cascade_c4_decode_sampled():
    shape, phases = configs.c4()
    ph = [phases[0], phases[1], phases[3]]
    res, _ = G.run(shape, ph, select=G.sample(6, 16), sparse=True, cascade={})
    G.check(res, "bf16", "c4-decode cascade")


ORDER_CASES = [
    # hq, hkv, d: tails on the vector kernel, on the matrix cores, and a
    # small grouped-head launch (halved tail chunk)
    (32, 32, 128),
    (32, 8, 128),
    (8, 1, 64),
]


@pytest.mark.timeout(400)
@pytest.mark.parametrize("hq,hkv,d", ORDER_CASES)
def test_cascade_tail_order_changes_only_the_schedule(hq, hkv, d):
    """The order in which the tail splits are handed out (the engine's
    longest-first order, batch order, a reversed order) changes no output
    bit; an order entry outside [0, B) is skipped without touching the
    other requests' outputs."""
    from inputs import content
    shape = configs.Shape(f"cas-order-{hq}-{hkv}-{d}", hq, hkv, d, "bf16", 1 << 17, 91)
    phases = tree_decode_workload(seed=hq + hkv + d, B=48, max_len=2500)
    res, cache = G.run(shape, phases, content_device="cpu", cascade={}, select=G.sample(2, 8), sparse=True)
    G.check(res, "bf16", f"cascade tail order {hq}/{hkv} d{d}")
    (r,) = res
    b = r["batch"]
    seqs = phases[-1].seqs
    B = len(seqs)
    q, _, _ = content.batch_rows(shape.seed, seqs, b.host["prefix_lens"], hq, hkv, d, torch.bfloat16, "cuda",
                                 shape.q_scale)
    eng = cache.cascade_plan_host(b, hq)
    # the engine's order (a small launch keeps batch order: then requests by
    # length, longest first)
    base = eng.tail_order
    if base is None:
        base = np.argsort(-b.host["seq_lens"].astype(np.int64), kind="stable").astype(np.int32)
    assert sorted(base.tolist()) == list(range(B))

    def decode(order):
        p = cache.cascade_plan_host(b, hq, longest_tails_first=False)
        assert p.tail_order is None
        p.tail_order = None if order is None else np.asarray(order, dtype=np.int32)
        p.to("cuda")
        o = torch.empty_like(q)
        lse = torch.empty(B, hq, dtype=torch.float32, device="cuda")
        cache.decode_cascade(b, q, plan=p, o=o, lse=lse)
        torch.cuda.synchronize()
        return o.view(torch.int16).cpu(), lse.view(torch.int32).cpu()

    ref = decode(base)
    assert torch.equal(ref[0], r["o_full"].view(torch.int16).cpu())
    for order in (None, np.arange(B)[::-1]):
        out = decode(order)
        assert torch.equal(out[0], ref[0]) and torch.equal(out[1], ref[1])
    bad = base.copy()
    victim = int(bad[0])
    bad[0] = B + 5
    out = decode(bad)
    keep = torch.ones(B, dtype=torch.bool)
    keep[victim] = False
    assert torch.equal(out[0][keep], ref[0][keep]) and torch.equal(out[1][keep], ref[1][keep])
