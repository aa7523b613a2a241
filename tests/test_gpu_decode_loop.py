"""GPU parity of a decode loop that extends a prepared batch step by step
(engine.append: rkv_batch_append on the host tables, rkv_table_append on the
device ones) against the oracle tree driven through the same steps and the
float64 oracle's decode attention.

Every step: the device token table and lengths equal the oracle's bit for bit,
the new slots too, and plain decode (and prefix-shared decode on the
grouped-head case) over the grown rows is within the decode tolerances; after
the final commit the native tree dump equals the oracle's.  A pool small
enough that the steps evict cached leaves is one of the cases."""
import numpy as np
import pytest
import torch

from inputs import configs, content
from oracle import attention as oatt
from oracle.pool import OraclePool, scatter as oscatter
from oracle.radix import OracleTree
from tests import gpu_runner as G
from tests.test_decode_append import decode_tokens, histories

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from prefix_shared_kv_host_amd import rkv
    rkv.lib()


CASES = [
    # hq, hkv, d, dtype, pool, steps
    (8, 2, 128, "bf16", 1 << 14, 12),
    (4, 4, 64, "f32", 1 << 14, 9),
    (16, 2, 128, "bf16", 4900, 40),      # the steps evict the unrelated cached sequences
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("hq,hkv,d,dtype,pool,steps", CASES)
def test_decode_loop_append(hq, hkv, d, dtype, pool, steps):
    from prefix_shared_kv_host_amd.engine import RadixKVCache
    seed = hq * 10 + d
    G.log(f"decode loop {hq}/{hkv} d{d} {dtype} pool {pool} steps {steps}")
    dt = content.torch_dtype(dtype)
    hist = histories(seed, B=24, max_len=500)
    B, ld = len(hist), 500 + steps + 2
    perm = configs.free_list(pool, seed)
    otree, opool = OracleTree(pool, perm), OraclePool(pool, hkv, d)
    cache = RadixKVCache(pool, hkv, d, dt, "cuda", perm)

    def store(seqs, starts, ob, nb):
        _, k, v = content.batch_rows(seed, seqs, starts, hq, hkv, d, dt, "cpu", with_q=False)
        oscatter(opool, np.asarray(ob, dtype=np.int64), k, v)
        cache.store(nb, k.to("cuda"), v.to("cuda"))

    for i in range(2):
        if i == 0:
            seqs = hist
        else:
            # unrelated 60-token sequences: 10, or on the small pool as many as
            # leave ~500 slots free, fewer than the steps will take
            free = otree.stats()[1]
            n = 10 if pool >= 1 << 14 else (free - 500) // 60
            seqs = [[200000 + 100 * j + x for x in range(60)] for j in range(n)]
        st, otb = otree.batch_prepare(seqs)
        assert st == 0
        nb = cache.prepare(seqs)
        store(seqs, otb["prefix_lens"], otb["new_slots"], nb)
        otree.batch_commit(seqs, otb["req_to_token"], otb["nodes"])
        cache.commit(nb)

    seqs = [h + [t] for h, t in zip(hist, decode_tokens(0, B))]
    st, otb = otree.batch_prepare(seqs, ld)
    assert st == 0
    nb = cache.prepare(seqs, ld)
    store(seqs, otb["prefix_lens"], otb["new_slots"], nb)
    o_r2t, o_lens = otb["req_to_token"], list(otb["seq_lens"])
    mm = None
    for k in range(steps + 1):
        if k > 0:
            st, new = otree.batch_append(o_r2t, o_lens)
            assert st == 0, k
            cache.append(nb)
            assert nb.new_slots.cpu().tolist() == new, k
            seqs = [s + [t] for s, t in zip(seqs, decode_tokens(k, B))]
            store(seqs, [L - 1 for L in o_lens], new, nb)
        assert nb.req_to_token.cpu().numpy().tolist() == o_r2t, k
        assert nb.seq_lens.cpu().tolist() == o_lens, k
        assert nb.host["seq_lens"].tolist() == o_lens, k
        assert nb.max_len == max(o_lens)
        q, _, _ = content.batch_rows(seed, seqs, [L - 1 for L in o_lens], hq, hkv, d, dt, "cpu")
        rq = sorted(np.random.default_rng(seed + k).choice(B, size=6, replace=False).tolist())
        o_ref, l_ref = oatt.decode(q.float().numpy(), opool, o_r2t, o_lens, hq, hkv, requests=rq)
        qd = q.to("cuda")
        lse = torch.full((B, hq), float("nan"), device="cuda")
        outs = [("plain", cache.decode(nb, qd, lse=lse))]
        if hq // hkv >= 4 and k % 4 == 0:
            if mm is None:
                from prefix_shared_kv_host_amd import rkv
                mm = rkv.cascade_max_members(hq, hkv, d)
            lse2 = torch.full((B, hq), float("nan"), device="cuda")
            plan = cache.cascade_plan(nb, hq, seg_chunk=64, tail_chunk=96, min_keys=8, max_members=mm)
            outs.append(("cascade", cache.decode_cascade(nb, qd, plan=plan, lse=lse2), lse2))
        torch.cuda.synchronize()
        for item in outs:
            name, o = item[0], item[1]
            lg = (lse if name == "plain" else item[2]).cpu().numpy()[rq]
            res = [dict(phase=k, o=o.float().cpu().numpy()[rq], o_ref=o_ref[rq], lse=lg, lse_ref=l_ref[rq])]
            G.check(res, dtype, f"step {k} {name}")
    otree.batch_commit(seqs, o_r2t, otb["nodes"])
    cache.commit(nb, seqs)
    from tests.native_tree import NativeTree
    nt = NativeTree.__new__(NativeTree)
    nt.t = cache.tree
    assert nt.serialize() == otree.serialize()
    assert cache.tree.free_list() == otree.free_list()
    if pool < 1 << 14:
        assert otree.stats()[7] > 0
