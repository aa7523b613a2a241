"""The extend work order (rkv_attn_extend's req_order) changes the schedule
only: on ragged batches of the multi-turn chat trace (up to 64 turns of
32-512 new tokens over cached histories), o and lse with no order, with the
engine's longest-first order and with a seeded random permutation are
bit-identical, and they match the float64 oracle on sampled requests (the
engine's order is longest first on 8 kv heads, dealt over the XCDs on 2)."""
import numpy as np
import pytest
import torch

from inputs import configs, content
from tests import gpu_runner as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from prefix_shared_kv_host_amd import rkv
    rkv.lib()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 2, 64)])
def test_extend_order_is_schedule_only(hq, hkv, d):
    from prefix_shared_kv_host_amd import rkv
    s5, phases = configs.build("c5")
    shape = configs.Shape(f"order-{hq}-{hkv}-{d}", hq, hkv, d, "bf16", 1 << 18, s5.seed)
    ph = phases[:10]
    res, cache = G.run(shape, ph, select=G.sample(9, 3), sparse=True)
    G.check(res, "bf16", f"extend with the engine's order {hq}/{hkv} d{d}")
    checked = 0
    for r in res:
        b, o_eng = r["batch"], r["o_full"]
        B = int(b.host["seq_lens"].shape[0])
        lens = b.host["seq_lens"]
        eng = np.arange(B) if b.order is None else b.order.cpu().numpy()
        assert sorted(eng.tolist()) == list(range(B))
        if hkv % 8 == 0:
            assert np.all(np.diff(lens[eng]) <= 0)      # whole heads per XCD: longest first
        q, _, _ = content.batch_rows(shape.seed, ph[r["phase"]].seqs, b.host["prefix_lens"], hq, hkv, d,
                                     torch.bfloat16, "cuda", shape.q_scale)
        perm = torch.from_numpy(np.random.default_rng(r["phase"]).permutation(B).astype(np.int32)).cuda()
        outs = []
        for order in (None, b.order, perm):
            o = torch.empty_like(q)
            lse = torch.empty(q.shape[0], hq, dtype=torch.float32, device="cuda")
            rkv.attn_extend(q, cache.k_pool, cache.v_pool, o, b.req_to_token, b.qo_indptr, b.prefix_lens,
                            b.max_new, lse=lse, order=order)
            outs.append((o, lse))
        torch.cuda.synchronize()
        for o, lse in outs[1:]:
            assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
            assert torch.equal(lse.view(torch.int32), outs[0][1].view(torch.int32))
        checked += 1
    assert checked >= 8
