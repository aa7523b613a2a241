"""Batches whose requests all have the same number of new tokens take a
shorter request lookup in rkv_attn_extend (bf16): the request and tile come
from the work item's index and the prefix length is loaded beside the first
slot indices.  On such batches (short requests, whose keys end inside the
first three key tiles, and longer ones; with and without a request order)
o and lse are bit-identical to the general lookup, which a max_new one larger
than every request's count selects, and they match the float64 oracle."""
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


CASES = [
    # (seed, hq, hkv, d, prefix, new): 5 requests with `new` new tokens each,
    # 4 of them behind a shared cached prefix and one with none
    (51, 8, 2, 128, 70, 37),      # every request ends inside the first three key tiles
    (52, 8, 2, 128, 300, 129),    # several row tiles per request; one short request
    (53, 4, 1, 64, 190, 1),       # one query row per request, keys end at 191
    (54, 32, 32, 128, 1024, 16),  # multi-head, one key tile past the prefix
    (55, 4, 1, 128, 128, 64),     # keys end exactly at the third tile's end (192)
    (56, 4, 1, 128, 127, 64),     # one key short of it (191): the slots are read again
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("seed,hq,hkv,d,prefix,new", CASES)
def test_uniform_lookup_is_bit_identical(seed, hq, hkv, d, prefix, new):
    from prefix_shared_kv_host_amd import rkv
    shape, phases = configs.tiny(seed, hq=hq, hkv=hkv, d=d, dtype="bf16", pool=8192, prefix=prefix,
                                 new=(new,) * 5)
    res, cache = G.run(shape, phases)
    G.check(res, "bf16", f"uniform extend {hq}/{hkv} d{d} p{prefix} n{new}")
    (r,) = res
    b = r["batch"]
    B = int(b.host["seq_lens"].shape[0])
    assert b.max_new == new and b.total_new == B * new
    q, _, _ = content.batch_rows(shape.seed, phases[r["phase"]].seqs, b.host["prefix_lens"], hq, hkv, d,
                                 torch.bfloat16, "cuda", shape.q_scale)
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(B).astype(np.int32)).cuda()
    outs = []
    for max_new in (new, new + 1):           # uniform lookup, then the general one
        for order in (None, perm):
            o = torch.empty_like(q)
            lse = torch.empty(q.shape[0], hq, dtype=torch.float32, device="cuda")
            rkv.attn_extend(q, cache.k_pool, cache.v_pool, o, b.req_to_token, b.qo_indptr, b.prefix_lens,
                            max_new, lse=lse, order=order)
            outs.append((o, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(torch.int16), r["o_full"].view(torch.int16))
    for o, lse in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(lse.view(torch.int32), outs[0][1].view(torch.int32))
