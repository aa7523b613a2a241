"""The decode entry point that allocates nothing (rkv_attn_decode_noalloc)
against rkv_attn_decode with a caller workspace, through the C ABI: bit-equal
o and lse on two calls in a row, the second with a smaller batch (the scratch
keeps the first call's partials, which must not leak into the second), on the
vector-unit path and the grouped-head matrix-core path; sizes beyond the
scratch are refused."""
import numpy as np
import pytest
import torch

from inputs import configs, content

pytestmark = pytest.mark.gpu


def _decode_batch(cache, seqs, shape):
    from prefix_shared_kv_host_amd import rkv
    batch = cache.prepare(seqs)
    dt = content.torch_dtype(shape.dtype)
    q, k, v = content.batch_rows(shape.seed, seqs, batch.host["prefix_lens"], shape.hq, shape.hkv, shape.d, dt,
                                 "cuda", shape.q_scale)
    cache.store(batch, k, v)
    return batch, q


def _both(cache, batch, q, num_splits):
    from prefix_shared_kv_host_amd import rkv
    B, hq, d = q.shape
    o1, o2 = torch.empty_like(q), torch.full_like(q, float("nan"))
    l1 = torch.empty(B, hq, dtype=torch.float32, device="cuda")
    l2 = torch.full((B, hq), float("nan"), dtype=torch.float32, device="cuda")
    ws = cache.workspace(B, hq, batch.max_len, num_splits)
    rkv.attn_decode(q, cache.k_pool, cache.v_pool, o1, batch.req_to_token, batch.seq_lens, batch.max_len, ws,
                    lse=l1, num_splits=num_splits)
    rkv.attn_decode_noalloc(q, cache.k_pool, cache.v_pool, o2, batch.req_to_token, batch.seq_lens,
                            batch.max_len, lse=l2, num_splits=num_splits)
    torch.cuda.synchronize()
    bits = torch.int16 if q.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(o1.view(bits), o2.view(bits))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    assert not torch.isnan(o2.float()).any()


@pytest.mark.parametrize("hq,hkv,num_splits", [(8, 8, 0), (16, 2, 0), (8, 1, 5)])
def test_noalloc_equals_decode_with_workspace(hq, hkv, num_splits):
    from prefix_shared_kv_host_amd.engine import RadixKVCache
    shape = configs.Shape(f"noalloc-{hq}-{hkv}", hq, hkv, 128, "bf16", 1 << 16, 91)
    rng = np.random.default_rng(91 + hq)
    hist = [[int(x) for x in rng.integers(0, 32000, int(L))] for L in rng.integers(700, 4000, 24)]
    for i, h in enumerate(hist):
        h[0] = 40000 + i
    cache = RadixKVCache(shape.pool, hkv, 128, torch.bfloat16, "cuda", configs.free_list(shape.pool, shape.seed))
    setup = cache.prepare(hist)
    _, k, v = content.batch_rows(shape.seed, hist, setup.host["prefix_lens"], hq, hkv, 128, torch.bfloat16,
                                 "cuda", with_q=False)
    cache.store(setup, k, v)
    cache.commit(setup)
    # first call: every history + 1 token; second: a smaller, shorter batch
    big = [h + [7] for h in hist]
    small = [h[: len(h) // 3] + [9] for h in hist[:5]]
    for seqs in (big, small):
        batch, q = _decode_batch(cache, seqs, shape)
        _both(cache, batch, q, num_splits)
        cache.commit(batch)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    from prefix_shared_kv_host_amd import rkv
    B, hq, d, L = 512, 64, 128, 8192
    need = rkv.attn_decode_workspace_bytes(B, hq, d, L)
    assert need > rkv.DECODE_NOALLOC_MAX_BYTES
    q = torch.zeros(B, hq, d, dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros(16, 8, d, dtype=torch.bfloat16, device="cuda")
    r2t = torch.zeros(B, L, dtype=torch.int32, device="cuda")
    sl = torch.ones(B, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    with pytest.raises(rkv.RkvError) as e:
        rkv.attn_decode_noalloc(q, pool, pool, o, r2t, sl, L)
    assert e.value.code == rkv.EINVAL and "entry point holds" in str(e.value)
