"""Radix keys of multimodal inputs: rkv_image_keys against the oracle
(oracle/mm_keys.py), and the reuse they give in the tree.

Pins of the oracle:
  * FNV-1a 64: the empty input hashes to the offset basis 0xcbf29ce484222325,
    a one-byte input to (basis XOR byte) * prime mod 2^64, and the published
    test vectors "a" -> 0xaf63dc4c8601ec8c, "foobar" -> 0x85944171f73967e8;
  * splitmix64 started at 0: the published first outputs 0xe220a8397b1dcdaf,
    0x6e789e6aa1b965f4, 0x06c45d188009454f.
Native against oracle: keys and hashes bit-exact on random images.  Tree
semantics on the LLaVA-style trace: a later question about an image reuses
the system prompt and the whole image; a question about another image reuses
the system prompt only; with one constant placeholder id for every image the
tree would hand one image's KV to another (the failure the hash prevents).
Hit rate on the full trace equals a closed form counted from the trace's
structure alone."""
import os

import numpy as np
import pytest

from inputs import configs
from oracle import mm_keys as om
from oracle.radix import OK, OracleTree
from prefix_shared_kv_host_amd import mm, rkv


def test_published_hash_vectors():
    basis, prime = 0xCBF29CE484222325, 0x100000001B3
    assert om.fnv1a64(b"") == basis
    assert om.fnv1a64(b"a") == ((basis ^ 0x61) * prime) % (1 << 64) == 0xAF63DC4C8601EC8C
    assert om.fnv1a64(b"foobar") == 0x85944171F73967E8
    assert om.splitmix64(0, 3) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


@pytest.mark.parametrize("n", [0, 1, 2, 7, 64, 4096, 100003])
def test_native_keys_equal_oracle(n):
    data = os.urandom(n)
    for count in (0, 1, 576):
        k, h = rkv.image_keys(data, count)
        ko, ho = om.image_keys(data, count)
        assert h == ho
        assert k.tolist() == ko


def test_key_range_and_distinctness():
    rng = np.random.default_rng(0)
    firsts = set()
    for i in range(2000):
        data = rng.integers(0, 256, 64, dtype=np.uint8).tobytes()
        k, _ = rkv.image_keys(data, 16)
        assert (k <= -1).all() and (k >= -(1 << 31)).all()
        assert len(set(k.tolist())) == 16
        assert rkv.image_keys(data, 16)[0].tolist() == k.tolist()
        firsts.add(tuple(k.tolist()))
    assert len(firsts) == 2000
    with pytest.raises(rkv.RkvError):
        rkv.image_keys(b"x", -1)


def _replay(tree_cls, batches, pool=1 << 18):
    t = tree_cls(pool, list(range(pool)))
    reuse = []
    for seqs in batches:
        if tree_cls is OracleTree:
            st, tb = t.batch_prepare(seqs)
            assert st == OK
            t.batch_commit(seqs, tb["req_to_token"], tb["nodes"])
            reuse.append([int(x) for x in tb["prefix_lens"]])
        else:
            code, tb = t.batch_prepare(seqs)
            assert code == rkv.OK
            t.batch_commit(seqs, tb["req_to_token"], tb["nodes"])
            reuse.append(tb["prefix_lens"].tolist())
    return reuse, t


def _small_trace():
    return configs.mm_trace(seed=3, images=6, questions=3, image_bytes=512, max_batch=4)


def test_tree_reuse_hashed_vs_placeholder():
    sys_tokens, blobs, batches = _small_trace()
    n_img = 40
    seqs = mm.trace_batches((sys_tokens, blobs, batches), n_img)
    oseqs = [[om.request_tokens(sys_tokens, blobs[i], n_img, q) for i, q in b] for b in batches]
    assert seqs == oseqs
    reuse, _ = _replay(rkv.Tree, seqs)
    oreuse, _ = _replay(OracleTree, oseqs)
    assert reuse == oreuse
    S = len(sys_tokens)
    seen = set()
    for k, b in enumerate(batches):
        for (img, _), p in zip(b, reuse[k]):
            expect = (S if k > 0 else 0) + (n_img if img in seen else 0)
            assert p == expect
        seen |= {img for img, _ in b}
    # one constant placeholder for every image: a later request with another
    # image matches that image's positions too
    place = [[list(sys_tokens) + [32000] * n_img + list(q) for _, q in b] for b in batches]
    preuse, _ = _replay(rkv.Tree, place)
    wrong = 0
    seen = set()
    for k, b in enumerate(batches):
        for (img, _), p in zip(b, preuse[k]):
            if img not in seen:
                wrong += max(0, min(p, S + n_img) - S)
        seen |= {img for img, _ in b}
    assert wrong > 0


def test_trace_hit_rate_closed_form():
    s, trace, n_img = configs.mm()
    sys_tokens, blobs, batches = trace
    seqs = mm.trace_batches(trace, n_img)
    reuse, t = _replay(rkv.Tree, seqs, pool=s.pool)
    S = len(sys_tokens)
    seen, exp = set(), 0
    for k, b in enumerate(batches):
        exp += sum((S if k > 0 else 0) + (n_img if img in seen else 0) for img, _ in b)
        seen |= {img for img, _ in b}
    assert sum(map(sum, reuse)) == exp
    prompt = sum(len(x) for b in seqs for x in b)
    st = t.stats()
    assert st[5] == exp and st[6] == prompt
