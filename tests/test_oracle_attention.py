"""Pins for the oracle's attention: brute force, a library routine, closed
forms and invariants.  CPU only."""
import math

import numpy as np
import pytest
import torch

from inputs import configs, content
from oracle import attention as oa
from oracle import pipeline
from oracle.pool import OraclePool, scatter


def brute_force_request(seed, seq, p, hq, hkv, d, dtype, q_scale=1.0):
    """Dense causal attention over the whole sequence with no pool, no tables
    and no cache: Q, K, V for every position come straight from the
    generator; rows p..L-1 are returned.  Written with explicit loops and
    math.fsum so that it shares no code path with the oracle."""
    keys = content.prefix_keys(seed, seq)
    dt = content.torch_dtype(dtype)
    K = content.rows(keys, content.TAG_K, hkv, d, dt).double().numpy()
    V = content.rows(keys, content.TAG_V, hkv, d, dt).double().numpy()
    Q = content.rows(keys, content.TAG_Q, hq, d, dt, scale=q_scale).double().numpy()
    L = len(seq)
    sigma = 1.0 / math.sqrt(d)
    o = np.zeros((L - p, hq, d))
    lse = np.zeros((L - p, hq))
    for i in range(p, L):
        for h in range(hq):
            g = h * hkv // hq
            s = [sigma * math.fsum(Q[i, h, :] * K[t, g, :]) for t in range(i + 1)]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            tot = math.fsum(w)
            for dd in range(d):
                o[i - p, h, dd] = math.fsum(w[t] * V[t, g, dd] for t in range(i + 1)) / tot
            lse[i - p, h] = mx + math.log(tot)
    return o, lse


@pytest.mark.parametrize("seed,hq,hkv", [(11, 4, 2), (12, 2, 2), (13, 4, 1)])
def test_oracle_equals_brute_force_full_sequence(seed, hq, hkv):
    shape, phases = configs.tiny(seed, hq=hq, hkv=hkv, d=16, pool=1024, prefix=9,
                                 new=(1, 5, 12, 3, 7))
    res = pipeline.run(shape, phases)[-1]
    tb = res["tables"]
    for r, seq in enumerate(phases[-1].seqs):
        a, b = tb["qo_indptr"][r], tb["qo_indptr"][r + 1]
        o_bf, lse_bf = brute_force_request(shape.seed, seq, tb["prefix_lens"][r], hq, hkv, 16, "f32")
        assert np.max(np.abs(res["o"][a:b] - o_bf)) <= 1e-12
        assert np.max(np.abs(res["lse"][a:b] - lse_bf)) <= 1e-12


def test_oracle_equals_sdpa_when_no_prefix():
    """p = 0: Q and K have equal length, so the standard causal mask applies;
    torch's scaled_dot_product_attention on CPU in float64 is the pin."""
    rng = np.random.default_rng(5)
    L, D = 37, 32
    q = rng.standard_normal((L, D)); k = rng.standard_normal((L, D)); v = rng.standard_normal((L, D))
    o, _, _ = oa.attend_rows(q, k, v, np.arange(L), 1 / math.sqrt(D))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], is_causal=True, scale=1 / math.sqrt(D))[0, 0].numpy()
    assert np.max(np.abs(o - ref)) <= 1e-12


def test_oracle_equals_sdpa_with_prefix_mask():
    """With a prefix the visible set is keys 0..p+j; an explicit boolean mask
    handed to the library routine expresses the same thing."""
    rng = np.random.default_rng(6)
    p, n, D = 23, 9, 16
    L = p + n
    q = rng.standard_normal((n, D)); k = rng.standard_normal((L, D)); v = rng.standard_normal((L, D))
    o, _, _ = oa.attend_rows(q, k, v, p + np.arange(n), 0.3)
    allowed = torch.arange(L)[None, :] <= (p + torch.arange(n))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], attn_mask=allowed[None, None], scale=0.3)[0, 0].numpy()
    assert np.max(np.abs(o - ref)) <= 1e-12


def test_special_cases_closed_form():
    rng = np.random.default_rng(7)
    D = 8
    # one key: the weight is exactly 1
    q = rng.standard_normal((1, D)); k = rng.standard_normal((1, D)); v = rng.standard_normal((1, D))
    o, lse, w = oa.attend_rows(q, k, v, [0], 0.5)
    assert np.array_equal(o, v) and w[0, 0] == 1.0
    assert lse[0] == pytest.approx(0.5 * float(q[0] @ k[0]), abs=1e-15)
    # all keys equal -> mean of V
    L = 13
    k = np.tile(rng.standard_normal((1, D)), (L, 1)); v = rng.standard_normal((L, D))
    o, _, _ = oa.attend_rows(rng.standard_normal((1, D)), k, v, [L - 1], 0.7)
    assert np.max(np.abs(o[0] - v.mean(axis=0))) <= 1e-12
    # all V rows equal c -> o = c
    c = rng.standard_normal(D)
    o, _, _ = oa.attend_rows(rng.standard_normal((1, D)), rng.standard_normal((L, D)),
                             np.tile(c, (L, 1)), [L - 1], 1.3)
    assert np.max(np.abs(o[0] - c)) <= 1e-12
    # q = 0 -> uniform weights -> mean of V; lse = ln L
    v = rng.standard_normal((L, D))
    o, lse, _ = oa.attend_rows(np.zeros((1, D)), rng.standard_normal((L, D)), v, [L - 1], 1.0)
    assert np.max(np.abs(o[0] - v.mean(axis=0))) <= 1e-12
    assert lse[0] == pytest.approx(math.log(L), abs=1e-12)
    # one logit 40 above all others -> that row, within e^-40 max|v|
    k = np.zeros((L, D)); k[4, 0] = 40.0
    q = np.zeros((1, D)); q[0, 0] = 1.0
    o, _, _ = oa.attend_rows(q, k, v, [L - 1], 1.0)
    assert np.max(np.abs(o[0] - v[4])) <= L * math.exp(-40) * np.abs(v).max()


def test_softmax_rows_sum_to_one_and_lse_consistent():
    rng = np.random.default_rng(8)
    p, n, D = 17, 6, 16
    q = rng.standard_normal((n, D)) * 3; k = rng.standard_normal((p + n, D)); v = rng.standard_normal((p + n, D))
    limits = p + np.arange(n)
    o, lse, w = oa.attend_rows(q, k, v, limits, 0.25)
    assert np.max(np.abs(w.sum(axis=1) - 1.0)) <= 1e-12
    s = 0.25 * q @ k.T
    for i in range(n):
        vis = s[i, : limits[i] + 1]
        assert abs(np.exp(vis - lse[i]).sum() - 1.0) <= 1e-12
        assert np.all(w[i, limits[i] + 1:] == 0.0)


@pytest.mark.parametrize("cuts", [[5], [1, 2, 3], [7, 19, 20], list(range(1, 40, 3))])
def test_split_merge_algebra(cuts):
    """Any partition of the keys into contiguous ranges, merged by rescaling
    (m, l, acc), equals the unsplit result."""
    rng = np.random.default_rng(9)
    L, D = 41, 16
    q = rng.standard_normal(D) * 2; k = rng.standard_normal((L, D)); v = rng.standard_normal((L, D))
    full_o, full_lse, _ = oa.attend_rows(q[None], k, v, [L - 1], 0.4)
    bounds = [0] + list(cuts) + [L]
    states = [oa.partial_state(q, k[a:b], v[a:b], 0.4) for a, b in zip(bounds[:-1], bounds[1:])]
    o, lse = oa.merge_states(states)
    assert np.max(np.abs(o - full_o[0])) <= 1e-12
    assert abs(lse - full_lse[0]) <= 1e-12


def _recompute(shape, seqs):
    """Every sequence from scratch on a fresh tree: one request per batch,
    nothing cached."""
    outs = []
    for s in seqs:
        ph = [configs.Phase("extend", [s])]
        outs.append(pipeline.run(shape, ph)[0]["o"])
    return outs


def test_cached_prefix_equals_recompute():
    shape, phases = configs.c1()
    res = pipeline.run(shape, phases)[-1]
    tb = res["tables"]
    assert tb["prefix_lens"] == [64] * 4
    scratch = _recompute(shape, phases[-1].seqs)
    for r, full in enumerate(scratch):
        a, b = tb["qo_indptr"][r], tb["qo_indptr"][r + 1]
        assert np.max(np.abs(res["o"][a:b] - full[64:])) <= 1e-12


def test_extend_with_one_new_token_equals_decode():
    shape, phases = configs.tiny(21, hq=4, hkv=2, d=16, new=(1, 1, 1, 1, 1))
    res = pipeline.run(shape, phases, keep=(keep := {}))[-1]
    tb = res["tables"]
    assert tb["qo_indptr"] == list(range(6))
    q, _, _ = content.batch_rows(shape.seed, phases[-1].seqs, tb["prefix_lens"], 4, 2, 16)
    o_dec, lse_dec = oa.decode(q.double().numpy(), keep["pool"], tb["req_to_token"], tb["seq_lens"], 4, 2)
    assert np.array_equal(o_dec, res["o"]) and np.array_equal(lse_dec, res["lse"])


def test_unwritten_slot_reads_as_nan_and_scatter_is_exact():
    pool = OraclePool(16, 2, 4)
    k = torch.arange(24, dtype=torch.float32).view(3, 2, 4)
    scatter(pool, [5, 1, 9], k, -k)
    K, V = pool.gather([1, 5, 9, 2])
    assert np.array_equal(K[0], k[1].numpy()) and np.array_equal(K[1], k[0].numpy())
    assert np.array_equal(V[2], -k[2].numpy())
    assert np.all(np.isnan(K[3])) and np.all(np.isnan(V[3]))


# ----------------------------------------------------------------------------
# Planted mistakes: each plausible bug in the oracle must trip a pin above.

def _mutant_attend(kind):
    real = oa.attend_rows

    def f(q, K, V, limits, scale):
        if kind == "mask_off_by_one":
            return real(q, K, V, np.asarray(limits) - 1 if len(K) > 1 else limits, scale)
        if kind == "no_scale":
            return real(q, K, V, limits, 1.0)
        if kind == "transposed_v":
            o, lse, w = real(q, K, V, limits, scale)
            return (w @ V[::-1]), lse, w
        raise AssertionError(kind)
    return f


@pytest.mark.parametrize("kind", ["mask_off_by_one", "no_scale", "transposed_v"])
def test_planted_attention_mistakes_are_caught(kind, monkeypatch):
    monkeypatch.setattr(oa, "attend_rows", _mutant_attend(kind))
    with pytest.raises(AssertionError):
        test_oracle_equals_brute_force_full_sequence(11, 4, 2)


def test_planted_gqa_mapping_mistake_is_caught(monkeypatch):
    real = oa.extend

    def wrong(q, pool, r2t, indptr, pl, hq, hkv, scale=None, requests=None):
        # pairs q head h with kv head h % hkv instead of h // (hq/hkv)
        qq = np.asarray(q).copy()
        perm = [(h % hkv) * (hq // hkv) + h // hkv for h in range(hq)]
        o, lse = real(qq[:, perm], pool, r2t, indptr, pl, hq, hkv, scale, requests)
        inv = np.argsort(perm)
        return o[:, inv], lse[:, inv]
    monkeypatch.setattr(pipeline, "extend", wrong)
    with pytest.raises(AssertionError):
        test_oracle_equals_brute_force_full_sequence(11, 4, 2)
