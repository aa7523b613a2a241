"""Oracle attention over a token-slot KV pool, in float64.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the native library and never imports it.

What is computed.  RadixAttention lets a request reuse the KV cache of its
longest cached prompt prefix instead of recomputing it (unite.ai, "SGLang:
Efficient Execution of Structured Language Model Programs", section
"Introduccion a SGLang", RadixAttention bullet; walkthrough Step 3).  The
attention that consumes that cache is plain causal softmax attention: request
r has p cached tokens and n new ones; its new row j sits at absolute position
c = p + j and sees keys 0..c (inclusive).  The pages say nothing more; the
readings taken are

  * scale sigma = 1/sqrt(D);
  * grouped heads: q head h reads kv head floor(h / (Hq/Hkv));
  * K_t, V_t are pool rows req_to_token[r, t] (the oracle tree's own table);
  * o = sum_t softmax_t(sigma q.K_t) V_t, lse = m + ln(l) in natural log;
  * decode is the same formula with n = 1 (the query is the last position).

Everything runs in float64 on values already rounded to the input dtype.  A
matrix product is used as a library step; there is no blocking or fusion.
"""
from __future__ import annotations

import math

import numpy as np


def attend_rows(q, K, V, limits, scale):
    """Causal softmax attention of rows q [n, D] over K, V [L, D].

    Row i sees keys 0..limits[i].  Returns (o [n, D], lse [n], w [n, L]) with
    w the normalised softmax weights (zero where masked).
    """
    q = np.asarray(q, dtype=np.float64)
    s = scale * (q @ K.T)
    L = K.shape[0]
    mask = np.arange(L)[None, :] > np.asarray(limits)[:, None]
    s = np.where(mask, -np.inf, s)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    w = e / l
    o = w @ V
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse, w


def extend(q, pool, req_to_token, qo_indptr, prefix_lens, hq, hkv, scale=None,
           requests=None):
    """Extend attention for a batch.

    q is [T, Hq, D] packed by qo_indptr; returns (o [T, Hq, D], lse [T, Hq])
    in float64.  Rows of requests not in `requests` (when given) are left NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    T, _, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    group = hq // hkv
    o = np.full((T, hq, D), np.nan)
    lse = np.full((T, hq), np.nan)
    B = len(prefix_lens)
    for r in (range(B) if requests is None else requests):
        a, b = int(qo_indptr[r]), int(qo_indptr[r + 1])
        n, p = b - a, int(prefix_lens[r])
        K, V = pool.gather(req_to_token[r][: p + n])
        limits = p + np.arange(n)
        for h in range(hq):
            g = h // group
            oo, ll, _ = attend_rows(q[a:b, h, :], K[:, g, :], V[:, g, :], limits, scale)
            o[a:b, h, :] = oo
            lse[a:b, h] = ll
    return o, lse


def decode(q, pool, req_to_token, seq_lens, hq, hkv, scale=None, requests=None):
    """Single-token decode: q [B, Hq, D], the query of request r at position
    seq_lens[r]-1 sees all seq_lens[r] keys.  Returns (o [B, Hq, D], lse)."""
    q = np.asarray(q, dtype=np.float64)
    B, _, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    group = hq // hkv
    o = np.full((B, hq, D), np.nan)
    lse = np.full((B, hq), np.nan)
    for r in (range(B) if requests is None else requests):
        L = int(seq_lens[r])
        K, V = pool.gather(req_to_token[r][:L])
        for h in range(hq):
            g = h // group
            oo, ll, _ = attend_rows(q[r:r + 1, h, :], K[:, g, :], V[:, g, :], [L - 1], scale)
            o[r, h, :] = oo[0]
            lse[r, h] = ll[0]
    return o, lse


def partial_state(q, K, V, scale):
    """Unnormalised softmax state of one query over a contiguous key range:
    (m, l, acc) with m = max score, l = sum exp(s - m), acc = sum exp(s - m) V."""
    s = scale * (K @ np.asarray(q, dtype=np.float64))
    m = s.max()
    e = np.exp(s - m)
    return m, e.sum(), e @ V


def merge_states(states):
    """Combine per-range (m, l, acc) states: every part is rescaled to the
    global max before summing.  Returns (o, lse)."""
    M = max(st[0] for st in states)
    l = sum(st[1] * math.exp(st[0] - M) for st in states)
    acc = sum(st[2] * math.exp(st[0] - M) for st in states)
    return acc / l, M + math.log(l)
