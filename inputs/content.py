"""Seeded synthetic content for Q, K and V rows.

This module is an input source shared by the float64 oracle and the GPU path.
It holds none of the attention or radix-tree arithmetic: it only turns a seed
and token ids into numbers.

Content is a pure function of (seed, token prefix): the hash chain

    u[-1] = seed,   u[t] = splitmix64(u[t-1] XOR tok[t])

gives each position a 64-bit key that depends on the whole prefix up to and
including that token.  Element (tag, head, d) of the row at position t is a
standard normal drawn by the Box-Muller transform (Box & Muller, 1958) from the
two 32-bit halves of splitmix64(u[t] XOR tag<<56 XOR (head*D + d)*PHI).
splitmix64 is Steele, Lea & Flood's SplitMix64 output function (2014).

Because the K/V of a token depends on its whole prefix, two requests that share
a prefix get identical K/V for it, and a prefix recomputed after eviction
regenerates the same K/V: "cached prefix = recompute" is then a meaningful
check, and a wrong slot gathers another prefix's vectors.

The chain runs in NumPy uint64 on the host (cheap: one step per token).  Row
values are computed with torch in float64 on whichever device the caller names
and rounded once (round-to-nearest-even) to the requested dtype.
"""
from __future__ import annotations

import numpy as np
import torch

TAG_Q, TAG_K, TAG_V = 1, 2, 3

_GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK64 = (1 << 64) - 1


def _s64(x: int) -> int:
    """Reinterpret an unsigned 64-bit constant as a signed int64."""
    x &= _MASK64
    return x - (1 << 64) if x >> 63 else x


def splitmix64_np(x: np.ndarray) -> np.ndarray:
    """SplitMix64 output function on uint64 arrays (wrapping arithmetic)."""
    with np.errstate(over="ignore"):
        z = x + np.uint64(_GOLDEN)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
        return z ^ (z >> np.uint64(31))


def prefix_keys(seed: int, tokens) -> np.ndarray:
    """u[t] for every position t of one token sequence (uint64 array)."""
    tok = np.asarray(tokens, dtype=np.int64).astype(np.uint64)
    out = np.empty(tok.shape[0], dtype=np.uint64)
    u = np.uint64(seed & _MASK64)
    for t in range(tok.shape[0]):
        u = splitmix64_np(np.array([u ^ tok[t]], dtype=np.uint64))[0]
        out[t] = u
    return out


def prefix_keys_batch(seed: int, seqs) -> list:
    """prefix_keys for many sequences, vectorised across sequences."""
    n = len(seqs)
    if n == 0:
        return []
    lens = np.array([len(s) for s in seqs], dtype=np.int64)
    lmax = int(lens.max()) if n else 0
    mat = np.zeros((n, lmax), dtype=np.uint64)
    for i, s in enumerate(seqs):
        mat[i, : len(s)] = np.asarray(s, dtype=np.int64).astype(np.uint64)
    keys = np.zeros((n, lmax), dtype=np.uint64)
    u = np.full(n, np.uint64(seed & _MASK64), dtype=np.uint64)
    for t in range(lmax):
        u = splitmix64_np(u ^ mat[:, t])
        keys[:, t] = u
    return [keys[i, : lens[i]].copy() for i in range(n)]


def _splitmix64_t(z: torch.Tensor) -> torch.Tensor:
    """SplitMix64 on int64 tensors; >> is made logical by masking."""
    def lsr(v, k):
        return (v >> k) & ((1 << (64 - k)) - 1)

    z = z + _s64(_GOLDEN)
    z = (z ^ lsr(z, 30)) * _s64(_M1)
    z = (z ^ lsr(z, 27)) * _s64(_M2)
    return z ^ lsr(z, 31)


def rows(keys, tag: int, heads: int, dim: int, dtype=torch.float32,
         device="cpu", scale: float = 1.0, chunk_elems: int = 1 << 25) -> torch.Tensor:
    """Rows [N, heads, dim] for the positions whose chain keys are `keys`.

    Values are N(0,1) (times `scale`), computed in float64 and rounded once
    to `dtype`.
    """
    keys = np.ascontiguousarray(np.asarray(keys, dtype=np.uint64))
    n = keys.shape[0]
    out = torch.empty((n, heads, dim), dtype=dtype, device=device)
    if n == 0:
        return out
    k_t = torch.from_numpy(keys.view(np.int64)).to(device)
    col = torch.arange(heads * dim, dtype=torch.int64, device=device)
    salt = (col * _s64(_GOLDEN)) ^ _s64(tag << 56)
    step = max(1, chunk_elems // (heads * dim))
    two32 = float(1 << 32)
    for i in range(0, n, step):
        kk = k_t[i:i + step].unsqueeze(1) ^ salt.unsqueeze(0)
        h = _splitmix64_t(kk)
        a = (h & 0xFFFFFFFF).to(torch.float64)
        b = ((h >> 32) & 0xFFFFFFFF).to(torch.float64)
        u1 = (a + 1.0) / two32
        u2 = b / two32
        z = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * np.pi) * u2)
        if scale != 1.0:
            z = z * scale
        out[i:i + step] = z.view(-1, heads, dim).to(dtype)
    return out


def random_tokens(rng: np.random.Generator, n: int, vocab: int = 32000) -> list:
    """n token ids drawn uniformly from [0, vocab)."""
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32).tolist()


def batch_rows(seed: int, seqs, starts, hq: int, hkv: int, d: int, dtype=torch.float32,
               device="cpu", q_scale: float = 1.0, with_q: bool = True):
    """Q, K, V rows for positions starts[r]..len(seqs[r])-1 of every sequence,
    packed in request order: q [T, hq, d], k and v [T, hkv, d]."""
    keys = prefix_keys_batch(seed, seqs)
    sel = [keys[r][int(starts[r]):] for r in range(len(seqs))]
    flat = np.concatenate(sel) if sel else np.zeros(0, dtype=np.uint64)
    k = rows(flat, TAG_K, hkv, d, dtype, device)
    v = rows(flat, TAG_V, hkv, d, dtype, device)
    q = rows(flat, TAG_Q, hq, d, dtype, device, scale=q_scale) if with_q else None
    return q, k, v


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]
