"""Oracle of the radix keys of multimodal inputs.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the native library and never imports it.

For RadixAttention on multimodal models the runtime hashes each input image
and uses the hash as the radix-tree key, so requests with the same image
reuse the KV of its tokens (unite.ai, "SGLang: Efficient Execution of
Structured Language Model Programs", section "Resultados en modelos
multimodales").  The page names no hash and no way to turn it into token
keys; the readings taken:

  * content hash: 64-bit FNV-1a over the image bytes (its published
    definition: offset basis 14695981039346656037, prime 1099511628211, XOR
    each byte then multiply, modulo 2^64);
  * an image occupying n positions gets n keys, one per position, from
    splitmix64 seeded with the hash (its published definition: the state
    advances by 0x9e3779b97f4a7c15 and each output is the state passed
    through two xor-shift-multiply rounds and a final xor-shift); key i is
    -1 - (output_i >> 33), in [-2^31, -1], so it never equals a text id.
"""
from __future__ import annotations

M64 = (1 << 64) - 1


def fnv1a64(data: bytes) -> int:
    h = 14695981039346656037
    for byte in data:
        h ^= byte
        h = (h * 1099511628211) & M64
    return h


def splitmix64(state: int, count: int):
    """The first `count` outputs of splitmix64 started at `state`."""
    out = []
    for _ in range(count):
        state = (state + 0x9E3779B97F4A7C15) & M64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
        out.append(z ^ (z >> 31))
    return out


def image_keys(data: bytes, n_tokens: int):
    """(keys, hash): the n_tokens radix keys of an image and its hash."""
    h = fnv1a64(data)
    return [-1 - (z >> 33) for z in splitmix64(h, n_tokens)], h


def request_tokens(prefix, image: bytes, n_image_tokens: int, suffix):
    """prefix text ids, then the image's keys, then suffix text ids."""
    keys, _ = image_keys(image, n_image_tokens)
    return [int(t) for t in prefix] + keys + [int(t) for t in suffix]
