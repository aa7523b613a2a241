"""Request token sequences for multimodal inputs.

The runtime hashes each input image and uses the hash as the radix key, so
requests with the same image reuse the KV of its tokens (unite.ai, "SGLang:
Efficient Execution of Structured Language Model Programs", section
"Resultados en modelos multimodales").  An image occupying n positions
becomes the n keys of rkv_image_keys (content hash -> int32 keys disjoint
from text ids); the tree, the tables and the kernels then treat them like
tokens.  This module only assembles sequences; the keys come from librkv.
"""
from __future__ import annotations

from . import rkv


def request_tokens(prefix, image: bytes, n_image_tokens: int, suffix):
    """prefix text ids, then the image's keys, then suffix text ids."""
    keys, _ = rkv.image_keys(image, n_image_tokens)
    return [int(t) for t in prefix] + keys.tolist() + [int(t) for t in suffix]


def trace_batches(trace, n_image_tokens: int):
    """The batches of an inputs.configs.mm_trace as token sequences."""
    sys_tokens, blobs, batches = trace
    keys = [rkv.image_keys(b, n_image_tokens)[0].tolist() for b in blobs]
    return [[list(sys_tokens) + keys[img] + list(q) for img, q in batch] for batch in batches]
