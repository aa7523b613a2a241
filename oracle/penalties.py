"""Oracle of the batched sampling penalties, in float64.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the native library and never imports it.

What is computed.  SGLang's sampling parameters (the sampling page,
sglang-zh.llamafactory.cn, `sampling_params`, "Penalties" block) define four
penalties applied to a running request's next-token logits, and the page's
section on the performance implications of penalties says they are computed
on the GPU for the whole batch, with state of size vocab x running requests:

  * frequency_penalty f in [-2, 2]: penalizes a token by how often it occurs
    in the text generated so far (0 disables);
  * presence_penalty p in [-2, 2]: penalizes a token that occurs in the
    generated text so far (0 disables);
  * repetition_penalty r in [0, 2]: penalizes a token that occurs in the
    prompt or in the generated text (1 disables; above 1 discourages
    repeats);
  * min_new_tokens m: until the output holds m tokens, the EOS token and the
    request's stop token ids get logit -inf (0 disables).

The page states intent and ranges, not formulas.  The readings taken:

  * frequency and presence are additive: x - f * count - p * [count > 0],
    with count = occurrences of the token among the generated tokens;
  * repetition is multiplicative on the sign: x / r if x > 0 else x * r, for
    every token in the prompt or the generated tokens (r = 0 follows IEEE:
    a positive logit becomes +inf, a negative one 0);
  * order: repetition first, then the additive terms, then the
    min_new_tokens mask; a token's penalties are applied once, whatever its
    count;
  * "EOS and stop_token_ids" is one list of token ids per request, given as
    input; the mask applies while len(output) < m.

Every step below is the definition written out over the whole vocabulary, in
float64, with counts from the token lists by plain counting.
"""
from __future__ import annotations

import numpy as np


def counts_of(tokens, vocab):
    """Occurrences of every vocabulary id among `tokens`."""
    c = np.zeros(vocab, dtype=np.int64)
    for t in tokens:
        c[int(t)] += 1
    return c


def apply(logits, prompts, outputs, freq, pres, rep, min_new, stops):
    """Penalized logits.  logits [B, V] (any float type, taken exactly as
    float64); prompts, outputs, stops: per request lists of token ids; freq,
    pres, rep: per request floats; min_new: per request ints.  Returns a new
    float64 array."""
    x = np.array(logits, dtype=np.float64)
    B, V = x.shape
    for b in range(B):
        gen = counts_of(outputs[b], V)
        seen = gen > 0
        seen_or_prompt = seen | (counts_of(prompts[b], V) > 0)
        r = float(rep[b])
        row = x[b]
        with np.errstate(divide="ignore"):
            divided = row / r if r != 0 else np.full(V, np.inf)
        rep_row = np.where(row > 0, divided, row * r)
        row = np.where(seen_or_prompt, rep_row, row)
        row = row - float(freq[b]) * gen - float(pres[b]) * seen.astype(np.float64)
        if len(outputs[b]) < int(min_new[b]):
            for s in stops[b]:
                row[int(s)] = -np.inf
        x[b] = row
    return x
