"""Pins for the oracle of the sampling penalties (oracle/penalties.py).

  * hand-worked cases (tests/golden/penalties_worked.txt), two of them with
    the page's "all penalties" benchmark settings;
  * neutral settings (f = p = 0, r = 1, m = 0) leave every logit bit-exact;
  * tokens in neither the prompt, the output nor a masked stop list are
    untouched, bit-exact;
  * repetition r then 1/r gives back the logits (f = p = 0);
  * the drop of a generated token's logit is linear in its count, with slope
    f, plus p once (tokens outside the prompt, r = 1);
  * the order of the generated tokens does not matter;
  * the min_new_tokens mask holds at len(output) = m - 1 and is gone at m.
Planted mistakes (frequency counted over the prompt too, repetition
multiplying positive logits, presence scaled by the count) each fail a pin.
"""
import os

import numpy as np
import pytest

from oracle import penalties as op

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "penalties_worked.txt")


def _cases():
    cases, cur = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        if key == "case":
            cur = {"name": vals[0]}
            cases.append(cur)
        elif key == "vocab":
            cur["V"] = int(vals[0])
        elif key in ("logits", "expect"):
            cur[key] = [float(v) for v in vals]
        elif key in ("prompt", "output", "stops", "mask"):
            cur[key] = [int(v) for v in vals]
        elif key == "params":
            cur["params"] = (float(vals[0]), float(vals[1]), float(vals[2]), int(vals[3]))
    return cases


def _run(c):
    f, p, r, m = c["params"]
    return op.apply(np.array([c["logits"]]), [c["prompt"]], [c["output"]], [f], [p], [r], [m], [c["stops"]])[0]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_worked_cases(case):
    out = _run(case)
    exp = np.array(case["expect"])
    exp[case["mask"]] = -np.inf
    np.testing.assert_allclose(out, exp, rtol=0, atol=1e-12)


def _random(seed, B=6, V=300):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((B, V)) * 3
    prompts = [list(rng.integers(0, V, int(rng.integers(0, 40)))) for _ in range(B)]
    outputs = [list(rng.zipf(1.5, int(rng.integers(0, 60))) % V) for _ in range(B)]
    stops = [list(rng.integers(0, V, int(rng.integers(0, 4)))) for _ in range(B)]
    return rng, logits, prompts, outputs, stops


@pytest.mark.parametrize("seed", range(8))
def test_neutral_settings_and_untouched_tokens(seed):
    rng, x, pr, out, st = _random(seed)
    B, V = x.shape
    y = op.apply(x, pr, out, [0.0] * B, [0.0] * B, [1.0] * B, [0] * B, st)
    assert (y == x).all()
    f, p, r = rng.uniform(-2, 2, B), rng.uniform(-2, 2, B), rng.uniform(0.05, 2, B)
    m = rng.integers(0, 80, B)
    y = op.apply(x, pr, out, f, p, r, m, st)
    for b in range(B):
        touched = set(pr[b]) | set(out[b]) | (set(st[b]) if len(out[b]) < m[b] else set())
        free = [v for v in range(V) if v not in touched]
        assert (y[b, free] == x[b, free]).all()


@pytest.mark.parametrize("seed", range(8))
def test_repetition_inverse_and_linear_count(seed):
    rng, x, pr, out, st = _random(seed)
    B, V = x.shape
    r = rng.uniform(0.2, 2, B)
    zeros = [0.0] * B
    y = op.apply(x, pr, out, zeros, zeros, r, [0] * B, st)
    z = op.apply(y, pr, out, zeros, zeros, 1.0 / r, [0] * B, st)
    np.testing.assert_allclose(z, x, rtol=1e-12, atol=1e-12)
    # linear in the count, outside the prompt, r = 1
    f, p = rng.uniform(-2, 2, B), rng.uniform(-2, 2, B)
    y = op.apply(x, [[]] * B, out, f, p, [1.0] * B, [0] * B, st)
    for b in range(B):
        for v, k in zip(*np.unique(out[b], return_counts=True)):
            assert abs((x[b, v] - y[b, v]) - (f[b] * k + p[b])) <= 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_output_order_and_min_new_boundary(seed):
    rng, x, pr, out, st = _random(seed)
    B, V = x.shape
    f, p, r = rng.uniform(-2, 2, B), rng.uniform(-2, 2, B), rng.uniform(0.05, 2, B)
    shuffled = [list(rng.permutation(o)) for o in out]
    m = [len(o) for o in out]
    np.testing.assert_array_equal(op.apply(x, pr, out, f, p, r, m, st), op.apply(x, pr, shuffled, f, p, r, m, st))
    for b in range(B):
        if not st[b]:
            continue
        at = op.apply(x[b:b + 1], [pr[b]], [out[b]], [f[b]], [p[b]], [r[b]], [len(out[b]) + 1], [st[b]])[0]
        assert np.isneginf(at[st[b]]).all()
        past = op.apply(x[b:b + 1], [pr[b]], [out[b]], [f[b]], [p[b]], [r[b]], [len(out[b])], [st[b]])[0]
        assert np.isfinite(past[st[b]]).all()


def test_pins_catch_planted_mistakes(monkeypatch):
    real = op.apply

    def freq_over_prompt(logits, prompts, outputs, freq, pres, rep, min_new, stops):
        return real(logits, [[]] * len(prompts), [list(a) + list(b) for a, b in zip(prompts, outputs)],
                    freq, pres, rep, min_new, stops)

    def rep_multiplies(logits, prompts, outputs, freq, pres, rep, min_new, stops):
        return real(logits, prompts, outputs, freq, pres, [1.0 / r if r else r for r in rep], min_new, stops)

    def pres_times_count(logits, prompts, outputs, freq, pres, rep, min_new, stops):
        return real(logits, prompts, outputs, [f + p for f, p in zip(freq, pres)], [0.0] * len(pres), rep,
                    min_new, stops)

    for fn in (freq_over_prompt, rep_multiplies, pres_times_count):
        with monkeypatch.context() as m:
            m.setattr(op, "apply", fn)
            with pytest.raises(AssertionError):
                for c in _cases():
                    test_worked_cases(c)
