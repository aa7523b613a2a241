"""GPU parity of the sampling penalties (rkv_penalty_admit / accumulate /
apply) against the float64 oracle (oracle/penalties.py), over a simulated
decode loop: requests are admitted into scattered slots with their prompts;
every step penalizes fresh seeded logits, is compared with the oracle, and
then records one seeded output token per request, on alternate steps by
rkv_penalty_accumulate and by the next rkv_penalty_apply itself.

Tolerance (derived from the arithmetic): the kernel divides once (correctly
rounded), then one fma and one subtraction in fp32, so
|gpu - oracle| <= 4 * 2^-24 * (|x| * max(r, 1/r, 1) + |f| * count + |p| + |z|)
with z the oracle's value; bf16 logits add half a bf16 ulp, 2^-8 * |z|.
Untouched logits, -inf masks and infinities must match exactly.  The state
(counts, prompt bits, the seen set, out_len) must match the token lists
exactly."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from oracle import penalties as op
from tests import gpu_runner as G

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from prefix_shared_kv_host_amd import rkv
    rkv.lib()


def _tol(x, z, f, p, r, g, dtype):
    scale = max(r, 1.0 / r, 1.0) if r > 0 else 1.0       # r = 0 gives exact 0 or inf
    t = 4 * 2.0 ** -24 * (np.abs(x) * scale + np.abs(f) * g + np.abs(p) + np.abs(z))
    if dtype == torch.bfloat16:
        t = t + 2.0 ** -8 * np.abs(z)
    return t


def _check_step(lg_before, lg_after, prompts, outputs, f, p, r, m, stops, dtype, V):
    ref = op.apply(lg_before, prompts, outputs, f, p, r, m, stops)
    got = lg_after
    B = ref.shape[0]
    for b in range(B):
        gen = op.counts_of(outputs[b], V)
        x, z, y = lg_before[b], ref[b], got[b]
        fin = np.isfinite(z)
        assert (y[~fin] == z[~fin]).all(), b                       # -inf masks, +inf from r = 0
        same = z == x
        assert (y[same & fin] == x[same & fin]).all(), b            # untouched entries bit-exact
        err = np.abs(y[fin] - z[fin])
        tol = _tol(x[fin], z[fin], f[b], p[b], r[b], gen[fin], dtype)
        assert (err <= tol).all(), (b, float(err.max()), float(tol[np.argmax(err - tol)]))
    return ref


def _check_state(st, slot_of, prompts, outputs, V):
    counts = st.counts.cpu().numpy().view(np.uint32)
    seen = st.seen.cpu().numpy()
    seen_len = st.seen_len.cpu().numpy()
    out_len = st.out_len.cpu().numpy()
    for i, s in enumerate(slot_of):
        gen = op.counts_of(outputs[i], V)
        inp = op.counts_of(prompts[i], V) > 0
        assert ((counts[s] & 0x7FFFFFFF) == gen).all()
        assert (((counts[s] >> 31) == 1) == inp).all()
        listed = seen[s, :seen_len[s]]
        assert len(set(listed.tolist())) == len(listed)
        assert set(listed.tolist()) == set(prompts[i]) | set(outputs[i])
        assert out_len[s] == len(outputs[i])


@pytest.mark.parametrize("dtype,V,B,steps", [(torch.float32, 1000, 24, 12), (torch.bfloat16, 1000, 24, 8),
                                             (torch.float32, 32000, 64, 6), (torch.float32, 1003, 16, 4)])
def test_penalty_decode_loop(dtype, V, B, steps):
    from prefix_shared_kv_host_amd import rkv
    rng = np.random.default_rng(V + B + steps)
    n_slots, cap = 3 * B, 700
    st = rkv.PenaltyState(n_slots, V, cap)
    st.counts.fill_(-1)                     # stale state must be reset by admit
    slot_of = rng.permutation(n_slots)[:B].astype(np.int32)
    prompts = []
    for i in range(B):
        n = int(rng.integers(0, 300)) if i % 5 else 0
        prompts.append([int(t) for t in rng.zipf(1.3, n) % V])
    outputs = [[] for _ in range(B)]
    f = rng.uniform(-2, 2, B).astype(np.float32)
    p = rng.uniform(-2, 2, B).astype(np.float32)
    r = rng.uniform(0, 2, B).astype(np.float32)
    r[0], r[1], f[2], p[2] = 0.0, 1.0, 0.0, 0.0                      # r = 0 (IEEE inf), r = 1, no additive terms
    m = rng.integers(0, steps + 2, B).astype(np.int32)
    stops = [[int(t) for t in rng.integers(0, V, int(rng.integers(0, 4)))] for _ in range(B)]
    stops[3] = prompts[3][:2] + [V - 1]                                # stop ids that are also prompt tokens
    dev = lambda a, dt=torch.int32: torch.as_tensor(np.asarray(a), dtype=dt).cuda()
    indptr = np.concatenate([[0], np.cumsum([len(x) for x in prompts])]).astype(np.int32)
    flat = np.concatenate([np.asarray(x, dtype=np.int32) for x in prompts]) if indptr[-1] else np.zeros(0, np.int32)
    st.admit(dev(slot_of), dev(indptr), dev(flat))
    torch.cuda.synchronize()
    _check_state(st, slot_of, prompts, outputs, V)
    sp = np.concatenate([[0], np.cumsum([len(s) for s in stops])]).astype(np.int32)
    sf = np.concatenate([np.asarray(s, dtype=np.int32) for s in stops])
    args = dict(freq=dev(f, torch.float32), pres=dev(p, torch.float32), rep=dev(r, torch.float32),
                min_new=dev(m), stop_indptr=dev(sp), stop_ids=dev(sf))
    ld = V + 37
    pending = None
    for step in range(steps):
        full = torch.randn(B, ld, generator=torch.Generator().manual_seed(step), dtype=torch.float32) * 4
        full[0, :7] = 0.0                                              # zero logits, r = 0 path
        lg = full.to(dtype).cuda()
        before = lg.float().cpu().numpy()[:, :V].astype(np.float64)
        pad_before = lg.float().cpu().numpy()[:, V:]
        if pending is not None:
            # the previous step's tokens are recorded inside this launch
            for i in range(B):
                outputs[i].append(pending[i])
            st.apply(lg, dev(slot_of), new_tokens=dev(pending), **args)
            pending = None
        else:
            st.apply(lg, dev(slot_of), **args)
        torch.cuda.synchronize()
        _check_state(st, slot_of, prompts, outputs, V)
        after = lg.float().cpu().numpy()
        assert np.array_equal(after[:, V:], pad_before, equal_nan=True)   # past vocab: untouched
        _check_step(before, after[:, :V].astype(np.float64), prompts, outputs, f, p, r, m, stops, dtype, V)
        # one output token per request: repeats of prompt and earlier output are common
        nxt = []
        for i in range(B):
            pool = prompts[i] + outputs[i]
            nxt.append(int(rng.choice(pool)) if pool and rng.random() < 0.6 else int(rng.integers(0, V)))
        if step % 2 == 0:
            st.accumulate(dev(slot_of), dev(nxt))
            for i in range(B):
                outputs[i].append(nxt[i])
            torch.cuda.synchronize()
            _check_state(st, slot_of, prompts, outputs, V)
        else:
            pending = nxt
    G.log(f"penalties {dtype} V={V} B={B}: {steps} steps checked")


_DEBUG_PENALTY_SCRIPT = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
from prefix_shared_kv_host_amd import rkv
st = rkv.PenaltyState(8, 100, 16)
i32 = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
def run(fn):
    try:
        fn(); torch.cuda.synchronize(); print("NO-ERROR")
    except rkv.RkvError as e:
        print("CODE", e.code)
run(lambda: st.admit(i32([1]), i32([0, 3]), i32([5, 100, 7])))         # prompt token past the vocabulary
run(lambda: st.accumulate(i32([1, 9]), i32([3, 4])))                  # slot past n_slots
run(lambda: st.admit(i32([2]), i32([0, 20]), i32(list(range(20)))))    # 20 distinct tokens, cap 16
lg = torch.zeros(1, 100, device="cuda")
f = torch.zeros(1, device="cuda")
run(lambda: st.apply(lg, i32([1]), f, f, f + 1, i32([5]), i32([0, 1]), i32([250])))   # stop id past the vocabulary
run(lambda: st.apply(lg, i32([1]), f, f, f + 1, i32([5]), i32([0, 1]), i32([50])))
print("CLEAN-OK")
"""


def test_debug_mode_flags_penalty_indices():
    """A prompt token or a stop id past the vocabulary, a slot past n_slots
    and a full seen list are skipped and reported (RKV_EINVAL under
    RKV_DEBUG=1); a valid call then runs clean."""
    env = dict(os.environ, RKV_DEBUG="1")
    p = subprocess.run([sys.executable, "-c", _DEBUG_PENALTY_SCRIPT, ROOT], env=env, capture_output=True,
                       text=True, timeout=180)
    G.log(p.stdout + p.stderr[-2000:])
    assert p.stdout.split() == ["CODE", "-1"] * 4 + ["NO-ERROR", "CLEAN-OK"], p.stdout + p.stderr[-2000:]
