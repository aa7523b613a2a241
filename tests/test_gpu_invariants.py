"""GPU invariants of the attention kernels (through the C ABI):

  * bit-exact under a permutation of slot placement (same data at other
    slots gives identical output bits);
  * bit-exact batch-composition invariance (a request's output does not
    depend on the rest of its batch);
  * decode output independent of num_splits within tolerance;
  * extend with one new token per request equals decode within tolerance;
  * debug mode turns an out-of-range slot into RKV_EINVAL (the kernels clamp
    it, so nothing is read out of bounds).
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from inputs import configs, content
from tests import gpu_runner as G

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_cache(shape, phases, perm, kind_num_splits=0, subset=None):
    """Runs phases through a RadixKVCache with the given free-list order;
    returns the outputs (o, lse) of the last phase (optionally on a subset of
    its requests)."""
    from prefix_shared_kv_host_amd.engine import RadixKVCache
    dt = content.torch_dtype(shape.dtype)
    cache = RadixKVCache(shape.pool, shape.hkv, shape.d, dt, "cuda", perm)
    out = None
    for i, ph in enumerate(phases):
        seqs = ph.seqs if (subset is None or i < len(phases) - 1) else [ph.seqs[r] for r in subset]
        b = cache.prepare(seqs)
        last = i == len(phases) - 1
        q, k, v = content.batch_rows(shape.seed, seqs, b.host["prefix_lens"], shape.hq, shape.hkv, shape.d,
                                     dt, "cpu", shape.q_scale, with_q=last)
        cache.store(b, k.cuda(), v.cuda())
        if last:
            lse = torch.empty(q.shape[0], shape.hq, device="cuda")
            if ph.kind == "extend":
                o = cache.extend(b, q.cuda(), lse=lse)
            else:
                o = cache.decode(b, q.cuda(), lse=lse, num_splits=kind_num_splits)
            torch.cuda.synchronize()
            out = (o.cpu(), lse.cpu(), b.host)
        cache.commit(b)
    return out


def _decode_phases(lengths, seed=9):
    from tests.test_gpu_parity import decode_workload
    shape = configs.Shape("inv-dec", 8, 2, 128, "bf16", 8192, seed)
    return shape, decode_workload(shape, lengths, seed=seed)


@pytest.mark.parametrize("kind", ["extend", "decode"])
def test_bit_exact_under_slot_permutation(kind):
    if kind == "extend":
        shape, phases = configs.tiny(61, hq=8, hkv=2, d=128, dtype="bf16", pool=4096, prefix=100,
                                     new=(1, 70, 129, 5, 64))
    else:
        shape, phases = _decode_phases([1, 70, 600, 1300, 513])
    rng = np.random.default_rng(1)
    a = _run_cache(shape, phases, rng.permutation(shape.pool).astype(np.int32))
    b = _run_cache(shape, phases, rng.permutation(shape.pool).astype(np.int32))
    assert not np.array_equal(a[2]["req_to_token"], b[2]["req_to_token"])   # really moved
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


@pytest.mark.parametrize("kind", ["extend", "decode"])
def test_bit_exact_batch_composition(kind):
    if kind == "extend":
        shape, phases = configs.tiny(62, hq=8, hkv=2, d=128, dtype="bf16", pool=4096, prefix=100,
                                     new=(1, 70, 129, 5, 64))
    else:
        shape, phases = _decode_phases([1, 70, 600, 1300, 513])
    perm = np.random.default_rng(2).permutation(shape.pool).astype(np.int32)
    full = _run_cache(shape, phases, perm)
    for subset in ([2], [4, 0], [1, 3]):
        part = _run_cache(shape, phases, perm, subset=subset)
        qo_f, qo_p = full[2]["qo_indptr"], part[2]["qo_indptr"]
        for j, r in enumerate(subset):
            fo = full[0][qo_f[r]:qo_f[r + 1]]
            po = part[0][qo_p[j]:qo_p[j + 1]]
            assert torch.equal(fo.view(torch.int16), po.view(torch.int16)), (kind, subset, r)


def test_decode_independent_of_num_splits():
    shape, phases = _decode_phases([1, 2, 511, 512, 513, 1500, 2048, 777])
    perm = np.random.default_rng(3).permutation(shape.pool).astype(np.int32)
    ref = _run_cache(shape, phases, perm, kind_num_splits=1)
    for ns in (0, 2, 3, 7, 16):
        o = _run_cache(shape, phases, perm, kind_num_splits=ns)
        err = (o[0].float() - ref[0].float()).abs().max().item()
        lerr = (o[1] - ref[1]).abs().max().item()
        G.log(f"num_splits {ns}: max |o - o(1 split)| = {err:.3e}, lse {lerr:.3e}")
        # this shape (8 q heads per 2 kv heads) takes the matrix-core path,
        # whose lse sums bf16-rounded weights: bound ln(1 + 2^-8)
        assert err <= 2e-2 and lerr <= 3.9e-3


def test_extend_with_one_token_equals_decode():
    shape, phases = _decode_phases([1, 70, 600, 1300, 513, 64])
    perm = np.random.default_rng(4).permutation(shape.pool).astype(np.int32)
    dec = _run_cache(shape, phases, perm)
    ext_phases = [phases[0], configs.Phase("extend", phases[1].seqs)]
    ext = _run_cache(shape, ext_phases, perm)
    assert ext[2]["qo_indptr"].tolist() == list(range(len(phases[1].seqs) + 1))
    err = (ext[0].float() - dec[0].float()).abs().max().item()
    G.log(f"extend(n=1) vs decode: max abs {err:.3e}")
    assert err <= 2e-2


_DEBUG_SCRIPT = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
from prefix_shared_kv_host_amd import rkv
P, hkv, d = 64, 2, 128
kp = torch.zeros(P, hkv, d, dtype=torch.bfloat16, device="cuda")
vp = torch.zeros_like(kp)
q = torch.zeros(2, 4, d, dtype=torch.bfloat16, device="cuda")
o = torch.empty_like(q)
r2t = torch.tensor([[0, 1, 2, 3], [4, 5, 10**6, 7]], dtype=torch.int32, device="cuda")  # one bad slot
sl = torch.tensor([4, 4], dtype=torch.int32, device="cuda")
ws = torch.empty(rkv.attn_decode_workspace_bytes(2, 4, d, 4) // 4 + 1, device="cuda")
try:
    rkv.attn_decode(q, kp, vp, o, r2t, sl, 4, ws)
    print("NO-ERROR")
except rkv.RkvError as e:
    print("CODE", e.code)
r2t_ok = torch.tensor([[0, 1, 2, 3], [4, 5, 6, 7]], dtype=torch.int32, device="cuda")
rkv.attn_decode(q, kp, vp, o, r2t_ok, sl, 4, ws)
print("CLEAN-OK")
"""


_DEBUG_EXTEND_SCRIPT = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
from prefix_shared_kv_host_amd import rkv
P, hkv, d, hq = 512, 2, 128, 8
kp = torch.zeros(P, hkv, d, dtype=torch.bfloat16, device="cuda")
vp = torch.zeros_like(kp)
# two requests: 200 cached + 70 new, 0 cached + 5 new; one bad slot deep in
# the first request's prefix (a later tile, reached through the gathers)
pl = torch.tensor([200, 0], dtype=torch.int32, device="cuda")
qo = torch.tensor([0, 70, 75], dtype=torch.int32, device="cuda")
r2t = torch.arange(2 * 270, dtype=torch.int32).view(2, 270) % P
bad = r2t.clone(); bad[0, 130] = 10**6
q = torch.zeros(75, hq, d, dtype=torch.bfloat16, device="cuda")
o = torch.empty_like(q)
try:
    rkv.attn_extend(q, kp, vp, o, bad.cuda(), qo, pl, max_new=70)
    print("NO-ERROR")
except rkv.RkvError as e:
    print("CODE", e.code)
rkv.attn_extend(q, kp, vp, o, r2t.cuda(), qo, pl, max_new=70)
torch.cuda.synchronize()
print("CLEAN-OK")
"""


_DEBUG_CASCADE_SCRIPT = r"""
import sys, numpy as np, torch
sys.path.insert(0, sys.argv[1])
from prefix_shared_kv_host_amd import rkv
P, hkv, d, hq = 256, 2, 128, 2
kp = torch.zeros(P, hkv, d, dtype=torch.bfloat16, device="cuda")
vp = torch.zeros_like(kp)
# three requests share slots 0..39, then private tails
L = np.array([60, 55, 70], dtype=np.int32)
r2t = np.full((3, 80), -1, dtype=np.int32)
nxt = 40
for r in range(3):
    r2t[r, :40] = np.arange(40)
    r2t[r, 40:L[r]] = np.arange(nxt, nxt + L[r] - 40); nxt += L[r] - 40
q = torch.zeros(3, hq, d, dtype=torch.bfloat16, device="cuda")
o = torch.empty_like(q)
sl = torch.from_numpy(L).cuda()

def run(table, plan):
    plan.to("cuda")
    ws = torch.empty(rkv.attn_decode_cascade_workspace_bytes(plan.n_records, hq, d) // 4 + 1, device="cuda")
    try:
        rkv.attn_decode_cascade(q, kp, vp, o, torch.from_numpy(table).cuda(), sl, 80, plan, ws)
        torch.cuda.synchronize()
        print("NO-ERROR")
    except rkv.RkvError as e:
        print("CODE", e.code)

base = rkv.cascade_plan(r2t, L, 16, 32, 8, 8)
assert base.n_jobs >= 1
bad_slot = r2t.copy(); bad_slot[:, 20] = 10**6          # inside the shared run (every row)
run(bad_slot, base)
p = rkv.cascade_plan(r2t, L, 16, 32, 8, 8); p.jobs[0, 2] = 2; p.jobs[0, 3] = 2   # members past B
run(r2t, p)
p = rkv.cascade_plan(r2t, L, 16, 32, 8, 8); p.jobs[0, 4] = 100                 # record past the request's
run(r2t, p)
p = rkv.cascade_plan(r2t, L, 16, 32, 8, 8); p.tail_begin[2] = 70               # empty tail
run(r2t, p)
run(r2t, rkv.cascade_plan(r2t, L, 16, 32, 8, 8))
print("CLEAN-OK")
"""


@pytest.mark.parametrize("script", [_DEBUG_SCRIPT, _DEBUG_EXTEND_SCRIPT], ids=["decode", "extend"])
def test_debug_mode_flags_out_of_range_slot(script):
    env = dict(os.environ, RKV_DEBUG="1")
    p = subprocess.run([sys.executable, "-c", script, ROOT], env=env, capture_output=True,
                       text=True, timeout=180)
    G.log(p.stdout + p.stderr[-2000:])
    assert "CODE -1" in p.stdout and "CLEAN-OK" in p.stdout


def test_debug_mode_flags_cascade_plan_that_does_not_fit():
    """An out-of-range slot in a shared run, a job whose members run past the
    batch, a record past the request's range and an empty tail are each
    caught by the kernels' checks (RKV_EINVAL under RKV_DEBUG=1, nothing
    indexed out of range); the unmodified plan then runs clean."""
    env = dict(os.environ, RKV_DEBUG="1")
    p = subprocess.run([sys.executable, "-c", _DEBUG_CASCADE_SCRIPT, ROOT], env=env, capture_output=True,
                       text=True, timeout=180)
    G.log(p.stdout + p.stderr[-2000:])
    assert p.stdout.split() == ["CODE", "-1"] * 4 + ["NO-ERROR", "CLEAN-OK"], p.stdout + p.stderr[-2000:]
