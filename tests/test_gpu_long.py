"""GPU parity at long contexts: one cached history of 120k tokens, extended
by two requests (one through the whole history, one branching off at 60k),
then decoded, plain and prefix-shared.  Every offset and split count here is
far beyond the benchmark batches (8k contexts): 157 splits of 768 keys per
request, about 1900 key tiles per extend workgroup, slot and row offsets
past 2^24 bytes.  Tolerances as everywhere: max-abs 1e-5 (fp32) / 2e-2
(bf16) against the float64 oracle."""
import numpy as np
import pytest
import torch

from inputs import configs
from tests import gpu_runner as G

pytestmark = pytest.mark.gpu


def long_workload(seed, L=120_000):
    rng = np.random.default_rng(seed)
    hist = [int(x) for x in rng.integers(0, 32000, L)]
    a = hist + [int(x) for x in rng.integers(0, 32000, 64)]
    b = hist[: L // 2] + [90001] + [int(x) for x in rng.integers(0, 32000, 31)]
    return [configs.Phase("setup", [hist]), configs.Phase("extend", [a, b]),
            configs.Phase("decode", [a + [90002], b + [90003], hist + [90004]])]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 4, 4, 128), ("bf16", 16, 2, 128), ("f32", 4, 2, 64)])
def test_long_context_extend_and_decode(dtype, hq, hkv, d):
    shape = configs.Shape(f"long-{dtype}-{hq}-{hkv}-{d}", hq, hkv, d, dtype, 1 << 18, 81)
    res, _ = G.run(shape, long_workload(81 + hq), content_device="cpu", sparse=True)
    assert len(res) == 2
    G.check(res, dtype, f"long context {dtype} {hq}/{hkv} d{d}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("hq,hkv", [(4, 4), (16, 2)])
def test_long_context_prefix_shared_decode(hq, hkv):
    shape = configs.Shape(f"long-cas-{hq}-{hkv}", hq, hkv, 128, "bf16", 1 << 18, 83)
    res, _ = G.run(shape, long_workload(83 + hq), select=lambda i, B: [] if i == 1 else None,
                   content_device="cpu", sparse=True, cascade={})
    G.check(res, "bf16", f"long context prefix-shared {hq}/{hkv}")
