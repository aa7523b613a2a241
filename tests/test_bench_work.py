"""The work counts bench.py divides by (CPU): extend flop, decode and scatter
bytes, each against a count made element by element on small batches, and
the guard that drops a recorded traffic figure once the kernel sources it was
measured on have changed."""
import hashlib
import json
import os

import numpy as np

import bench


def test_extend_flops_counts_visible_pairs():
    """4 * D * Hq flop (a multiply-add each in QK^T and PV) per causal
    (query, key) pair: query i of a request with p cached tokens sees keys
    0 .. p + i."""
    rng = np.random.default_rng(3)
    for _ in range(5):
        B = int(rng.integers(1, 7))
        p = rng.integers(0, 40, B)
        n = rng.integers(1, 30, B)
        hq, d = int(rng.choice([1, 4, 32])), int(rng.choice([64, 128]))
        pairs = 0
        for r in range(B):
            for i in range(int(n[r])):
                pairs += sum(1 for j in range(int(p[r] + n[r])) if j <= p[r] + i)
        assert bench.extend_flops(p, p + n, hq, d) == 4.0 * d * hq * pairs


def test_decode_bytes_counts_rows_indices_q_and_o():
    """Every key of a request brings its K and V rows of all kv heads and a
    4-byte slot index; each request's q and o rows are read and written
    once.  With unique_slots the K/V rows are counted once per slot."""
    rng = np.random.default_rng(4)
    L = rng.integers(1, 50, 6)
    hq, hkv, d, b = 8, 2, 128, 2
    total = 0
    for r in range(len(L)):
        for _ in range(int(L[r])):
            total += 2 * hkv * d * b + 4
        total += 2 * hq * d * b
    assert bench.decode_bytes(L, hq, hkv, d, b) == total
    slots = [set(rng.integers(0, 60, int(x)).tolist()) for x in L]
    uniq = len(set().union(*slots))
    expect = uniq * 2 * hkv * d * b + 4 * int(L.sum()) + 2 * len(L) * hq * d * b
    assert bench.decode_bytes(L, hq, hkv, d, b, unique_slots=uniq) == expect


def test_scatter_bytes_reads_and_writes_each_row_once():
    T, hkv, d, b = 37, 4, 64, 2
    assert bench.scatter_bytes(T, hkv, d, b) == T * (2 * 2 * hkv * d * b + 4)


def test_recorded_traffic_is_dropped_when_sources_change(tmp_path, monkeypatch):
    """The figure is returned only while the listed sources hash to the
    recorded digest."""
    src = tmp_path / "kernel.hip"
    src.write_text("// a kernel\n")
    digest = hashlib.sha256(src.read_bytes()).hexdigest()
    (tmp_path / "profiles").mkdir()
    rec = {"kernels": {"k": {"sources": ["kernel.hip"], "sources_sha256": digest, "bytes_per_launch": 1.5e9}}}
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("k") == 1.5e9
    assert bench.measured_traffic("other") is None
    src.write_text("// a kernel, edited\n")
    assert bench.measured_traffic("k") is None
    os.remove(src)
    assert bench.measured_traffic("k") is None
