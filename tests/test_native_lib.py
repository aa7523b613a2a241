"""The C-ABI library loads and exports every symbol include/rkv.h declares;
host-side argument checks.  CPU only (no device calls)."""
import ctypes
import os
import re

import pytest

from prefix_shared_kv_host_amd import rkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    with open(os.path.join(ROOT, "include", "rkv.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rkv_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = rkv.lib()
    decl = declared_symbols()
    assert len(decl) >= 20
    for name in decl:
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value
    assert sorted(rkv.EXPORTS) == decl
    assert rkv.version().startswith("rkv")


def test_host_argument_errors():
    with pytest.raises(rkv.RkvError) as e:
        rkv.Tree(0)
    assert e.value.code == rkv.EINVAL
    with pytest.raises(rkv.RkvError):
        rkv.Tree(4, [0, 1, 1, 3])          # not a permutation
    t = rkv.Tree(8)
    assert t.alloc(9)[0] == rkv.ENOSPC
    assert t.radix_unlock(5) == rkv.EINVAL
    assert t.free([8]) == rkv.EINVAL       # out of range
    assert t.free([0]) == rkv.EINVAL       # FIFO already holds every slot
    code, _ = t.alloc(2)
    assert t.radix_insert([1, 2], [0, 99]) == rkv.EINVAL
    with pytest.raises(rkv.RkvError):
        t.batch_prepare([[1, 2], []])
    L = rkv.lib()
    assert L.rkv_attn_decode_workspace_bytes(4, 8, 96, 100, 0) == 0   # unsupported D
    # B * Hq * splits(1024 keys / 256 per split) * (D + 4) floats
    assert L.rkv_attn_decode_workspace_bytes(4, 8, 128, 1024, 0) == 4 * 8 * 2 * 132 * 4   # 768-key chunks
    assert L.rkv_attn_decode_workspace_bytes(4, 8, 128, 1024, 3) == 4 * 8 * 3 * 132 * 4


def test_extend_rejects_rows_beyond_the_division_bound():
    """rkv_attn_extend divides row numbers by Hq/Hkv with a multiply-high,
    exact below 2^28 rows per request: larger batches are refused on the
    host, before any device call (dummy pointers are never touched)."""
    L = rkv.lib()
    p = 16  # any non-null value: the call returns before dereferencing
    args = lambda max_new, hq, hkv: (p, p, p, p, None, p, 4096, p, p, None, 2, 2 * max_new, max_new,
                                     hq, hkv, 128, 0.088, rkv.BF16, 1 << 20, None)
    assert L.rkv_attn_extend(*args(1 << 25, 8, 1)) == rkv.ENOTSUP      # 2^25 tokens x 8 heads = 2^28 rows
    assert L.rkv_attn_extend(*args(1 << 28, 1, 1)) == rkv.ENOTSUP
    assert L.rkv_attn_extend(*args(1 << 27, 3, 1)) == rkv.ENOTSUP      # 3 * 2^27 >= 2^28
    assert L.rkv_attn_extend(*args(1 << 24, 17, 1)) == rkv.ENOTSUP     # Hq/Hkv above 16
