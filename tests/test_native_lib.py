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
