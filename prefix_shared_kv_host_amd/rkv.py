"""ctypes binding of librkv (include/rkv.h).  Argument marshalling only: every
step of the path runs in the native library.

Names follow the C ABI without the `rkv_` prefix.  Device entry points take
torch tensors (torch provides device memory and the current HIP stream) and
pass their raw pointers; host tree calls take Python sequences or NumPy
arrays.  Errors raise RkvError carrying the status code and the library's
message.
"""
from __future__ import annotations

import ctypes
import itertools
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# RKV_LIB may point at another build of the same library (for A/B timing)
LIB_PATH = os.environ.get("RKV_LIB") or os.path.join(_HERE, "librkv.so")

OK, EINVAL, ENOSPC, EBUSY, EHIP, ENOTSUP = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1
_NAMES = {EINVAL: "EINVAL", ENOSPC: "ENOSPC", EBUSY: "EBUSY", EHIP: "EHIP", ENOTSUP: "ENOTSUP"}

# every symbol include/rkv.h declares
EXPORTS = (
    "rkv_last_error", "rkv_version", "rkv_tree_create", "rkv_tree_destroy", "rkv_radix_match",
    "rkv_radix_lock", "rkv_radix_unlock", "rkv_radix_insert", "rkv_radix_evict", "rkv_alloc",
    "rkv_free", "rkv_stats", "rkv_radix_serialize", "rkv_free_list", "rkv_batch_prepare",
    "rkv_batch_commit", "rkv_kv_scatter", "rkv_attn_extend", "rkv_attn_decode_workspace_bytes",
    "rkv_attn_decode", "rkv_radix_peek", "rkv_schedule", "rkv_cascade_plan",
    "rkv_attn_decode_cascade_workspace_bytes", "rkv_attn_decode_cascade", "rkv_penalty_admit",
    "rkv_penalty_accumulate", "rkv_penalty_apply", "rkv_image_keys", "rkv_batch_append",
    "rkv_table_append", "rkv_attn_decode_noalloc",
)

# the scratch that rkv_attn_decode_noalloc holds per GPU (include/rkv.h)
DECODE_NOALLOC_MAX_BYTES = 32 << 20


class TokenBatch:
    """Token ids of a batch as one int32 array with int64 offsets (request r
    is flat[indptr[r]:indptr[r+1]]); the tree calls take it in place of a
    list of sequences, so a batch is converted once for prepare and commit."""

    def __init__(self, seqs):
        self.lens = np.array([len(x) for x in seqs], dtype=np.int64)
        self.indptr = np.zeros(len(self.lens) + 1, dtype=np.int64)
        np.cumsum(self.lens, out=self.indptr[1:])
        total = int(self.indptr[-1])
        self.flat = np.fromiter(itertools.chain.from_iterable(seqs), dtype=np.int32, count=total) \
            if total else np.zeros(0, dtype=np.int32)
        # data addresses, taken once: prepare and commit pass them as they are
        self.ptrs = (self.flat.ctypes.data, self.indptr.ctypes.data)

    def __len__(self):
        return len(self.lens)


class RkvError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{_NAMES.get(code, code)}: {msg}")
        self.code = code


_lib = None

c_i32p = ctypes.POINTER(ctypes.c_int32)
c_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p
_i32, _i64, _f32, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


def lib():
    """Loads librkv.so; raises (never falls back) when it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m prefix_shared_kv_host_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "rkv_last_error": (ctypes.c_char_p, []),
        "rkv_version": (ctypes.c_char_p, []),
        "rkv_tree_create": (ctypes.c_int, [ctypes.POINTER(_vp), _i64, c_i32p]),
        "rkv_tree_destroy": (None, [_vp]),
        "rkv_radix_match": (ctypes.c_int, [_vp, c_i32p, _i64, c_i32p, c_i64p, c_i64p]),
        "rkv_radix_peek": (ctypes.c_int, [_vp, c_i32p, _i64, c_i64p]),
        "rkv_schedule": (ctypes.c_int, [_vp, _i32, c_i32p, c_i64p, c_i32p, c_i64p]),
        "rkv_radix_lock": (ctypes.c_int, [_vp, _i64]),
        "rkv_radix_unlock": (ctypes.c_int, [_vp, _i64]),
        "rkv_radix_insert": (ctypes.c_int, [_vp, c_i32p, c_i32p, _i64, c_i64p]),
        "rkv_radix_evict": (ctypes.c_int, [_vp, _i64, c_i64p]),
        "rkv_alloc": (ctypes.c_int, [_vp, _i64, c_i32p]),
        "rkv_free": (ctypes.c_int, [_vp, c_i32p, _i64]),
        "rkv_stats": (ctypes.c_int, [_vp, c_i64p]),
        "rkv_radix_serialize": (ctypes.c_int, [_vp, c_i64p, _i64, c_i64p]),
        "rkv_free_list": (ctypes.c_int, [_vp, c_i32p, _i64, c_i64p]),
        # the batch calls take integer addresses (marshalling typed pointers
        # costs microseconds per argument, per batch)
        "rkv_batch_prepare": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _vp]),
        "rkv_batch_commit": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _i64, _vp]),
        "rkv_batch_append": (ctypes.c_int, [_vp, _i32, _vp, _i64, _vp, _vp]),
        "rkv_table_append": (ctypes.c_int, [_vp, _i64, _vp, _vp, _i32, _vp]),
        "rkv_kv_scatter": (ctypes.c_int, [_vp, _vp, _vp, _i64, _vp, _vp, _i64, _i32, _i32, _i32, _vp]),
        "rkv_attn_extend": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _i32, _i64, _i32,
                                           _i32, _i32, _i32, _f32, _i32, _i64, _vp]),
        "rkv_attn_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
        "rkv_attn_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i32, _i32, _i32, _i32,
                                           _i32, _f32, _i32, _i32, _vp, _sz, _i64, _vp]),
        "rkv_attn_decode_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i32, _i32, _i32,
                                                   _i32, _i32, _f32, _i32, _i32, _i64, _vp]),
        "rkv_cascade_plan": (ctypes.c_int, [c_i32p, _i64, c_i32p, _i32, _i32, _i32, _i32, _i32, c_i32p,
                                            c_i32p, c_i32p, c_i32p, _i64, c_i64p, c_i32p]),
        "rkv_attn_decode_cascade_workspace_bytes": (_sz, [_i64, _i32, _i32]),
        "rkv_attn_decode_cascade": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i32, _i32, _i32,
                                                   _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp, _i64, _vp,
                                                   _i32, _i32, _i32, _i64, _vp, _sz, _i64, _vp]),
        "rkv_image_keys": (ctypes.c_int, [ctypes.c_char_p, _i64, _i64, c_i32p, ctypes.POINTER(ctypes.c_uint64)]),
        "rkv_penalty_admit": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
        "rkv_penalty_accumulate": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
        "rkv_penalty_apply": (ctypes.c_int, [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp,
                                             _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(code):
    if code != OK:
        raise RkvError(code, lib().rkv_last_error().decode())
    return code


def version() -> str:
    return lib().rkv_version().decode()


def _i32arr(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return a, a.ctypes.data_as(c_i32p)


class Tree:
    """Radix tree + FIFO slot allocator (host).  Methods mirror rkv_radix_*,
    rkv_alloc/free, rkv_batch_*; status codes other than OK raise RkvError
    unless the method documents returning them."""

    def __init__(self, pool_slots: int, initial_free=None):
        self._h = _vp()
        self.pool_slots = int(pool_slots)
        if initial_free is None:
            _check(lib().rkv_tree_create(ctypes.byref(self._h), self.pool_slots, None))
        else:
            a, p = _i32arr(initial_free)
            if a.shape[0] != self.pool_slots:
                raise RkvError(EINVAL, "initial_free must have pool_slots entries")
            _check(lib().rkv_tree_create(ctypes.byref(self._h), self.pool_slots, p))

    def close(self):
        if self._h:
            lib().rkv_tree_destroy(self._h)
            self._h = _vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- single operations -------------------------------------------------
    def radix_match(self, tok):
        a, p = _i32arr(tok)
        out = np.empty(max(1, a.shape[0]), dtype=np.int32)
        m, node = _i64(), _i64()
        _check(lib().rkv_radix_match(self._h, p, a.shape[0], out.ctypes.data_as(c_i32p),
                                     ctypes.byref(m), ctypes.byref(node)))
        return m.value, out[: m.value].tolist(), node.value

    def radix_peek(self, tok) -> int:
        """Longest cached prefix length of tok, with no side effect on the tree."""
        a, p = _i32arr(tok)
        m = _i64()
        _check(lib().rkv_radix_peek(self._h, p, a.shape[0], ctypes.byref(m)))
        return m.value

    def schedule(self, seqs):
        """Cache-aware order of a waiting queue: (order, matched) as NumPy
        arrays; order = queue positions by matched prefix, longest first, ties
        in queue order."""
        Q = len(seqs)
        flat, indptr, _ = self._flat(seqs)
        order = np.empty(max(Q, 1), dtype=np.int32)
        matched = np.empty(max(Q, 1), dtype=np.int64)
        _check(lib().rkv_schedule(self._h, Q, flat.ctypes.data_as(c_i32p), indptr.ctypes.data_as(c_i64p),
                                  order.ctypes.data_as(c_i32p), matched.ctypes.data_as(c_i64p)))
        return order[:Q], matched[:Q]

    def radix_lock(self, node) -> int:
        return lib().rkv_radix_lock(self._h, int(node))

    def radix_unlock(self, node) -> int:
        return lib().rkv_radix_unlock(self._h, int(node))

    def radix_insert(self, tok, slots) -> int:
        a, p = _i32arr(tok)
        b, q = _i32arr(slots)
        if a.shape[0] != b.shape[0]:
            return EINVAL
        out = _i64()
        code = lib().rkv_radix_insert(self._h, p, q, a.shape[0], ctypes.byref(out))
        return out.value if code == OK else code

    def radix_evict(self, want):
        """Returns (status, freed); EBUSY is returned, not raised."""
        out = _i64()
        code = lib().rkv_radix_evict(self._h, int(want), ctypes.byref(out))
        if code not in (OK, EBUSY):
            _check(code)
        return code, out.value

    def alloc(self, n):
        """Returns (status, slots); ENOSPC is returned, not raised."""
        out = np.empty(max(1, int(n)), dtype=np.int32)
        code = lib().rkv_alloc(self._h, int(n), out.ctypes.data_as(c_i32p))
        if code not in (OK, ENOSPC):
            _check(code)
        return code, (out[: int(n)].tolist() if code == OK else [])

    def free(self, slots) -> int:
        a, p = _i32arr(slots)
        return lib().rkv_free(self._h, p, a.shape[0])

    def stats(self):
        out = np.zeros(8, dtype=np.int64)
        _check(lib().rkv_stats(self._h, out.ctypes.data_as(c_i64p)))
        return out.tolist()

    def radix_serialize(self):
        n = _i64()
        _check(lib().rkv_radix_serialize(self._h, None, 0, ctypes.byref(n)))
        buf = np.empty(n.value, dtype=np.int64)
        _check(lib().rkv_radix_serialize(self._h, buf.ctypes.data_as(c_i64p), n.value, ctypes.byref(n)))
        return buf.tolist()

    def free_list(self):
        n = _i64()
        _check(lib().rkv_free_list(self._h, None, 0, ctypes.byref(n)))
        buf = np.empty(max(1, n.value), dtype=np.int32)
        _check(lib().rkv_free_list(self._h, buf.ctypes.data_as(c_i32p), n.value, ctypes.byref(n)))
        return buf[: n.value].tolist()

    # -- batches ------------------------------------------------------------
    @staticmethod
    def _flat(seqs):
        if isinstance(seqs, TokenBatch):
            return seqs.flat, seqs.indptr, seqs.lens
        lens = np.array([len(s) for s in seqs], dtype=np.int64)
        indptr = np.zeros(len(seqs) + 1, dtype=np.int64)
        np.cumsum(lens, out=indptr[1:])
        flat = (np.concatenate([np.asarray(s, dtype=np.int32) for s in seqs])
                if len(seqs) else np.zeros(0, dtype=np.int32))
        return np.ascontiguousarray(flat, dtype=np.int32), indptr, lens

    @staticmethod
    def table_layout(B, ld, cap):
        """Word offsets of the int32 tables of a B-request batch in one
        buffer (batch_prepare's `out`): (req_to_token [B*ld], prefix_lens [B],
        seq_lens [B], qo_indptr [B+1], new_slots [cap], end).  B and cap are
        taken as at least 1."""
        Bx, cx = max(B, 1), max(cap, 1)
        o1 = Bx * ld
        return 0, o1, o1 + Bx, o1 + 2 * Bx, o1 + 3 * Bx + 1, o1 + 3 * Bx + 1 + cx

    @staticmethod
    def table_words(B, ld, cap):
        """int32 words of one buffer holding a batch's tables."""
        return Tree.table_layout(B, ld, cap)[-1]

    def batch_prepare(self, seqs, ld=None, out=None):
        """Returns (status, tables); tables hold NumPy arrays req_to_token
        [B, ld], prefix_lens, seq_lens, qo_indptr [B+1], new_slots [T] and
        nodes.  EBUSY is returned, not raised.  out: an optional contiguous
        int32 array of at least table_words(B, ld, sum of lengths) words;
        the int32 tables are then views of it, in the order table_words
        lists (so one copy moves them all)."""
        B = len(seqs)
        if not isinstance(seqs, TokenBatch):
            seqs = TokenBatch(seqs)
        lens = seqs.lens
        pf, pi = seqs.ptrs
        if ld is None:
            ld = int(lens.max()) if B else 1
        Bx = max(B, 1)
        cap = int(lens.sum())
        _, o1, o2, o3, o5, need = self.table_layout(B, ld, cap)
        if out is None:
            buf = np.empty(need, dtype=np.int32)
        else:
            if out.dtype != np.int32 or out.ndim != 1 or out.shape[0] < need or not out.flags.c_contiguous:
                raise RkvError(EINVAL, "batch_prepare: out must be a contiguous int32 array of table_words words")
            buf = out
        r2t, pl, sl = buf[:o1].reshape(Bx, ld), buf[o1:o2], buf[o2:o3]
        qo, ns = buf[o3:o5], buf[o5:need]
        qo[0] = 0
        nodes = np.empty(Bx, dtype=np.int64)
        base = buf.ctypes.data
        code = lib().rkv_batch_prepare(self._h, B, pf, pi, base, int(ld), base + 4 * o1, base + 4 * o2,
                                       base + 4 * o3, base + 4 * o5, cap, nodes.ctypes.data)
        if code == EBUSY:
            return code, None
        _check(code)
        T = int(qo[B])
        return OK, dict(req_to_token=r2t[:B], prefix_lens=pl[:B], seq_lens=sl[:B], qo_indptr=qo[:B + 1],
                        new_slots=ns[:T], nodes=nodes[:B], ld=int(ld))

    def batch_commit(self, seqs, req_to_token, nodes) -> int:
        B = len(seqs)
        if not isinstance(seqs, TokenBatch):
            seqs = TokenBatch(seqs)
        pf, pi = seqs.ptrs
        r2t = req_to_token if (isinstance(req_to_token, np.ndarray) and req_to_token.dtype == np.int32
                               and req_to_token.flags.c_contiguous) \
            else np.ascontiguousarray(np.asarray(req_to_token, dtype=np.int32))
        nd = nodes if (isinstance(nodes, np.ndarray) and nodes.dtype == np.int64 and nodes.flags.c_contiguous) \
            else np.ascontiguousarray(np.asarray(nodes, dtype=np.int64))
        ld = r2t.shape[1] if r2t.ndim == 2 and B else 1
        return _check(lib().rkv_batch_commit(self._h, B, pf, pi, r2t.ctypes.data, int(ld), nd.ctypes.data))

    def batch_append(self, req_to_token, seq_lens, out=None):
        """Decode continuation (rkv_batch_append): one new slot per request
        of a prepared, uncommitted batch, written into the host tables
        req_to_token [B, ld] and seq_lens [B] in place (contiguous int32
        arrays, e.g. the views batch_prepare returned).  Returns (status,
        new_slots [B]); EBUSY is returned, not raised."""
        for a in (req_to_token, seq_lens):
            if not (isinstance(a, np.ndarray) and a.dtype == np.int32 and a.flags.c_contiguous):
                raise RkvError(EINVAL, "batch_append: tables must be contiguous int32 arrays")
        B = int(seq_lens.shape[0])
        if req_to_token.ndim != 2 or req_to_token.shape[0] != B:
            raise RkvError(EINVAL, "batch_append: req_to_token must be [B, ld]")
        ns = np.empty(max(B, 1), dtype=np.int32) if out is None else out
        if ns.dtype != np.int32 or ns.shape[0] < B or not ns.flags.c_contiguous:
            raise RkvError(EINVAL, "batch_append: out must be a contiguous int32 array of B entries")
        code = lib().rkv_batch_append(self._h, B, req_to_token.ctypes.data, int(req_to_token.shape[1]),
                                      seq_lens.ctypes.data, ns.ctypes.data)
        if code == EBUSY:
            return code, None
        _check(code)
        return OK, ns[:B]


# ---------------------------------------------------------------------------
# device entry points (torch tensors in, pointers out)

def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise RkvError(ENOTSUP, f"unsupported dtype {t.dtype}")


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise RkvError(EINVAL, "device entry points take GPU tensors")
        if t is not None and not t.is_contiguous():
            raise RkvError(EINVAL, "tensors must be contiguous")


def kv_scatter(k_new, v_new, slots, k_pool, v_pool, stream=None):
    """k_pool[slots[i]] = k_new[i]; v_pool[slots[i]] = v_new[i]."""
    _need_cuda(k_new, v_new, slots, k_pool, v_pool)
    P, hkv, d = k_pool.shape
    return _check(lib().rkv_kv_scatter(_ptr(k_new), _ptr(v_new), _ptr(slots), int(slots.shape[0]),
                                       _ptr(k_pool), _ptr(v_pool), int(P), int(hkv), int(d),
                                       _dtype_code(k_pool), _stream(stream)))


def table_append(req_to_token, seq_lens, new_slots, stream=None):
    """Device tables: req_to_token[r, seq_lens[r]] = new_slots[r] and
    seq_lens[r] += 1 for every request r (int32 GPU tensors)."""
    import torch
    _need_cuda(req_to_token, seq_lens, new_slots)
    for t in (req_to_token, seq_lens, new_slots):
        if t.dtype != torch.int32:
            raise RkvError(EINVAL, "table_append takes int32 tensors")
    B = int(seq_lens.shape[0])
    if req_to_token.dim() != 2 or req_to_token.shape[0] != B or new_slots.shape[0] < B:
        raise RkvError(EINVAL, "table_append: req_to_token must be [B, ld], new_slots [B]")
    return _check(lib().rkv_table_append(_ptr(req_to_token), int(req_to_token.shape[1]), _ptr(seq_lens),
                                         _ptr(new_slots), B, _stream(stream)))


def attn_extend(q, k_pool, v_pool, o, req_to_token, qo_indptr, prefix_lens, max_new, lse=None,
                sm_scale=None, stream=None, order=None):
    """Causal extend attention of q [T, Hq, D] over each request's cached
    prefix plus its new tokens; writes o (and lse when given).  order: an
    optional int32 device permutation of the requests, the order in which
    their work is handed out (schedule only, e.g. longest first)."""
    _need_cuda(q, k_pool, v_pool, o, req_to_token, qo_indptr, prefix_lens, lse, order)
    T, hq, d = q.shape
    P, hkv, _ = k_pool.shape
    B = int(prefix_lens.shape[0])
    if order is not None and (order.dtype != prefix_lens.dtype or int(order.shape[0]) != B):
        raise RkvError(EINVAL, "attn_extend: order must be int32 [B]")
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    return _check(lib().rkv_attn_extend(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(o), _ptr(lse), _ptr(req_to_token),
        int(req_to_token.shape[1]), _ptr(qo_indptr), _ptr(prefix_lens), _ptr(order), B, int(T), int(max_new),
        int(hq), int(hkv), int(d), scale, _dtype_code(q), int(P), _stream(stream)))


def attn_decode_workspace_bytes(B, hq, d, max_seq_len, num_splits=0) -> int:
    return int(lib().rkv_attn_decode_workspace_bytes(int(B), int(hq), int(d), int(max_seq_len),
                                                     int(num_splits)))


def attn_decode(q, k_pool, v_pool, o, req_to_token, seq_lens, max_seq_len, workspace, lse=None,
                num_splits=0, sm_scale=None, stream=None):
    """Single-token split-KV decode of q [B, Hq, D] over all seq_lens[r] keys."""
    _need_cuda(q, k_pool, v_pool, o, req_to_token, seq_lens, lse, workspace)
    B, hq, d = q.shape
    P, hkv, _ = k_pool.shape
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return _check(lib().rkv_attn_decode(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(o), _ptr(lse), _ptr(req_to_token),
        int(req_to_token.shape[1]), _ptr(seq_lens), int(B), int(max_seq_len), int(hq), int(hkv),
        int(d), scale, _dtype_code(q), int(num_splits), _ptr(workspace), int(ws_bytes), int(P),
        _stream(stream)))


def attn_decode_noalloc(q, k_pool, v_pool, o, req_to_token, seq_lens, max_seq_len, lse=None, num_splits=0,
                        sm_scale=None, stream=None):
    """attn_decode without a workspace argument: the split partials go to the
    scratch the library holds per GPU (rkv_attn_decode_noalloc; it allocates
    nothing, and calls that overlap on one GPU race)."""
    _need_cuda(q, k_pool, v_pool, o, req_to_token, seq_lens, lse)
    B, hq, d = q.shape
    P, hkv, _ = k_pool.shape
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    return _check(lib().rkv_attn_decode_noalloc(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(o), _ptr(lse), _ptr(req_to_token),
        int(req_to_token.shape[1]), _ptr(seq_lens), int(B), int(max_seq_len), int(hq), int(hkv),
        int(d), scale, _dtype_code(q), int(num_splits), int(P), _stream(stream)))


class CascadePlan:
    """Host arrays of a prefix-shared decode plan (rkv_cascade_plan):
    perm [B], rec_indptr [B+1], tail_begin [B], jobs [n_jobs, 5] (int32
    NumPy), with tail_splits, n_records, max_members, tail_chunk and the
    seg_chunk it was planned with (host information only).  tail_order
    (int32 [B] or None): the order in which rkv_attn_decode_cascade hands
    out the requests' tail splits (None: batch order)."""

    def __init__(self, perm, rec_indptr, tail_begin, jobs, tail_splits, max_members, tail_chunk, seg_chunk=None):
        self.perm, self.rec_indptr, self.tail_begin, self.jobs = perm, rec_indptr, tail_begin, jobs
        self.tail_splits, self.max_members, self.tail_chunk = int(tail_splits), int(max_members), int(tail_chunk)
        self.seg_chunk = None if seg_chunk is None else int(seg_chunk)
        self.tail_order = None
        self.n_records = int(rec_indptr[-1])
        self.n_jobs = int(jobs.shape[0])
        self.dev = None

    def to(self, device):
        """Copies the arrays to `device` as int32 views of one buffer, each
        starting on a 16-byte boundary, sent by one asynchronous copy from
        pinned memory (a pageable copy would wait for the stream's earlier
        work, so a decode loop could not plan step k+1 while step k runs);
        returns self."""
        import torch
        parts = (("perm", self.perm), ("rec_indptr", self.rec_indptr), ("tail_begin", self.tail_begin),
                 ("jobs", self.jobs.reshape(-1)))
        if self.tail_order is not None:
            parts += (("tail_order", np.asarray(self.tail_order, dtype=np.int32)),)
        spans, off = {}, 0
        for k, v in parts:
            spans[k] = (off, int(v.size))
            off += (int(v.size) + 3) // 4 * 4
        pinned = torch.empty(max(off, 4), dtype=torch.int32, pin_memory=True)
        h = pinned.numpy()
        for k, v in parts:
            o, n = spans[k]
            h[o:o + n] = v.reshape(-1)
        dev = pinned.to(device, non_blocking=True)
        self.dev = {k: dev[o:o + n] for k, (o, n) in spans.items()}
        return self


def cascade_max_members(hq, hkv, d) -> int:
    """Largest max_members rkv_attn_decode_cascade accepts for these heads."""
    return max(1, (32 if int(d) == 128 else 64) // (int(hq) // int(hkv)))


def cascade_plan(req_to_token, seq_lens, seg_chunk=256, tail_chunk=768, min_keys=32, max_members=32):
    """Plans prefix-shared decode from the host table (NumPy int32 [B, ld]
    and seq_lens [B]).  Returns a CascadePlan."""
    r2t = np.ascontiguousarray(np.asarray(req_to_token, dtype=np.int32))
    L = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    B = int(L.shape[0])
    ld = int(r2t.shape[1]) if r2t.ndim == 2 else 0
    perm = np.empty(max(B, 1), dtype=np.int32)
    rec = np.empty(B + 1, dtype=np.int32)
    tb = np.empty(max(B, 1), dtype=np.int32)
    n_jobs, tail = _i64(), _i32()
    args = lambda jobs, cap: (r2t.ctypes.data_as(c_i32p), ld, L.ctypes.data_as(c_i32p), B, int(seg_chunk),
                              int(tail_chunk), int(min_keys), int(max_members), perm.ctypes.data_as(c_i32p),
                              rec.ctypes.data_as(c_i32p), tb.ctypes.data_as(c_i32p), jobs, cap,
                              ctypes.byref(n_jobs), ctypes.byref(tail))
    # one call with a generous capacity; a second only when it was too small
    jobs = np.empty((max(64, 8 * B), 5), dtype=np.int32)
    code = lib().rkv_cascade_plan(*args(jobs.ctypes.data_as(c_i32p), jobs.shape[0]))
    if code == ENOSPC:
        jobs = np.empty((n_jobs.value, 5), dtype=np.int32)
        code = lib().rkv_cascade_plan(*args(jobs.ctypes.data_as(c_i32p), n_jobs.value))
    _check(code)
    return CascadePlan(perm[:B], rec, tb[:B], jobs[: n_jobs.value], tail.value, max_members, tail_chunk, seg_chunk)


def attn_decode_cascade_workspace_bytes(n_records, hq, d) -> int:
    return int(lib().rkv_attn_decode_cascade_workspace_bytes(int(n_records), int(hq), int(d)))


def attn_decode_cascade(q, k_pool, v_pool, o, req_to_token, seq_lens, max_seq_len, plan, workspace, lse=None,
                        sm_scale=None, stream=None):
    """Prefix-shared decode of q [B, Hq, D] following `plan` (a CascadePlan
    already copied to the device with plan.to(device))."""
    _need_cuda(q, k_pool, v_pool, o, req_to_token, seq_lens, lse, workspace)
    if plan.dev is None:
        raise RkvError(EINVAL, "the plan's arrays are not on the device (call plan.to(device))")
    B, hq, d = q.shape
    P, hkv, _ = k_pool.shape
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dv = plan.dev
    return _check(lib().rkv_attn_decode_cascade(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(o), _ptr(lse), _ptr(req_to_token),
        int(req_to_token.shape[1]), _ptr(seq_lens), int(B), int(max_seq_len), int(hq), int(hkv), int(d),
        scale, _dtype_code(q), _ptr(dv["perm"]), _ptr(dv["rec_indptr"]), _ptr(dv["tail_begin"]),
        _ptr(dv["jobs"]) if plan.n_jobs else None, plan.n_jobs,
        _ptr(dv["tail_order"]) if "tail_order" in dv else None, plan.max_members, plan.tail_chunk,
        plan.tail_splits, plan.n_records, _ptr(workspace), int(ws_bytes), int(P), _stream(stream)))


class PenaltyState:
    """Device state of the sampling penalties for n_slots request slots over
    a vocabulary (rkv_penalty_*): counts [n_slots, vocab], seen [n_slots,
    cap], seen_len and out_len [n_slots], all int32 torch tensors."""

    def __init__(self, n_slots, vocab, cap, device="cuda"):
        import torch
        self.n_slots, self.vocab, self.cap = int(n_slots), int(vocab), int(cap)
        self.counts = torch.zeros(n_slots, vocab, dtype=torch.int32, device=device)
        self.seen = torch.zeros(n_slots, cap, dtype=torch.int32, device=device)
        self.seen_len = torch.zeros(n_slots, dtype=torch.int32, device=device)
        self.out_len = torch.zeros(n_slots, dtype=torch.int32, device=device)

    def _st(self):
        return (_ptr(self.counts), _ptr(self.seen), _ptr(self.seen_len), _ptr(self.out_len), self.n_slots,
                self.vocab, self.cap)

    def admit(self, rows, prompt_indptr, prompt_ids, stream=None):
        """rows [n], prompt_indptr [n+1], prompt_ids: device int32 tensors."""
        _need_cuda(rows, prompt_indptr, prompt_ids)
        return _check(lib().rkv_penalty_admit(*self._st(), int(rows.shape[0]), _ptr(rows), _ptr(prompt_indptr),
                                              _ptr(prompt_ids), _stream(stream)))

    def accumulate(self, rows, tokens, stream=None):
        """One output token per running request: rows [B], tokens [B] (device int32)."""
        _need_cuda(rows, tokens)
        return _check(lib().rkv_penalty_accumulate(*self._st(), int(rows.shape[0]), _ptr(rows), _ptr(tokens),
                                                   _stream(stream)))

    def apply(self, logits, rows, freq, pres, rep, min_new, stop_indptr, stop_ids, new_tokens=None, stream=None):
        """Penalizes logits [B, >= vocab] (fp32 or bf16) in place; per-entry
        device arrays freq, pres, rep (float32), min_new (int32), stop lists
        as CSR (stop_indptr [B+1], stop_ids).  new_tokens [B] (optional):
        each request's previous output token, recorded first in the same
        launch."""
        _need_cuda(logits, rows, freq, pres, rep, min_new, stop_indptr, stop_ids, new_tokens)
        B = int(rows.shape[0])
        return _check(lib().rkv_penalty_apply(
            _ptr(logits), int(logits.shape[1]), _dtype_code(logits), B, _ptr(rows), _ptr(self.counts),
            _ptr(self.seen), _ptr(self.seen_len), _ptr(self.out_len), self.n_slots, self.vocab, self.cap,
            _ptr(freq), _ptr(pres), _ptr(rep), _ptr(min_new), _ptr(stop_indptr),
            _ptr(stop_ids) if stop_ids is not None and stop_ids.numel() else None, _ptr(new_tokens),
            _stream(stream)))


def image_keys(data: bytes, n_tokens: int):
    """Radix keys of an image occupying n_tokens positions: (int32 NumPy
    array of n_tokens keys in [-2^31, -1], 64-bit content hash)."""
    keys = np.empty(max(int(n_tokens), 1), dtype=np.int32)
    h = ctypes.c_uint64()
    _check(lib().rkv_image_keys(bytes(data), len(data), int(n_tokens), keys.ctypes.data_as(c_i32p),
                                ctypes.byref(h)))
    return keys[: int(n_tokens)], h.value
