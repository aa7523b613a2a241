"""RadixKVCache: one token-slot KV pool on a GPU plus its radix tree.

A thin orchestration of the C-ABI calls in the order RadixAttention serves a
batch (unite.ai, "SGLang: Efficient Execution of Structured Language Model
Programs", walkthrough in section "SGLang: Modelo de programacion y
metodologia"): prepare (match the cached prefixes, lock them, allocate slots
for the rest, evicting least-recently-used nodes if the pool is short), store
the new tokens' K/V, attend, commit (insert the sequences, unlock).  Every
step runs in librkv; this module only moves arguments and owns the device
buffers (torch supplies the memory and the stream).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import rkv

POISON = {torch.bfloat16: 0x7FC0, torch.float32: 0x7FC00000}


@dataclass
class Batch:
    seqs: object                # the token ids as given (lists or an rkv.TokenBatch)
    host: dict                  # NumPy tables from batch_prepare
    req_to_token: torch.Tensor  # device int32 [B, ld]
    qo_indptr: torch.Tensor
    prefix_lens: torch.Tensor
    seq_lens: torch.Tensor
    new_slots: torch.Tensor
    max_new: int
    max_len: int
    total_new: int
    uploaded: object = None     # event after the tables' upload (the host tables are its source)
    order: torch.Tensor = None  # device int32 [B]: extend's work order (longest first); None = batch order


class RadixKVCache:
    def __init__(self, pool_slots: int, hkv: int, d: int, dtype=torch.bfloat16, device="cuda",
                 initial_free=None, poison: bool = True):
        self.pool_slots, self.hkv, self.d, self.dtype = int(pool_slots), hkv, d, dtype
        self.device = torch.device(device)
        self.tree = rkv.Tree(pool_slots, initial_free)
        shape = (self.pool_slots, hkv, d)
        if poison:
            bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
            val = POISON[dtype]
            val = val - (1 << 16) if (bits == torch.int16 and val >= 1 << 15) else val
            self.k_pool = torch.full(shape, val, dtype=bits, device=self.device).view(dtype)
            self.v_pool = torch.full(shape, val, dtype=bits, device=self.device).view(dtype)
        else:
            self.k_pool = torch.empty(shape, dtype=dtype, device=self.device)
            self.v_pool = torch.empty(shape, dtype=dtype, device=self.device)
        self._ws = None
        self._ws_retired = []

    # ---------------------------------------------------------------- host
    def prepare(self, seqs, ld=None) -> Batch:
        """seqs: a list of token-id sequences or an rkv.TokenBatch (converted
        once here either way and reused by commit)."""
        if not isinstance(seqs, rkv.TokenBatch):
            seqs = rkv.TokenBatch(seqs)
        B = len(seqs)
        if ld is None:
            ld = int(seqs.lens.max()) if B else 1
        # all int32 tables land in one pinned buffer and go up in one copy
        # (torch's pinned-block cache keeps the block until the copy is done)
        lay = rkv.Tree.table_layout(B, ld, int(seqs.lens.sum()))
        ow = (lay[-1] + 3) // 4 * 4          # the extend order follows, 16-byte aligned
        pinned = torch.empty(ow + max(B, 1), dtype=torch.int32, pin_memory=True)
        h = pinned.numpy()
        code, tb = self.tree.batch_prepare(seqs, ld, out=h[:lay[-1]])
        if code != rkv.OK:
            raise rkv.RkvError(code, "batch_prepare: eviction cannot free enough slots")
        order = self.extend_order(tb["seq_lens"])
        h[ow:ow + B] = order
        dev = pinned.to(self.device, non_blocking=True)
        uploaded = torch.cuda.Event()
        uploaded.record()
        T = int(tb["qo_indptr"][B])
        n = tb["seq_lens"].astype(np.int64) - tb["prefix_lens"]
        # batch order needs no order array (and spares extend one load)
        in_order = bool(np.array_equal(order, np.arange(B)))
        return Batch(seqs=seqs, host=tb, order=None if in_order else dev[ow:ow + B],
                     req_to_token=dev[:lay[1]].view(-1, ld)[:B],
                     prefix_lens=dev[lay[1]:lay[1] + B], seq_lens=dev[lay[2]:lay[2] + B],
                     qo_indptr=dev[lay[3]:lay[3] + B + 1], new_slots=dev[lay[4]:lay[4] + T],
                     max_new=int(n.max()) if len(n) else 0,
                     max_len=int(tb["seq_lens"].max()) if len(n) else 0, total_new=T, uploaded=uploaded)

    def append(self, batch: Batch) -> Batch:
        """Decode continuation of a prepared, uncommitted batch: one more
        position per request, without matching the histories again.  The
        host tables grow by rkv_batch_append, the device ones by
        rkv_table_append, so only the B new slot ids cross PCIe.  Updates
        and returns `batch` (new_slots then holds the step's B slots, for
        store); the batch must have been prepared with room in ld.  Commit
        with the extended sequences: commit(batch, seqs)."""
        if batch.uploaded is not None:
            batch.uploaded.synchronize()     # the prepare's upload reads the host tables
            batch.uploaded = None
        B = int(batch.host["seq_lens"].shape[0])
        pinned = torch.empty(max(B, 1), dtype=torch.int32, pin_memory=True)
        code, _ = self.tree.batch_append(batch.host["req_to_token"], batch.host["seq_lens"], out=pinned.numpy())
        if code != rkv.OK:
            raise rkv.RkvError(code, "batch_append: eviction cannot free enough slots")
        dev = pinned[:B].to(self.device, non_blocking=True)
        rkv.table_append(batch.req_to_token, batch.seq_lens, dev)
        batch.new_slots = dev
        batch.max_len += 1
        batch.max_new = 1 if B else 0
        batch.total_new = B
        return batch

    def commit(self, batch: Batch, seqs=None):
        """Inserts the batch's sequences (`seqs` when the batch was extended
        by append) and unlocks their paths.  Every sequence must be as long
        as its table row (seq_lens, grown by append): the tree inserts only
        len(seq) entries of a row, so a shorter sequence would leave the
        slots after it neither cached nor free."""
        seqs = batch.seqs if seqs is None else seqs
        lens = seqs.lens if isinstance(seqs, rkv.TokenBatch) else np.array([len(s) for s in seqs])
        want = batch.host["seq_lens"]
        if len(lens) != len(want) or not np.array_equal(np.asarray(lens, dtype=np.int64), want.astype(np.int64)):
            raise ValueError("commit: each sequence must be as long as its table row (after append, "
                             "pass the grown sequences)")
        self.tree.batch_commit(seqs, batch.host["req_to_token"], batch.host["nodes"])

    # ---------------------------------------------------------------- device
    def store(self, batch: Batch, k_new, v_new, stream=None):
        rkv.kv_scatter(k_new, v_new, batch.new_slots, self.k_pool, self.v_pool, stream)

    def extend(self, batch: Batch, q, o=None, lse=None, stream=None):
        if o is None:
            o = torch.empty_like(q)
        rkv.attn_extend(q, self.k_pool, self.v_pool, o, batch.req_to_token, batch.qo_indptr,
                        batch.prefix_lens, batch.max_new, lse=lse, stream=stream, order=batch.order)
        return o

    XCDS = 8    # MI355X: 256 CUs in 8 XCDs, each with its own L2

    def extend_order(self, seq_lens):
        """Extend's work order (schedule only: outputs do not depend on it).
        Each XCD takes a contiguous range of work items, kv head major.
        With the kv heads a multiple of 8 a range is whole heads, and the
        requests go longest first (ties in batch order), so no launch ends on
        a long request started late (chat batches 5-7 % faster).  Otherwise a
        range is a run of requests, where sorting would pile the longest onto
        one XCD (7-16 % slower on one kv head): the sorted requests are dealt
        back and forth over 8 bins (0..7, 7..0, ...) and the bins
        concatenated, so every range gets long and short ones, longest first
        within it (one kv head of the 64/8-head extend batch: 16 % faster
        than batch order)."""
        return self._xcd_order(seq_lens, self.hkv)

    def _xcd_order(self, keys, units):
        """Largest keys first when each XCD's contiguous item range is whole
        units (units a multiple of 8), else dealt over 8 bins as above."""
        srt = np.argsort(-np.asarray(keys, dtype=np.int64), kind="stable")
        if units % self.XCDS == 0:
            return srt
        k = np.arange(srt.shape[0]) % (2 * self.XCDS)
        bins = np.where(k < self.XCDS, k, 2 * self.XCDS - 1 - k)
        return srt[np.argsort(bins, kind="stable")]

    def workspace(self, B, hq, max_len, num_splits=0, need=None):
        """Decode workspace of at least `need` bytes (by default what plain
        decode of this shape needs).  It grows geometrically, and a replaced
        buffer is kept alive with the cache, since a captured StepGraph may
        still write into it."""
        if need is None:
            need = rkv.attn_decode_workspace_bytes(B, hq, self.d, max_len, num_splits)
        if self._ws is None or self._ws.numel() * 4 < need:
            if self._ws is not None:
                self._ws_retired.append(self._ws)
                need = max(need, 2 * self._ws.numel() * 4)
            self._ws = torch.empty(max((need + 3) // 4, 1), dtype=torch.float32, device=self.device)
        return self._ws

    def decode_splits(self, batch: Batch, hq):
        """Splits per request for plain decode: 0 (768-key chunks, so a
        request's output bits do not depend on its batch) unless the
        grouped-head kernel (bf16, Hq/Hkv >= 4) would then get fewer items
        than MIN_TAIL_ITEMS; then enough splits for that many items, with
        chunks of at least 256 keys.  Such launches are latency-bound and
        shorter items finish sooner (one GPU's 8/1 heads of the 64/8-head
        decode batch: 33.1 -> 30.9 us at 16 splits)."""
        L = batch.host["seq_lens"].astype(np.int64)
        if hq // self.hkv < 4 or self.k_pool.dtype != torch.bfloat16 or len(L) == 0:
            return 0
        if int(((L + 767) // 768).sum()) * self.hkv >= self.MIN_TAIL_ITEMS:
            return 0
        ns = -(-self.MIN_TAIL_ITEMS // (len(L) * self.hkv))
        ns = min(ns, int(L.max()) // 256)
        return ns if ns > -(-int(L.max()) // 768) else 0

    def decode(self, batch: Batch, q, o=None, lse=None, num_splits=None, stream=None):
        """Plain decode; num_splits None: the rule of decode_splits."""
        if o is None:
            o = torch.empty_like(q)
        B, hq, _ = q.shape
        if num_splits is None:
            num_splits = self.decode_splits(batch, hq)
        ws = self.workspace(B, hq, batch.max_len, num_splits)
        rkv.attn_decode(q, self.k_pool, self.v_pool, o, batch.req_to_token, batch.seq_lens,
                        batch.max_len, ws, lse=lse, num_splits=num_splits, stream=stream)
        return o

    # Tail chunk of the prefix-shared plan: 768 keys (measured best on the
    # 32-head and 64/8-head decode batches), halved when the tails would then
    # give the grouped-head kernel fewer items than the chip has SIMDs (1024):
    # such launches are latency-bound, and shorter items finish sooner (one
    # GPU's 8/1 heads of the 64/8 decode batch, 312 tail items at 768 keys:
    # 36.7 -> 33.9 us at 384).
    # Shared chunk: the tail chunk, so a shared item is no longer than a tail
    # item and a shared run is cut into as few partial states as that allows
    # (64/8-head decode under a 2048-key prefix: 207.0 us at 256-key chunks,
    # 191.2 at 512, 188.5 at 768, 194.4 at 1024; the 32-head tree batch 1135.8
    # / 1126.7 / 1127.5 us at 256 / 512 / 768).  When the tail chunk is halved
    # the shared chunk is 256 keys: a shared item computes several requests'
    # query columns per key and takes longer per step than a tail item, and
    # in a latency-bound launch the longest item sets the time (the 8/1-head
    # share: 28.4 us at 256, 29.5 at 192, 32.5 at 384).
    TAIL_CHUNK = 768
    MIN_TAIL_ITEMS = 1024
    SEG_CHUNK_SMALL = 256

    def cascade_plan(self, batch: Batch, hq, seg_chunk=None, tail_chunk=None, min_keys=32, max_members=None,
                     longest_tails_first=True):
        """Plans prefix-shared decode from the batch's host tables and copies
        the plan to the device.  seg_chunk / tail_chunk None: the rules
        above; longest_tails_first: the tail order below."""
        return self.cascade_plan_host(batch, hq, seg_chunk, tail_chunk, min_keys, max_members,
                                      longest_tails_first).to(self.device)

    def cascade_plan_host(self, batch: Batch, hq, seg_chunk=None, tail_chunk=None, min_keys=32, max_members=None,
                          longest_tails_first=True):
        """The host plan of cascade_plan, before its copy to the device.

        Tail order: the requests whose tail splits are longest go first
        (ties in batch order), so the launch ends on short items.  A
        request's splits have equal lengths (the kernels' rule: the tail in
        ceil(tail / tail_chunk) splits, rounded up to 64 keys, never above
        tail_chunk).  Each XCD takes a contiguous range of tail items, kv
        head (block) major, so as in extend_order the sorted requests are
        dealt over 8 bins unless a range is whole head blocks: on the matrix
        cores (Hq/Hkv >= 4) one item covers one kv head; on the vector units
        a workgroup covers up to 4 kv heads of up to 8 q heads each (the
        kernel's head blocking, repeated here).  Interleaved on one GPU:
        the 32-head tree batch 1130.8 -> 1118.4 us, the 64/8-head batch
        190.4 -> 185.5 us.  A launch of fewer tail items than
        MIN_TAIL_ITEMS runs its items in about one round, and there any
        order measured slower (the 8/1-head share: 31.1 us in batch order,
        31.8 longest first, 32.8 dealt over the XCDs): it keeps batch
        order."""
        mm = rkv.cascade_max_members(hq, self.hkv, self.d) if max_members is None else max_members
        tc = self.TAIL_CHUNK if tail_chunk is None else tail_chunk
        sc = tc if seg_chunk is None else seg_chunk
        rows, lens = batch.host["req_to_token"], batch.host["seq_lens"]
        plan = rkv.cascade_plan(rows, lens, sc, tc, min_keys, mm)
        if tail_chunk is None and hq // self.hkv >= 4:
            # where the tails start does not depend on either chunk
            tails = lens.astype(np.int64) - plan.tail_begin
            items = int(((tails + tc - 1) // tc).sum()) * self.hkv
            if 0 < items < self.MIN_TAIL_ITEMS:
                sc = self.SEG_CHUNK_SMALL if seg_chunk is None else seg_chunk
                plan = rkv.cascade_plan(rows, lens, sc, tc // 2, min_keys, mm)
        if longest_tails_first and len(lens) > 1:
            tails = np.maximum(lens.astype(np.int64) - plan.tail_begin, 1)
            tcp = plan.tail_chunk
            n = (tails + tcp - 1) // tcp
            split = np.minimum(np.minimum(((tails + n - 1) // n + 63) // 64 * 64, tcp), tails)
            G = hq // self.hkv
            if G >= 4:
                units = self.hkv
            else:
                hb = 4
                while hb > 1 and hb // 2 >= self.hkv:
                    hb //= 2
                units = -(-self.hkv // hb) * -(-G // 8)
            if int(n.sum()) * units >= self.MIN_TAIL_ITEMS:
                plan.tail_order = self._xcd_order(split, units).astype(np.int32)
        return plan

    def decode_cascade(self, batch: Batch, q, plan=None, o=None, lse=None, stream=None, **plan_args):
        """Decode that reads each run of keys shared by several requests of
        the batch once (plan from cascade_plan, made here when not given)."""
        if o is None:
            o = torch.empty_like(q)
        B, hq, _ = q.shape
        if plan is None:
            plan = self.cascade_plan(batch, hq, **plan_args)
        ws = self.workspace(B, hq, batch.max_len,
                            need=rkv.attn_decode_cascade_workspace_bytes(plan.n_records, hq, self.d))
        rkv.attn_decode_cascade(q, self.k_pool, self.v_pool, o, batch.req_to_token, batch.seq_lens,
                                batch.max_len, plan, ws, lse=lse, stream=stream)
        return o


class StepGraph:
    """A device step (a fixed sequence of library calls on fixed buffers)
    captured once into a HIP graph and replayed.  A replay skips the host
    side of every call (argument checks, marshalling, one launch per kernel),
    which bounds small decode steps: a decode over a few hundred thousand
    keys runs for tens of microseconds, about what its host side takes.

    `fn` issues the step on the current stream; everything it reads (query
    rows, tables, the plan, the pools) is read from the buffers it was given
    when captured, so refresh their contents in place before `replay()`.
    Sizes that fix a launch grid (batch size, maximum context length, the
    plan's job and record counts) are frozen at capture: capture again when
    they change.  `fn` must not allocate; run it once eagerly first (the
    constructor does, on a side stream) so that caches such as the decode
    workspace are sized.  Not under RKV_DEBUG=1, whose error check
    synchronizes the stream."""

    def __init__(self, fn, warmup: int = 1):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            fn()

    def replay(self):
        self.graph.replay()
