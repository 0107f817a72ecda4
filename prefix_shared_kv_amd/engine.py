"""Host-side sequencing of the hot path for one attention layer.

Owns the KV pool (two device tensors), the request->slot table (host copy and
device copy) and the radix tree.  Each method issues library calls only: the
tree and planners run in the C++ host library, K/V movement and attention in
the HIP kernels.  Host->device copies of integer metadata (table rows, slot
lists, lengths, plans) are the only other device traffic.

Flow of one batch ("Prompt Caching" glossary, GPT-2 example; SGLang summary,
RadixAttention and `fork`):
  schedule   longest cached prefix per request (pinned while the request
             runs), slots for the new tokens and for the decode steps,
             evicting least recently used unpinned nodes when the pool is
             short, table rows                           (host, C++)
  extend     store new K/V in the pool, attend            (kv_store, extend)
  commit     insert prompts into the tree; rows get the tree's slots; the
             request's pin moves to what it stored
  prepare_decode  share plan from the tree (who reads which node), per-step
             slot and length tables uploaded once
  decode_step  store the token's K/V, split-K attention over shared nodes,
             merge                                        (kv_store, decode)
"""
from __future__ import annotations

import collections
import dataclasses
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import _native as N
from . import api
from .api import DecodePlan, KVShape, RadixTree, TokenBatch


@dataclasses.dataclass
class Batch:
    tb: TokenBatch             # the requests' token ids, flattened once
    rows: np.ndarray           # table row of each request
    prefix_lens: np.ndarray    # P_b
    extend_lens: np.ndarray    # E_b
    reserve: int
    entries: np.ndarray        # table entries each row uses (tokens, or pages)
    new_slots: np.ndarray      # pool slots of the new tokens, request after request
    locks: Optional[np.ndarray] = None  # lock handles pinning each request's cached tokens
    dev: dict = dataclasses.field(default_factory=dict)
    own_rows: bool = True      # rows came from the engine's free list (returned at release)

    @property
    def size(self) -> int:
        return len(self.tb)

    @property
    def tokens(self) -> List[np.ndarray]:
        return [self.tb[i] for i in range(len(self.tb))]

    @property
    def total_extend(self) -> int:
        return int(self.extend_lens.sum())


@dataclasses.dataclass
class DecodeState:
    plan: DecodePlan
    base_lens: np.ndarray      # position of decode step 0 per request
    n_steps: int
    slots: torch.Tensor        # [n_steps, B] int32: slot of each step's token
    seq_lens: torch.Tensor     # [n_steps, B] int32: keys attended at each step
    workspace: torch.Tensor
    launcher: Optional[api.DecodeLauncher] = None  # built at the first fused step


class Engine:
    def __init__(self, shape: KVShape, stride: int, max_rows: int, device="cuda",
                 free_order: Optional[np.ndarray] = None, k_pool: Optional[torch.Tensor] = None,
                 v_pool: Optional[torch.Tensor] = None):
        self.shape = shape
        self.device = torch.device(device)
        S, H, D = shape.pool_slots, shape.num_kv_heads, shape.head_dim
        self.k_pool = k_pool if k_pool is not None else torch.zeros((S, H, D), dtype=shape.dtype, device=self.device)
        self.v_pool = v_pool if v_pool is not None else torch.zeros((S, H, D), dtype=shape.dtype, device=self.device)
        # Paged pool (shape.page_size > 1): the tree hands out and shares whole
        # pages, table rows hold page ids, and a position's slot is its page's
        # first slot plus its offset in the page.  free_order is then over pages.
        self.ps = shape.page_size
        if S % self.ps:
            raise ValueError("pool_slots must be a multiple of page_size")
        self.tree = RadixTree(S // self.ps, free_order, page_size=self.ps)
        self.stride = stride                     # most positions a row describes
        self.width = -(-stride // self.ps)       # table entries per row
        # Rows are handed out oldest-free first.  With about two batches' worth
        # of rows, a batch never waits for rows whose upload is still queued
        # behind the GPU work of the batch before it.  (Row uploads stay on the
        # compute stream: run beside the decode kernels on a copy stream they
        # cost those kernels more than the copy takes.)
        # The host table lives in pinned memory so that runs of rows upload
        # straight from it.  Such an upload reads the rows when the stream
        # reaches it, so a row is rewritten on the host only after the last
        # upload that covered it has completed: each row remembers the number
        # of that upload, and the uploads' events complete in stream order.
        self._table_pin = torch.full((max_rows, self.width), -1, dtype=torch.int32, pin_memory=True)
        self.table_h = self._table_pin.numpy()
        self._row_upload = np.zeros(max_rows, np.int64)  # number of the last upload reading each row
        self._uploads = collections.deque()              # (number, event) of uploads not known complete
        self._n_uploads = 0
        self.table_d = torch.full((max_rows, self.width), -1, dtype=torch.int32, device=self.device)
        self.free_rows = list(range(max_rows))

    # -- helpers ------------------------------------------------------------
    # Host->device copies go through a ring of persistent pinned staging
    # buffers and do not block the host, which keeps preparing (tree calls,
    # plans) while the GPU works.  A buffer is rewritten only after the copy
    # that last read it has completed (its event); allocating pinned memory
    # per copy instead can synchronise the whole device.
    # Every buffer is allocated up front at _RING_BYTES, so steady-state
    # copies allocate no pinned memory; a larger array gets a buffer of its own.
    _RING = 64
    _RING_BYTES = 1 << 20

    def _pinned(self, a: np.ndarray) -> torch.Tensor:
        a = np.ascontiguousarray(a)
        if not hasattr(self, "_ring"):
            self._ring = [[torch.empty(self._RING_BYTES, dtype=torch.uint8, pin_memory=True), None]
                          for _ in range(self._RING)]
            self._ring_i = 0
        slot = self._ring[self._ring_i]
        self._ring_i = (self._ring_i + 1) % self._RING
        buf, ev = slot
        if ev is not None:
            ev.synchronize()
        if buf.numel() < a.nbytes:
            buf = torch.empty(a.nbytes, dtype=torch.uint8, pin_memory=True)
            slot[0] = buf
        view = buf[:a.nbytes].view(torch.from_numpy(a[:0].reshape(-1)).dtype).view(a.shape)
        view.copy_(torch.from_numpy(a))
        slot[1] = None
        self._last_slot = slot
        return view

    def _h2d(self, a: np.ndarray, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        src = self._pinned(a)
        if out is None:
            out = torch.empty(src.shape, dtype=src.dtype, device=self.device)
        out.copy_(src, non_blocking=True)
        ev = torch.cuda.Event()
        ev.record(torch.cuda.current_stream(self.device))
        self._last_slot[1] = ev
        return out

    def _i32(self, a) -> torch.Tensor:
        return self._h2d(np.asarray(a, np.int32))

    def _i32_many(self, *arrays) -> List[torch.Tensor]:
        """Several int32 arrays in one upload: device views of one buffer, each in its array's shape."""
        parts = [np.asarray(a, np.int32) for a in arrays]
        flat = self._i32(np.concatenate([p.reshape(-1) for p in parts]) if parts else np.zeros(0, np.int32))
        out, o = [], 0
        for p in parts:
            out.append(flat[o:o + p.size].view(p.shape))
            o += p.size
        return out

    def _upload_rows(self, rows: np.ndarray, first: Optional[np.ndarray] = None,
                     end: Optional[np.ndarray] = None) -> None:
        """Upload entries [first[i], end[i]) of each row rows[i] (default: whole rows).  The
        device table then equals the host table on those rows: entries before first[i] must
        already be equal (emit_rows reports where a row starts to differ)."""
        if len(rows) == 0:
            return
        # one 2D copy per run of consecutive (distinct) rows, straight from the pinned table:
        # the rectangle spanning the run's changed entries
        r = np.asarray(rows, np.int64)
        order = np.argsort(r, kind="stable")
        r = r[order]
        lo = np.zeros(len(r), np.int64) if first is None else np.asarray(first, np.int64)[order]
        hi = np.full(len(r), self.width, np.int64) if end is None else np.asarray(end, np.int64)[order]
        cuts = np.flatnonzero(np.diff(r) != 1) + 1
        for i0, i1 in zip(np.concatenate([[0], cuts]), np.concatenate([cuts, [len(r)]])):
            a, b = int(r[i0]), int(r[i1 - 1]) + 1
            c0, c1 = int(lo[i0:i1].min()), int(hi[i0:i1].max())
            if c1 > c0:
                api.upload_table_rows(self.table_d, self._table_pin, a, b - a, c0, c1)
        ev = torch.cuda.Event()
        ev.record(torch.cuda.current_stream(self.device))
        self._n_uploads += 1
        self._uploads.append((self._n_uploads, ev))
        self._row_upload[r] = self._n_uploads

    def _rows_writable(self, rows: np.ndarray) -> None:
        """Wait until no pending upload still reads these rows of the host table."""
        if len(rows) == 0 or not self._uploads:
            return
        need = int(self._row_upload[np.asarray(rows, np.int64)].max())
        while self._uploads and self._uploads[0][0] <= need:
            n, ev = self._uploads.popleft()
            if n == need or not self._uploads or self._uploads[0][0] > need:
                ev.synchronize()  # later events of the stream imply the earlier ones
                break
        while self._uploads and self._uploads[0][1].query():
            self._uploads.popleft()

    # -- cache population (a sequence whose K/V are already known) -----------
    def populate(self, tokens: Sequence[int], k: torch.Tensor, v: torch.Tensor, expect_cached: Optional[int] = None) -> int:
        """Store K/V for the uncached tail of `tokens` and insert the sequence (K/V computed
        elsewhere, e.g. a prefix loaded from storage).  k, v hold rows for positions [cached, n),
        cached being the whole cached prefix (whole pages in a paged pool).  Returns it."""
        t = np.ascontiguousarray(tokens, np.int32)
        b = self.schedule(TokenBatch([t]), full_match=True)
        stored = False
        try:
            m, n_new = int(b.prefix_lens[0]), int(b.extend_lens[0])
            if expect_cached is not None and m != expect_cached:
                raise RuntimeError(f"expected {expect_cached} cached tokens, found {m}")
            if k.shape[0] != n_new or v.shape[0] != n_new:
                raise ValueError(f"need K/V for {n_new} uncached tokens, got {k.shape[0]}")
            if n_new:
                api.kv_store(self.shape, self.k_pool, self.v_pool, k, v, b.dev["slots"])
            self.commit(b)
            stored = True
        finally:
            # stored: slots past the tree's whole units (a partial last page) go back;
            # otherwise every slot the call took
            self.release(b, keep=None if stored else b.prefix_lens)
        return m

    # -- a batch of requests --------------------------------------------------
    def take_rows(self, n: int) -> np.ndarray:
        """Hand n table rows to the caller, who schedules batches on them (schedule's `rows`) until
        give_rows.  A request scheduled again on the row it had keeps that row's unchanged entries
        on the device: only the entries that differ are uploaded."""
        if n > len(self.free_rows):
            raise RuntimeError("no free table rows")
        rows = np.array(self.free_rows[:n], np.int32)
        del self.free_rows[:n]
        return rows

    def give_rows(self, rows: np.ndarray) -> None:
        self.free_rows.extend(int(r) for r in rows)

    def schedule(self, batch_tokens, reserve: int = 0, evict: bool = True,
                 rows: Optional[np.ndarray] = None, full_match: bool = False) -> Batch:
        """batch_tokens: a list of token-id arrays or a TokenBatch.  Each request's cached prefix
        is pinned until release; with evict, least recently used unpinned nodes make room when
        the free slots fall short.  rows: table rows from take_rows, one per request, not used by
        another live batch (default: rows from the free list).  full_match: a fully cached request
        gets no new tokens (populate), instead of recomputing its last one."""
        tb = batch_tokens if isinstance(batch_tokens, TokenBatch) else TokenBatch(batch_tokens)
        B = len(tb)
        own = rows is None
        if own:
            if B > len(self.free_rows):
                raise RuntimeError("no free table rows")
            rows = np.array(self.free_rows[:B], np.int32)
        else:
            rows = np.ascontiguousarray(rows, np.int32)
            if rows.shape != (B,):
                raise ValueError(f"{B} requests need {B} rows, got {rows.shape}")
        self._rows_writable(rows)
        locks = np.zeros(B, np.int64)
        first = np.zeros(B, np.int64)
        entries = np.zeros(B, np.int64)
        slots = np.zeros(max(tb.flat.size, 1), np.int32)
        P, E = self.tree.emit_rows(tb, self.table_h, rows=rows, reserve=reserve, evict=evict, handles=locks,
                                   first_changed=first, full_match=full_match, row_entries=entries, new_slots=slots)
        if own:
            del self.free_rows[:B]
        self._upload_rows(rows, first, entries)
        b = Batch(tb, rows, P, E, reserve, entries, slots[:int(E.sum())], locks, own_rows=own)
        # requests' new tokens are packed one after the other in q, k_new, v_new and o
        start = np.zeros(B, np.int32)
        if B:
            start[1:] = np.cumsum(E)[:-1]
        # every integer array the batch's launches read, in one upload
        names = ("rows", "P", "E", "start", "slots")
        b.dev = dict(zip(names, self._i32_many(rows, P, E, start, b.new_slots)))
        return b

    # workgroups of the cascade's split-K launch resident at once: one 8-wave workgroup per CU
    def _resident_workgroups(self) -> int:
        if not hasattr(self, "_resident"):
            self._resident = torch.cuda.get_device_properties(self.device).multi_processor_count
        return self._resident

    def _cascade_chunk(self, b: Batch) -> int:
        """Piece length for the shared ranges of a cascade extend: as many pieces as keep every
        workgroup of the launch resident at once (one round, no tail), no more.  Each piece of
        a shared range becomes ceil(new tokens / tokens per group) workgroups per kv head."""
        per_group = max(1, N.RC_EXTEND_SHARED_COLS // self.shape.group)
        groups = -(-b.total_extend // per_group) * self.shape.num_kv_heads
        pieces = max(1, self._resident_workgroups() // max(groups, 1))
        longest = int(b.prefix_lens.max()) if b.size else 0
        return max(64, -(-longest // pieces))

    def extend(self, b: Batch, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, sm_scale: float,
               o: Optional[torch.Tensor] = None, store: bool = True, cascade: bool = False,
               chunk: Optional[int] = None) -> torch.Tensor:
        """Store the new tokens' K/V in their slots, then attend (new tokens over prefix + themselves).
        cascade: compute it from a shared-prefix plan (rc_radix_plan_extend) with the split-K
        kernel, so a prefix shared by many requests is read once for all their new tokens; chunk
        (default: sized from the launch) is the plan's piece length."""
        T = b.total_extend
        if q.shape[0] != T:
            raise ValueError(f"q has {q.shape[0]} rows, the batch has {T} new tokens")
        if store or cascade:  # the cascade path reads every key, the new ones too, from the pool
            api.kv_store(self.shape, self.k_pool, self.v_pool, k_new, v_new, b.dev["slots"])
        if o is None:
            o = torch.empty_like(q)
        if T == 0:
            return o
        if cascade:
            chunk = chunk or self._cascade_chunk(b)
            plan = self.tree.plan_extend(b.tb, b.prefix_lens, b.extend_lens, self.shape.group, chunk, rows=b.rows)
            plan.dev, seq_d = self._i32_many(plan.host, plan.seq_lens)
            ws = torch.empty(api.decode_workspace_bytes(self.shape, plan), dtype=torch.uint8, device=self.device)
            api.extend_attention_shared(self.shape, o, q, self.k_pool, self.v_pool, self.table_d, seq_d,
                                        plan, sm_scale, ws)
            return o
        api.extend_attention(self.shape, o, q, k_new, v_new, self.k_pool, self.v_pool, self.table_d, b.dev["P"],
                             b.dev["E"], b.dev["start"], int(b.extend_lens.max()) if b.size else 0, sm_scale,
                             rows=b.dev["rows"])
        return o

    def commit(self, b: Batch, lengths: Optional[Sequence[int]] = None) -> None:
        """Insert each request's first `lengths[i]` tokens (default: all) into the tree.
        Where the tree already held them, the row is rewritten to the tree's slots."""
        # The insert works on a copy of the batch's rows (the table's rows may
        # still be uploading); only rows the tree rewrote are written back.
        width = max(int(b.entries.max()) if b.size else 0, 1)
        work = np.ascontiguousarray(self.table_h[b.rows, :width])
        changed = self.tree.insert_rows(b.tb, work, np.arange(b.size, dtype=np.int32), lengths)
        if b.locks is not None:  # pin what is stored now, then drop the old pins
            locks, _ = self.tree.lock(b.tb, lengths)
            self.tree.unlock(b.locks)
            b.locks = locks
        if changed.any():
            rows = b.rows[changed]
            self._rows_writable(rows)
            self.table_h[rows, :width] = work[changed]
            self._upload_rows(np.sort(rows))

    # Decode piece length when the caller gives none.  A step that reads much
    # (more than fits the Infinity Cache) streams HBM, where long pieces start
    # up fewest times; a small step is latency-bound and wants many short items.
    _STREAM_BYTES = 128 << 20

    def _decode_chunk(self, unique_positions: int) -> int:
        """Pieces of 4096 positions when the step's unique K/V bytes exceed _STREAM_BYTES; below
        that, the power of two nearest unique_positions * kv_heads / 512 (within [64, 4096]), so
        a small step spreads over many short work items."""
        el = 4 if self.shape.dtype == torch.float32 else 2
        row = 2 * self.shape.num_kv_heads * self.shape.head_dim * el
        if unique_positions * row >= self._STREAM_BYTES:
            return 4096
        x = max(unique_positions * self.shape.num_kv_heads / 512.0, 1.0)
        return int(min(4096, max(64, 2 ** round(np.log2(x)))))

    def prepare_decode(self, b: Batch, base_lens: Sequence[int], n_steps: int, chunk: Optional[int] = None,
                       shared: bool = True, committed: Optional[Sequence[int]] = None) -> DecodeState:
        """Plan decode steps t = 0..n_steps-1; step t's token sits at position base_lens[i] + t.
        `committed[i]` tokens of request i are in the tree (default: base_lens).  chunk: the
        plan's piece length (default: from the step's size, _decode_chunk)."""
        base = np.asarray(base_lens, np.int32)
        com = base if committed is None else np.asarray(committed, np.int32)
        if np.any(com > base):
            # the plan would share positions the decode steps overwrite
            raise ValueError("committed tokens reach past a request's first decode position")
        if n_steps < 1:
            raise ValueError("n_steps must be at least 1")
        # each step's token slot and context length, from the table rows (positions past a row's
        # reserved entries are rejected)
        slots, seq = api.decode_steps(self.table_h, b.rows, base, n_steps, self.ps, row_entries=b.entries)
        g = self.shape.group

        def make(c):
            if shared:
                return self.tree.plan_decode(b.tb, seq[-1], g, c, rows=b.rows, lengths=com)
            return api.plan_decode_unshared(seq[-1], g, c, rows=b.rows)

        plan = make(chunk or 4096)
        if chunk is None:
            auto = self._decode_chunk(plan.info.unique_positions)
            if auto != 4096:
                plan = make(auto)
        plan.dev, slots_d, seq_d = self._i32_many(plan.host, slots, seq)
        ws = torch.empty(api.decode_workspace_bytes(self.shape, plan), dtype=torch.uint8, device=self.device)
        return DecodeState(plan, base, n_steps, slots_d, seq_d, ws)

    def decode_step(self, st: DecodeState, t: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    sm_scale: float, o: Optional[torch.Tensor] = None, fused_store: bool = True) -> torch.Tensor:
        """Store step t's K/V in the pool and attend over each request's whole context
        (one call with fused_store, else a scatter then the attention)."""
        if o is None:
            o = torch.empty_like(q)
        if not 0 <= t < st.n_steps:
            raise IndexError(f"step {t} outside the {st.n_steps} planned")
        if fused_store:
            ln = st.launcher
            if ln is None or ln._scale != float(sm_scale):
                ln = st.launcher = api.DecodeLauncher(self.shape, self.k_pool, self.v_pool, self.table_d, st.plan,
                                                      st.workspace, sm_scale, st.seq_lens.shape[1])
            B4 = 4 * st.seq_lens.shape[1]  # int32 rows of seq_lens and slots
            ln(o, q, st.seq_lens.data_ptr() + t * B4, k_new=k, v_new=v, new_slots_ptr=st.slots.data_ptr() + t * B4)
        else:
            api.kv_store(self.shape, self.k_pool, self.v_pool, k, v, st.slots[t])
            api.decode_attention(self.shape, o, q, self.k_pool, self.v_pool, self.table_d, st.seq_lens[t], st.plan,
                                 sm_scale, st.workspace)
        return o

    def release(self, b: Batch, keep: Optional[Sequence[int]] = None) -> None:
        """Return the batch's table rows; slots past `keep[i]` (default: tokens given) go back to the pool
        unless the tree holds them."""
        if b.locks is not None:
            self.tree.unlock(b.locks)
            b.locks = None
        keep = b.tb.lens() if keep is None else np.asarray(keep, np.int64)
        # the units past the kept tokens (a partly kept page included) are the request's own
        self.tree.free_rows(b.rows, self.table_h, keep, b.entries)
        # the rows' entries are left as they are: the next schedule rewrites
        # every entry a request can read
        if b.own_rows:
            self.free_rows.extend(int(r) for r in b.rows)
