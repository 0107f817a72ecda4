"""Python binding of the C ABI (include/rc.h).

Argument marshalling only: tensors are checked for device, dtype and layout,
then their device pointers and the current HIP stream are handed to the
library.  Every computation runs in the library's HIP kernels (GPU calls) or
its C++ radix tree (host calls).  PyTorch provides device memory and streams.
"""
from __future__ import annotations

import ctypes as C
import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import _native as N
from ._native import RcPlanInfo, RcProfEntry, RcRadixStats, RcShape, check, lib

_DT = {torch.float32: N.RC_F32, torch.bfloat16: N.RC_BF16}


def _vp(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _np_ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


@dataclasses.dataclass(frozen=True)
class KVShape:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: torch.dtype
    pool_slots: int
    page_size: int = 1  # > 1: req_to_token holds page ids, one per page_size positions

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def c(self) -> RcShape:
        if self.dtype not in _DT:
            raise TypeError(f"dtype {self.dtype} not supported")
        return RcShape(_DT[self.dtype], self.num_q_heads, self.num_kv_heads, self.head_dim, self.pool_slots,
                       self.page_size, 0)


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None:
        for i, (a, b) in enumerate(zip(t.shape, shape)):
            if b is not None and a != b:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
        if len(t.shape) != len(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    return t


def set_error_word(word: Optional[torch.Tensor]) -> None:
    """Register a device int32 tensor (1 element) that kernels OR error bits into."""
    if word is not None:
        _dev(word, "error word", torch.int32)
    check(lib.rc_set_error_word(_vp(word)))


def upload_table_rows(dev_table: torch.Tensor, host_table: torch.Tensor, row0: int, n_rows: int, col0: int, col1: int,
                      stream=None) -> None:
    """Copy rows [row0, row0 + n_rows) x entries [col0, col1) of a pinned host int32 table to the
    device table (rc_upload_table_rows): one asynchronous 2D copy."""
    _dev(dev_table, "dev_table", torch.int32)
    if host_table.device.type != "cpu" or host_table.dtype != torch.int32 or host_table.dim() != 2:
        raise ValueError("host_table must be a 2-D int32 CPU tensor")
    if not (dev_table.is_contiguous() and host_table.is_contiguous()):
        raise ValueError("tables must be contiguous")
    if row0 + n_rows > min(dev_table.shape[0], host_table.shape[0]):
        raise ValueError("rows outside the tables")
    check(lib.rc_upload_table_rows(_vp(dev_table), dev_table.shape[1], C.c_void_p(host_table.data_ptr()),
                                   host_table.shape[1], row0, n_rows, col0, col1, _stream(stream)))


def kv_store(shape: KVShape, k_pool, v_pool, k_new, v_new, slots, stream=None) -> None:
    """pool[slots[i]] = new[i] for K and V (see rc_kv_store)."""
    H, D, S = shape.num_kv_heads, shape.head_dim, shape.pool_slots
    _dev(k_pool, "k_pool", shape.dtype, (S, H, D))
    _dev(v_pool, "v_pool", shape.dtype, (S, H, D))
    n = slots.numel()
    _dev(k_new, "k_new", shape.dtype, (n, H, D))
    _dev(v_new, "v_new", shape.dtype, (n, H, D))
    _dev(slots, "slots", torch.int32)
    sh = shape.c()
    check(lib.rc_kv_store(C.byref(sh), _vp(k_pool), _vp(v_pool), _vp(k_new), _vp(v_new), _vp(slots), n, _stream(stream)))


def extend_attention(shape: KVShape, o, q, k_new, v_new, k_pool, v_pool, req_to_token, prefix_lens, extend_lens,
                     extend_start, max_extend: int, sm_scale: float, rows=None, stream=None) -> None:
    """Causal attention of each request's new tokens over its cached prefix plus themselves (rc_extend_attention)."""
    Hq, Hkv, D, S = shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.pool_slots
    T = q.shape[0]
    _dev(q, "q", shape.dtype, (T, Hq, D))
    _dev(o, "o", shape.dtype, (T, Hq, D))
    _dev(k_new, "k_new", shape.dtype, (T, Hkv, D))
    _dev(v_new, "v_new", shape.dtype, (T, Hkv, D))
    _dev(k_pool, "k_pool", shape.dtype, (S, Hkv, D))
    _dev(v_pool, "v_pool", shape.dtype, (S, Hkv, D))
    _dev(req_to_token, "req_to_token", torch.int32)
    if req_to_token.dim() != 2:
        raise ValueError("req_to_token must be [rows, stride]")
    B = prefix_lens.numel()
    for t, nm in ((prefix_lens, "prefix_lens"), (extend_lens, "extend_lens"), (extend_start, "extend_start")):
        _dev(t, nm, torch.int32, (B,))
    if rows is not None:
        _dev(rows, "rows", torch.int32, (B,))
    sh = shape.c()
    check(lib.rc_extend_attention(C.byref(sh), _vp(o), _vp(q), _vp(k_new), _vp(v_new), _vp(k_pool), _vp(v_pool),
                                  _vp(req_to_token), req_to_token.shape[0], req_to_token.shape[1], _vp(rows),
                                  _vp(prefix_lens), _vp(extend_lens), _vp(extend_start), B, T, int(max_extend),
                                  float(sm_scale), _stream(stream)))


def label_distribution(logits, label_ids, counts=None, vocab: Optional[int] = None, out=None, stream=None):
    """Stable softmax over each row's allowed label logits, the most probable option, the expected
    index and the confidence 1 - H/log k (rc_label_distribution).  logits: [rows, stride] fp32 or
    bf16 (rows may be a strided view with unit inner stride); label_ids: int32 [n_labels]; counts:
    int32 [rows] options per row or None.  Returns (probs [rows, n_labels], choice, expected,
    confidence), written into `out` when given."""
    if not isinstance(logits, torch.Tensor) or logits.device.type != "cuda" or logits.dim() != 2:
        raise ValueError("logits must be a 2-D GPU tensor")
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    dt = _DT.get(logits.dtype)
    if dt is None:
        raise TypeError(f"logits dtype {logits.dtype} not supported")
    R = logits.shape[0]
    L = label_ids.numel()
    _dev(label_ids, "label_ids", torch.int32, (L,))
    if counts is not None:
        _dev(counts, "counts", torch.int32, (R,))
    if out is None:
        dev = logits.device
        out = (torch.empty(R, L, dtype=torch.float32, device=dev), torch.empty(R, dtype=torch.int32, device=dev),
               torch.empty(R, dtype=torch.float32, device=dev), torch.empty(R, dtype=torch.float32, device=dev))
    probs, choice, expected, confidence = out
    _dev(probs, "probs", torch.float32, (R, L))
    _dev(choice, "choice", torch.int32, (R,))
    _dev(expected, "expected", torch.float32, (R,))
    _dev(confidence, "confidence", torch.float32, (R,))
    stride = logits.stride(0) if R > 1 else logits.shape[1]
    check(lib.rc_label_distribution(_vp(logits), dt, stride, int(vocab or logits.shape[1]), R, _vp(label_ids), L,
                                    _vp(counts), _vp(probs), _vp(choice), _vp(expected), _vp(confidence),
                                    _stream(stream)))
    return probs, choice, expected, confidence


class DecodePlan:
    """A decode work plan: the host int32 buffer, its summary, and a device copy."""

    def __init__(self, buf: np.ndarray, info: RcPlanInfo):
        self.host = buf
        self.info = info
        self.dev: Optional[torch.Tensor] = None
        self.seq_lens: Optional[np.ndarray] = None  # cascade extend plans: each new token's context length

    def to(self, device, uploader=None) -> "DecodePlan":
        """Device copy of the plan; `uploader(array) -> tensor` may supply an asynchronous copy."""
        self.dev = uploader(self.host) if uploader is not None else torch.from_numpy(self.host).to(device)
        return self

    @property
    def summary(self) -> dict:
        return {f: getattr(self.info, f) for f, _ in RcPlanInfo._fields_}

    def items(self) -> np.ndarray:
        n = self.info.n_items
        return self.host[N.RC_PLAN_HEADER:N.RC_PLAN_HEADER + n * N.RC_PLAN_ITEM].reshape(n, N.RC_PLAN_ITEM)

    def members(self) -> np.ndarray:
        o = N.RC_PLAN_HEADER + self.info.n_items * N.RC_PLAN_ITEM
        return self.host[o:o + self.info.n_members]

    def n_splits(self) -> np.ndarray:
        o = N.RC_PLAN_HEADER + self.info.n_items * N.RC_PLAN_ITEM + self.info.n_members
        return self.host[o:o + self.info.batch]


def _run_planner(call, guess: int = 0) -> DecodePlan:
    """Build a plan into a buffer of `guess` int32; when that is too small the
    planner reports the size it needs and runs once more."""
    info = RcPlanInfo()
    buf = np.empty(max(int(guess), 0), np.int32)
    st = call(_np_ptr(buf) if buf.size else None, buf.size, info)
    if st == N.RC_OK:
        return DecodePlan(buf[:info.plan_ints], info)
    if st != N.RC_ERR_RANGE or info.plan_ints <= buf.size:
        check(st)
    buf = np.empty(info.plan_ints, np.int32)
    check(call(_np_ptr(buf), buf.size, info))
    return DecodePlan(buf, info)


def _plan_guess(max_seq: np.ndarray, group: int, chunk: int) -> int:
    """Plan size for the usual case: every request's positions in chunks, a few
    shared node ranges per request, members about as many as items."""
    items = int(np.sum((max_seq.astype(np.int64) + chunk - 1) // chunk)) + 4 * max_seq.size
    return N.RC_PLAN_HEADER + items * (N.RC_PLAN_ITEM + 2) + max_seq.size


def plan_decode_unshared(max_seq_lens: Sequence[int], group: int, chunk: int = 512,
                         rows: Optional[Sequence[int]] = None) -> DecodePlan:
    ms = np.ascontiguousarray(max_seq_lens, np.int32)
    rw = None if rows is None else np.ascontiguousarray(rows, np.int32)
    return _run_planner(lambda p, cap, info: lib.rc_plan_decode_unshared(
        ms.size, _np_ptr(rw), _np_ptr(ms), group, chunk, p, cap, C.byref(info)), _plan_guess(ms, group, chunk))


def decode_steps(table: np.ndarray, rows: Sequence[int], base_lens: Sequence[int], n_steps: int, page_size: int = 1,
                 row_entries: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """(slots, seq_lens), both int32 [n_steps, batch]: the pool slot of request b's step-t token,
    at position base_lens[b] + t of host table row rows[b], and the number of positions it attends
    over (rc_decode_steps)."""
    if table.dtype != np.int32 or table.ndim != 2 or not table.flags.c_contiguous:
        raise ValueError("table must be a C-contiguous int32 [rows, stride] array")
    rw = np.ascontiguousarray(rows, np.int32)
    base = np.ascontiguousarray(base_lens, np.int32)
    re = None if row_entries is None else np.ascontiguousarray(row_entries, np.int64)
    if base.shape != rw.shape or (re is not None and re.shape != rw.shape):
        raise ValueError("one base length (and row entry count) per row")
    slots = np.zeros((n_steps, rw.size), np.int32)
    seq = np.zeros((n_steps, rw.size), np.int32)
    check(lib.rc_decode_steps(_np_ptr(table), table.shape[0], table.shape[1], page_size, rw.size, _np_ptr(rw),
                              _np_ptr(re), _np_ptr(base), n_steps, _np_ptr(slots), _np_ptr(seq)))
    return slots, seq


def decode_workspace_bytes(shape: KVShape, plan: DecodePlan) -> int:
    sh = shape.c()
    return int(lib.rc_decode_workspace_bytes(C.byref(sh), C.byref(plan.info)))


def decode_attention(shape: KVShape, o, q, k_pool, v_pool, req_to_token, seq_lens, plan: DecodePlan, sm_scale: float,
                     workspace, k_new=None, v_new=None, new_slots=None, stream=None) -> None:
    """One query token per request over its whole context, through a share plan (rc_decode_attention).
    With k_new/v_new/new_slots the current tokens' K/V are stored into the pool by the same call."""
    Hq, Hkv, D, S = shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.pool_slots
    B = q.shape[0]
    _dev(q, "q", shape.dtype, (B, Hq, D))
    _dev(o, "o", shape.dtype, (B, Hq, D))
    _dev(k_pool, "k_pool", shape.dtype, (S, Hkv, D))
    _dev(v_pool, "v_pool", shape.dtype, (S, Hkv, D))
    _dev(req_to_token, "req_to_token", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32, (B,))
    if (k_new is None) != (v_new is None) or (k_new is None) != (new_slots is None):
        raise ValueError("k_new, v_new and new_slots go together")
    if k_new is not None:
        _dev(k_new, "k_new", shape.dtype, (B, Hkv, D))
        _dev(v_new, "v_new", shape.dtype, (B, Hkv, D))
        _dev(new_slots, "new_slots", torch.int32, (B,))
    if plan.dev is None:
        raise ValueError("plan has no device copy; call plan.to(device)")
    _dev(workspace, "workspace")
    sh = shape.c()
    check(lib.rc_decode_attention(C.byref(sh), _vp(o), _vp(q), _vp(k_pool), _vp(v_pool), _vp(k_new), _vp(v_new),
                                  _vp(new_slots), _vp(req_to_token), req_to_token.shape[0], req_to_token.shape[1],
                                  _vp(seq_lens), B, _vp(plan.dev), C.byref(plan.info), float(sm_scale),
                                  _vp(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


class DecodeLauncher:
    """rc_decode_attention for the steps of one decode batch: the arguments that stay fixed over
    the steps (pools, table, plan, workspace, scale, stream) are checked once here, and each call
    checks only the step's own tensors, so a step costs little host time.  The stream is the one
    current at construction unless given."""

    def __init__(self, shape: KVShape, k_pool, v_pool, req_to_token, plan: DecodePlan, workspace, sm_scale: float,
                 batch: int, stream=None):
        Hq, Hkv, D, S = shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.pool_slots
        _dev(k_pool, "k_pool", shape.dtype, (S, Hkv, D))
        _dev(v_pool, "v_pool", shape.dtype, (S, Hkv, D))
        _dev(req_to_token, "req_to_token", torch.int32)
        _dev(workspace, "workspace")
        if plan.dev is None:
            raise ValueError("plan has no device copy; call plan.to(device)")
        if plan.info.batch != batch:
            raise ValueError(f"plan built for batch {plan.info.batch}, launcher for {batch}")
        self._sh = shape.c()
        self._info = plan.info
        self._dtype = shape.dtype
        self._q_shape = (batch, Hq, D)
        self._kv_shape = (batch, Hkv, D)
        self.batch = batch
        self._keep = (k_pool, v_pool, req_to_token, plan, workspace)  # alive while the launcher is
        self._pools = (k_pool.data_ptr(), v_pool.data_ptr())
        self._table = (req_to_token.data_ptr(), req_to_token.shape[0], req_to_token.shape[1])
        self._plan = plan.dev.data_ptr()
        self._ws = (workspace.data_ptr(), workspace.numel() * workspace.element_size())
        self._scale = float(sm_scale)
        self._stream = _stream(stream)

    def _check(self, t, name, dtype, shape):
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dtype and tuple(t.shape) == shape
                and t.is_contiguous()):
            raise ValueError(f"{name}: expected a contiguous device tensor {dtype} {shape}")

    def __call__(self, o, q, seq_lens_ptr: int, k_new=None, v_new=None, new_slots_ptr: Optional[int] = None) -> None:
        """o, q: [batch, Hq, D]; k_new/v_new: [batch, Hkv, D] or None; seq_lens_ptr / new_slots_ptr:
        device addresses of batch int32 each (the caller's tensors, kept alive by it)."""
        self._check(o, "o", self._dtype, self._q_shape)
        self._check(q, "q", self._dtype, self._q_shape)
        if (k_new is None) != (v_new is None) or (k_new is None) != (new_slots_ptr is None):
            raise ValueError("k_new, v_new and new_slots go together")
        kn = vn = None
        if k_new is not None:
            self._check(k_new, "k_new", self._dtype, self._kv_shape)
            self._check(v_new, "v_new", self._dtype, self._kv_shape)
            kn, vn = k_new.data_ptr(), v_new.data_ptr()
        check(lib.rc_decode_attention(C.byref(self._sh), o.data_ptr(), q.data_ptr(), self._pools[0], self._pools[1],
                                      kn, vn, new_slots_ptr, self._table[0], self._table[1], self._table[2],
                                      seq_lens_ptr, self.batch, self._plan, C.byref(self._info), self._scale,
                                      self._ws[0], self._ws[1], self._stream))


def decode_attention_static(shape: KVShape, o, q, k_pool, v_pool, req_to_token, seq_lens, plan: DecodePlan,
                            sm_scale: float, k_new=None, v_new=None, new_slots=None, stream=None) -> None:
    """decode_attention without a workspace (rc_decode_attention_static): the partials go to the
    library's static per-GPU workspace, so the call allocates nothing.  Calls that may overlap on
    one GPU race on that workspace."""
    Hq, Hkv, D, S = shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.pool_slots
    B = q.shape[0]
    _dev(q, "q", shape.dtype, (B, Hq, D))
    _dev(o, "o", shape.dtype, (B, Hq, D))
    _dev(k_pool, "k_pool", shape.dtype, (S, Hkv, D))
    _dev(v_pool, "v_pool", shape.dtype, (S, Hkv, D))
    _dev(req_to_token, "req_to_token", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32, (B,))
    if (k_new is None) != (v_new is None) or (k_new is None) != (new_slots is None):
        raise ValueError("k_new, v_new and new_slots go together")
    if k_new is not None:
        _dev(k_new, "k_new", shape.dtype, (B, Hkv, D))
        _dev(v_new, "v_new", shape.dtype, (B, Hkv, D))
        _dev(new_slots, "new_slots", torch.int32, (B,))
    if plan.dev is None:
        raise ValueError("plan has no device copy; call plan.to(device)")
    sh = shape.c()
    check(lib.rc_decode_attention_static(C.byref(sh), _vp(o), _vp(q), _vp(k_pool), _vp(v_pool), _vp(k_new),
                                         _vp(v_new), _vp(new_slots), _vp(req_to_token), req_to_token.shape[0],
                                         req_to_token.shape[1], _vp(seq_lens), B, _vp(plan.dev), C.byref(plan.info),
                                         float(sm_scale), _stream(stream)))


def extend_attention_shared(shape: KVShape, o, q, k_pool, v_pool, req_to_token, seq_lens, plan: DecodePlan,
                            sm_scale: float, workspace, stream=None) -> None:
    """Extend attention over a shared-prefix plan (rc_extend_attention_shared): row m of q/o is new
    token m of the batch; the new tokens' K/V must already be in the pool."""
    Hq, Hkv, D, S = shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.pool_slots
    T = q.shape[0]
    _dev(q, "q", shape.dtype, (T, Hq, D))
    _dev(o, "o", shape.dtype, (T, Hq, D))
    _dev(k_pool, "k_pool", shape.dtype, (S, Hkv, D))
    _dev(v_pool, "v_pool", shape.dtype, (S, Hkv, D))
    _dev(req_to_token, "req_to_token", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32, (T,))
    if plan.dev is None:
        raise ValueError("plan has no device copy; call plan.to(device)")
    _dev(workspace, "workspace")
    sh = shape.c()
    check(lib.rc_extend_attention_shared(C.byref(sh), _vp(o), _vp(q), _vp(k_pool), _vp(v_pool), _vp(req_to_token),
                                         req_to_token.shape[0], req_to_token.shape[1], _vp(seq_lens), T,
                                         _vp(plan.dev), C.byref(plan.info), float(sm_scale), _vp(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream)))


class TokenBatch:
    """A batch of token-id lists flattened once (CSR): request b owns
    flat[off[b]:off[b+1]].  Tree calls take it in place of a list of arrays, so
    one batch is flattened once for schedule, commit and plan."""

    def __init__(self, batch: Sequence[Sequence[int]]):
        lens = np.array([len(t) for t in batch], np.int64)
        self.off = np.zeros(len(batch) + 1, np.int64)
        np.cumsum(lens, out=self.off[1:])
        self.flat = np.empty(int(self.off[-1]), np.int32)
        for b, t in enumerate(batch):
            self.flat[self.off[b]:self.off[b + 1]] = t

    def __len__(self) -> int:
        return self.off.size - 1

    def lens(self) -> np.ndarray:
        return np.diff(self.off)

    def __getitem__(self, b: int) -> np.ndarray:
        return self.flat[self.off[b]:self.off[b + 1]]


def _tb(batch) -> TokenBatch:
    return batch if isinstance(batch, TokenBatch) else TokenBatch(batch)


def _lens(tb: TokenBatch, lengths) -> Optional[np.ndarray]:
    if lengths is None:
        return None
    ln = np.ascontiguousarray(lengths, np.int64)
    if ln.shape != (len(tb),):
        raise ValueError("one length per request")
    return ln


class RadixTree:
    """Host radix tree over token ids with the pool's slot allocator (rc_radix_*)."""

    def __init__(self, pool_slots: int, free_order: Optional[np.ndarray] = None, page_size: int = 1):
        """pool_slots: slots, or with page_size > 1 pages (of page_size slots) of the pool; the tree's
        slots are then page ids and it stores and shares whole pages (rc_radix_create_paged)."""
        self._h = C.c_void_p()
        fo = None if free_order is None else np.ascontiguousarray(free_order, np.int32)
        if fo is not None and fo.size != pool_slots:
            raise ValueError("free_order must have pool_slots entries")
        if page_size == 1:
            check(lib.rc_radix_create(pool_slots, _np_ptr(fo), C.byref(self._h)))
        else:
            check(lib.rc_radix_create_paged(pool_slots, page_size, _np_ptr(fo), C.byref(self._h)))
        self.pool_slots = pool_slots
        self.page_size = page_size

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and lib is not None:  # lib is gone at interpreter shutdown
            lib.rc_radix_destroy(h)
            self._h = None

    def match(self, tokens) -> Tuple[int, np.ndarray]:
        """(matched tokens, the matched slots, or page ids in a paged tree)."""
        t = np.ascontiguousarray(tokens, np.int32)
        out = np.zeros(max(t.size, 1), np.int32)
        m = C.c_int64()
        check(lib.rc_radix_match(self._h, _np_ptr(t), t.size, _np_ptr(out), C.byref(m)))
        return m.value, out[:m.value // self.page_size].copy()

    def alloc(self, n: int) -> np.ndarray:
        out = np.zeros(max(n, 1), np.int32)
        check(lib.rc_radix_alloc(self._h, n, _np_ptr(out)))
        return out[:n].copy()

    def free(self, slots) -> None:
        s = np.ascontiguousarray(slots, np.int32)
        check(lib.rc_radix_free(self._h, _np_ptr(s), s.size))

    def insert(self, tokens, slots) -> Tuple[np.ndarray, int]:
        """Store tokens with their slots (paged tree: their len(tokens) // page_size full pages with
        those pages' ids).  Returns (the slots now backing them, units newly stored)."""
        t = np.ascontiguousarray(tokens, np.int32)
        s = np.array(slots, np.int32, copy=True)
        if s.size != t.size // self.page_size:
            raise ValueError("need one slot per token (one page id per full page in a paged tree)")
        n_new = C.c_int64()
        check(lib.rc_radix_insert(self._h, _np_ptr(t), _np_ptr(s), t.size, C.byref(n_new)))
        return s, n_new.value

    def emit_rows(self, batch: Sequence[Sequence[int]], table: np.ndarray, rows: Optional[Sequence[int]] = None,
                  reserve: int = 0, evict: bool = False, handles: Optional[np.ndarray] = None,
                  first_changed: Optional[np.ndarray] = None, full_match: bool = False,
                  row_entries: Optional[np.ndarray] = None,
                  new_slots: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
        """Fill rows of a host table [R, stride]; returns (prefix_lens, extend_lens).
        evict: evict least recently used unpinned nodes when the free slots fall short.
        full_match: do not cap the match at n - 1 tokens (storing K/V computed elsewhere).
        handles: an int64 array of one entry per request that receives locks on the matched prefixes.
        first_changed: an int64 array of one entry per request that receives the first entry of its
        row the call changed (the row's entry count if none).
        row_entries: an int64 array of one entry per request that receives the entries its row uses.
        new_slots: an int32 array with room for every token of the batch; its first sum(extend_lens)
        entries receive the new tokens' pool slots, request after request."""
        if table.dtype != np.int32 or table.ndim != 2 or not table.flags.c_contiguous:
            raise ValueError("table must be a C-contiguous int32 [rows, stride] array")
        tb = _tb(batch)
        B = len(tb)
        rw = np.arange(B, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, np.int32)
        P = np.zeros(B, np.int32)
        E = np.zeros(B, np.int32)
        for arr, nm in ((handles, "handles"), (first_changed, "first_changed"), (row_entries, "row_entries")):
            if arr is not None and (arr.dtype != np.int64 or arr.shape != (B,) or not arr.flags.c_contiguous):
                raise ValueError(f"{nm} must be a contiguous int64 array with one entry per request")
        if new_slots is not None and (new_slots.dtype != np.int32 or new_slots.ndim != 1 or new_slots.size < tb.flat.size
                                      or not new_slots.flags.c_contiguous):
            raise ValueError("new_slots must be a contiguous int32 array with room for every token of the batch")
        flags = (N.RC_EMIT_EVICT if evict else 0) | (N.RC_EMIT_FULL_MATCH if full_match else 0)
        check(lib.rc_radix_emit_rows(self._h, B, _np_ptr(tb.flat), _np_ptr(tb.off), reserve, _np_ptr(rw), _np_ptr(table),
                                     table.shape[0], table.shape[1], _np_ptr(P), _np_ptr(E), flags,
                                     _np_ptr(handles), _np_ptr(first_changed), _np_ptr(row_entries), _np_ptr(new_slots)))
        return P, E

    def free_rows(self, rows: Sequence[int], table: np.ndarray, keep_lens: Sequence[int],
                  row_entries: Sequence[int]) -> None:
        """Return each row's units from the first position not kept (keep_lens, tokens) to its end
        (row_entries, as emit_rows reported them) to the pool (rc_radix_free_rows)."""
        if table.dtype != np.int32 or table.ndim != 2 or not table.flags.c_contiguous:
            raise ValueError("table must be a C-contiguous int32 [rows, stride] array")
        rw = np.ascontiguousarray(rows, np.int32)
        kp = np.ascontiguousarray(keep_lens, np.int64)
        re = np.ascontiguousarray(row_entries, np.int64)
        if kp.shape != rw.shape or re.shape != rw.shape:
            raise ValueError("one keep length and one row entry count per row")
        check(lib.rc_radix_free_rows(self._h, rw.size, _np_ptr(rw), _np_ptr(table), table.shape[0], table.shape[1],
                                     _np_ptr(kp), _np_ptr(re)))

    def lock(self, batch, lengths: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
        """Pin the cached prefix of each request's first lengths[b] tokens (default: all) against
        eviction.  Returns (handles int64, locked lengths)."""
        tb = _tb(batch)
        ln = _lens(tb, lengths)
        B = len(tb)
        h = np.zeros(B, np.int64)
        m = np.zeros(B, np.int64)
        check(lib.rc_radix_lock(self._h, B, _np_ptr(tb.flat), _np_ptr(tb.off), _np_ptr(ln), _np_ptr(h), _np_ptr(m)))
        return h, m

    def unlock(self, handles) -> None:
        h = np.ascontiguousarray(handles, np.int64)
        check(lib.rc_radix_unlock(self._h, _np_ptr(h), h.size))

    def evict(self, n_slots: int) -> int:
        """Evict least recently used unpinned leaves until n_slots slots are freed; returns the number freed."""
        got = C.c_int64()
        check(lib.rc_radix_evict(self._h, int(n_slots), C.byref(got)))
        return got.value

    def insert_rows(self, batch: Sequence[Sequence[int]], table: np.ndarray, rows: Sequence[int],
                    lengths: Optional[Sequence[int]] = None) -> np.ndarray:
        """Insert each request's first lengths[i] tokens (default: all) with the slots of its table
        row; rows are rewritten in place to the tree's slots.  Returns a bool mask of changed rows."""
        if table.dtype != np.int32 or table.ndim != 2 or not table.flags.c_contiguous:
            raise ValueError("table must be a C-contiguous int32 [rows, stride] array")
        tb = _tb(batch)
        ln = _lens(tb, lengths)
        rw = np.ascontiguousarray(rows, np.int32)
        changed = np.zeros(len(tb), np.int32)
        check(lib.rc_radix_insert_rows(self._h, len(tb), _np_ptr(tb.flat), _np_ptr(tb.off), _np_ptr(ln), _np_ptr(rw),
                                       _np_ptr(table), table.shape[0], table.shape[1], _np_ptr(changed)))
        return changed.astype(bool)

    def fork(self, tokens, parent_slots, child_rows: Sequence[int], table: np.ndarray) -> None:
        t = np.ascontiguousarray(tokens, np.int32)
        s = np.ascontiguousarray(parent_slots, np.int32)
        cr = np.ascontiguousarray(child_rows, np.int32)
        check(lib.rc_radix_fork(self._h, _np_ptr(t), _np_ptr(s), t.size, cr.size, _np_ptr(cr), _np_ptr(table),
                                table.shape[0], table.shape[1]))

    def plan_decode(self, batch, max_seq_lens: Sequence[int], group: int, chunk: int = 512,
                    rows: Optional[Sequence[int]] = None, lengths: Optional[Sequence[int]] = None) -> DecodePlan:
        """Shared decode plan; request b's first lengths[b] tokens (default: all) are walked."""
        tb = _tb(batch)
        ln = _lens(tb, lengths)
        B = len(tb)
        rw = np.arange(B, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, np.int32)
        ms = np.ascontiguousarray(max_seq_lens, np.int32)
        return _run_planner(lambda p, cap, info: lib.rc_radix_plan_decode(
            self._h, B, _np_ptr(tb.flat), _np_ptr(tb.off), _np_ptr(ln), _np_ptr(rw), _np_ptr(ms), group, chunk, p, cap,
            C.byref(info)), _plan_guess(ms, group, chunk))

    def plan_extend(self, batch, prefix_lens: Sequence[int], extend_lens: Sequence[int], group: int,
                    chunk: int = 4096, rows: Optional[Sequence[int]] = None) -> DecodePlan:
        """Cascade extend plan: members are the batch's new tokens (rc_radix_plan_extend).  The plan's
        seq_lens holds each new token's context length (the seq_lens of extend_attention_shared)."""
        tb = _tb(batch)
        B = len(tb)
        P = np.ascontiguousarray(prefix_lens, np.int32)
        E = np.ascontiguousarray(extend_lens, np.int32)
        if P.shape != (B,) or E.shape != (B,):
            raise ValueError("one prefix and one extend length per request")
        rw = np.arange(B, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, np.int32)
        seq = np.zeros(int(E.sum()), np.int32)
        # buffer guess: every new token reads its request's context in pieces of chunk, plus a few shared ranges
        n_tok = int(E.sum())
        longest = int((P.astype(np.int64) + E).max()) if B else 0
        guess = N.RC_PLAN_HEADER + n_tok * (longest // max(chunk, 1) + 4) * (N.RC_PLAN_ITEM + 2) + n_tok
        plan = _run_planner(lambda p, cap, info: lib.rc_radix_plan_extend(
            self._h, B, _np_ptr(tb.flat), _np_ptr(tb.off), _np_ptr(P), _np_ptr(E), _np_ptr(rw), group, chunk, p, cap,
            C.byref(info), _np_ptr(seq)), guess)
        plan.seq_lens = seq
        return plan

    def stats(self) -> dict:
        st = RcRadixStats()
        check(lib.rc_radix_stats_get(self._h, C.byref(st)))
        return {f: getattr(st, f) for f, _ in RcRadixStats._fields_}


def prof_enable(on: bool = True) -> None:
    check(lib.rc_prof_enable(1 if on else 0))


def prof_tag(tag: Optional[str]) -> None:
    """Report the following launches as '<kernel>@<tag>' (None: plain names)."""
    check(lib.rc_prof_tag(tag.encode() if tag else None))


def prof_collect() -> dict:
    """{kernel name: (launches, total ms)} since the last collect; waits for the recorded events."""
    cap = 64
    arr = (RcProfEntry * cap)()
    n = C.c_int32()
    check(lib.rc_prof_collect(arr, cap, C.byref(n)))
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(min(n.value, cap))}


def version() -> str:
    return lib.rc_version().decode()
