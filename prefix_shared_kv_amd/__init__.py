"""Attention over a prefix-shared (radix) KV pool for AMD Instinct MI355X (gfx950).

GPU calls: kv_store, extend_attention, decode_attention (hand-written HIP
kernels in librcattn.so).  Host calls: RadixTree (C++ radix tree, slot
allocator, table rows, decode share plans).  See include/rc.h for the C ABI.
"""
from .api import (DecodePlan, KVShape, RadixTree, decode_attention, decode_workspace_bytes,  # noqa: F401
                  extend_attention, kv_store, plan_decode_unshared, prof_collect, prof_enable, prof_tag, set_error_word,
                  set_tuning, TokenBatch, version)
from ._native import RcError  # noqa: F401
