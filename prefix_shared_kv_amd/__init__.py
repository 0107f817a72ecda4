"""Attention over a prefix-shared (radix) KV pool for AMD Instinct MI355X (gfx950).

GPU calls: kv_store, extend_attention, extend_attention_shared, decode_attention,
label_distribution (hand-written HIP kernels in librcattn.so).  Host calls: RadixTree (C++ radix
tree, slot allocator, table rows, decode and shared-prefix extend plans).  See
include/rc.h for the C ABI.
"""
from .api import (DecodePlan, KVShape, RadixTree, TokenBatch, decode_attention, decode_attention_static,  # noqa: F401
                  decode_steps, decode_workspace_bytes, extend_attention, extend_attention_shared, kv_store, label_distribution,
                  plan_decode_unshared, prof_collect, prof_enable, prof_tag, set_error_word, version)
from ._native import RcError  # noqa: F401
