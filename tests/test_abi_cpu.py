"""The C ABI on the CPU: the library loads, exports every function rc.h
declares, and rejects bad arguments with the documented status before
launching anything (so no GPU is needed)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from prefix_shared_kv_amd import _native as N

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "rc.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rc_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(N.lib, n), n
    assert set(names) == set(N._SIGS), "binding and header disagree"


def test_version():
    assert "gfx950" in N.lib.rc_version().decode()


def shape(dtype=N.RC_BF16, hq=8, hkv=2, d=128, slots=16):
    return N.RcShape(dtype, hq, hkv, d, slots)


FAKE = C.c_void_p(0x1000)  # never dereferenced: validation fails first, or n == 0


@pytest.mark.parametrize("sh,code", [
    (shape(dtype=7), N.RC_ERR_DTYPE),
    (shape(d=96), N.RC_ERR_SHAPE),
    (shape(hq=6, hkv=4), N.RC_ERR_SHAPE),
    (shape(hq=0), N.RC_ERR_SHAPE),
    (shape(hq=512, hkv=2), N.RC_ERR_SHAPE),
])
def test_kv_store_rejects_bad_shapes(sh, code):
    st = N.lib.rc_kv_store(C.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 4, None)
    assert st == code
    assert N.last_error()


def test_kv_store_argument_checks():
    sh = shape()
    assert N.lib.rc_kv_store(None, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None) == N.RC_ERR_ARG
    assert N.lib.rc_kv_store(C.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, -1, None) == N.RC_ERR_ARG
    assert N.lib.rc_kv_store(C.byref(sh), None, FAKE, FAKE, FAKE, FAKE, 4, None) == N.RC_ERR_ARG
    assert N.lib.rc_kv_store(C.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == N.RC_OK  # nothing to do


def test_extend_argument_checks():
    sh = shape()
    args = [C.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, None, FAKE, FAKE, FAKE]
    assert N.lib.rc_extend_attention(*args, -1, 10, 8, 0.1, None) == N.RC_ERR_ARG
    assert N.lib.rc_extend_attention(*args, 2, 10, 8, float("nan"), None) == N.RC_ERR_ARG
    # the softmax scale must be positive: the kernels scale each column's
    # maximum after taking it, and masked keys carry -inf scores
    for bad_scale in (0.0, -0.125, -0.0, float("inf"), float("-inf")):
        assert N.lib.rc_extend_attention(*args, 2, 10, 8, bad_scale, None) == N.RC_ERR_ARG
        assert "sm_scale" in N.last_error()
    assert N.lib.rc_extend_attention(*args, 0, 0, 0, 0.1, None) == N.RC_OK
    bad = list(args)
    bad[1] = None
    assert N.lib.rc_extend_attention(*bad, 2, 10, 8, 0.1, None) == N.RC_ERR_ARG
    bad = list(args)
    bad[9] = 0  # stride
    assert N.lib.rc_extend_attention(*bad, 2, 10, 8, 0.1, None) == N.RC_ERR_ARG


def _plan(max_seq, group, chunk=64):
    info = N.RcPlanInfo()
    ms = np.ascontiguousarray(max_seq, np.int32)
    st = N.lib.rc_plan_decode_unshared(ms.size, None, ms.ctypes.data_as(C.c_void_p), group, chunk, None, 0, C.byref(info))
    assert st == N.RC_ERR_RANGE and info.plan_ints > 0
    buf = np.zeros(info.plan_ints, np.int32)
    N.check(N.lib.rc_plan_decode_unshared(ms.size, None, ms.ctypes.data_as(C.c_void_p), group, chunk,
                                          buf.ctypes.data_as(C.c_void_p), buf.size, C.byref(info)))
    return buf, info


def test_decode_argument_checks():
    sh = shape()  # group 4
    buf, info = _plan([100, 70], 4)
    need = N.lib.rc_decode_workspace_bytes(C.byref(sh), C.byref(info))
    # bf16 partial rows (128 x 2 bytes) and fp32 (max, sum) pairs; fp32 data keeps fp32 rows
    assert need == 2 * 8 * info.max_splits * (128 * 2 + 2 * 4)
    assert N.lib.rc_decode_workspace_bytes(C.byref(shape(dtype=N.RC_F32)), C.byref(info)) == \
        2 * 8 * info.max_splits * (128 * 4 + 2 * 4)

    def call(sh_, batch, ws):
        return N.lib.rc_decode_attention(C.byref(sh_), FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, 2, 128, FAKE,
                                         batch, FAKE, C.byref(info), 0.1, FAKE, ws, None)

    assert call(sh, 2, need - 1) == N.RC_ERR_RANGE
    assert call(sh, 3, need) == N.RC_ERR_ARG  # plan built for batch 2
    assert call(shape(hq=8, hkv=8), 2, need) == N.RC_ERR_SHAPE  # plan built for group 4
    assert call(sh, 0, need) == N.RC_OK
    for bad_scale in (0.0, -1.0, float("nan")):
        st = N.lib.rc_decode_attention(C.byref(sh), FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, 2, 128, FAKE,
                                       2, FAKE, C.byref(info), bad_scale, FAKE, need, None)
        assert st == N.RC_ERR_ARG
        st = N.lib.rc_extend_attention_shared(C.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 2, 128, FAKE, 2, FAKE,
                                              C.byref(info), bad_scale, FAKE, need, None)
        assert st == N.RC_ERR_ARG
    # the current token's K/V come as a triple
    st = N.lib.rc_decode_attention(C.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 2, 128, FAKE, 2, FAKE,
                                   C.byref(info), 0.1, FAKE, need, None)
    assert st == N.RC_ERR_ARG


def test_plan_columns_are_checked_against_the_launch():
    # a cascade extend plan fills eight-wave tiles (256 columns per item); the
    # decode launch runs four-wave tiles and rejects it before touching the
    # device, while the cascade launch accepts both kinds of plan
    from prefix_shared_kv_amd import RadixTree
    sh = shape()  # group 4
    t = RadixTree(4096)
    doc = np.arange(100, 400, dtype=np.int32)
    batch = [np.concatenate([doc, np.arange(1000 + 40 * k, 1000 + 40 * k + 40, dtype=np.int32)]) for k in range(2)]
    table = np.full((2, 400), -1, np.int32)
    t.emit_rows([doc], table[:1])
    t.insert_rows([doc], table[:1], np.zeros(1, np.int32))
    P, E = t.emit_rows(batch, table)
    plan = t.plan_extend(batch, P, E, 4, 4096)
    info = plan.info
    assert info.max_cols == N.RC_EXTEND_SHARED_COLS > N.RC_DECODE_COLS
    need = N.lib.rc_decode_workspace_bytes(C.byref(sh), C.byref(info))
    st = N.lib.rc_decode_attention(C.byref(sh), FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, 2, 400, FAKE,
                                   info.batch, FAKE, C.byref(info), 0.1, FAKE, need, None)
    assert st == N.RC_ERR_ARG and "plan summary" in N.last_error()
    _, dinfo = _plan([100, 70], 4)
    assert dinfo.max_cols == N.RC_DECODE_COLS


def test_static_decode_argument_checks():
    # the allocation-free decode rejects a plan whose workspace exceeds the
    # static one before it touches the device
    sh = shape()  # group 4, Hq 8, head_dim 128
    buf, info = _plan([640] * 4096, 4)  # 4096 x 8 heads x 9 splits x (256 + 8) B = 77.9 MB
    need = N.lib.rc_decode_workspace_bytes(C.byref(sh), C.byref(info))
    assert need > N.RC_DECODE_STATIC_WORKSPACE_BYTES
    call = N.lib.rc_decode_attention_static
    st = call(C.byref(sh), FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, 4096, 640, FAKE, 4096, FAKE,
              C.byref(info), 0.1, None)
    assert st == N.RC_ERR_RANGE and "static workspace" in N.last_error()
    assert call(None, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, 2, 128, FAKE, 2, FAKE, C.byref(info), 0.1,
                None) == N.RC_ERR_ARG


def test_unshared_plan_layout():
    # chunk 64: ranges up to 72 (chunk + chunk/8) stay whole, longer ones are
    # cut into the fewest near-equal pieces of at most 72
    buf, info = _plan([100, 70, 1, 200], 4, chunk=64)
    assert buf[0] == N.RC_PLAN_MAGIC
    assert info.n_items == 2 + 1 + 1 + 3
    assert info.max_splits == 3
    items = buf[8:8 + 8 * info.n_items].reshape(-1, 8)
    cover = {}
    for rep, pb, pe, sp, mo, mc, flags, _ in items:
        assert mc == 1 and flags == N.RC_PLAN_ITEM_OWN  # no sharing: every item is its request's own
        b = buf[8 + 8 * info.n_items + mo]
        cover.setdefault(int(b), []).append((int(pb), int(pe), int(sp)))
    assert sorted(cover[0]) == [(0, 50, 0), (50, 100, 1)]
    assert sorted(cover[1]) == [(0, 70, 0)]
    assert sorted(cover[2]) == [(0, 1, 0)]
    assert sorted(cover[3]) == [(0, 67, 0), (67, 134, 1), (134, 200, 2)]
    nsplit = buf[8 + 8 * info.n_items + info.n_members:]
    assert nsplit.tolist() == [2, 1, 1, 3]


def test_error_text_is_thread_local_and_set():
    sh = shape(d=96)
    N.lib.rc_kv_store(C.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 4, None)
    assert "head_dim" in N.last_error()


def test_table_upload_argument_checks():
    up = N.lib.rc_upload_table_rows
    # (dev, dev_stride, host, host_stride, row0, n_rows, col0, col1, stream)
    assert up(FAKE, 8, FAKE, 8, 0, 0, 0, 8, None) == N.RC_OK      # no rows: nothing to copy
    assert up(FAKE, 8, FAKE, 8, 0, 4, 3, 3, None) == N.RC_OK      # empty column range
    assert up(FAKE, 8, FAKE, 8, 0, 4, 0, 9, None) == N.RC_ERR_ARG  # past the device row
    assert up(FAKE, 16, FAKE, 8, 0, 4, 0, 9, None) == N.RC_ERR_ARG  # past the host row
    assert up(FAKE, 8, FAKE, 8, 0, 4, 5, 4, None) == N.RC_ERR_ARG  # reversed columns
    assert up(FAKE, 8, FAKE, 8, -1, 4, 0, 8, None) == N.RC_ERR_ARG
    assert up(FAKE, 8, FAKE, 8, 0, -1, 0, 8, None) == N.RC_ERR_ARG
    assert up(None, 8, FAKE, 8, 0, 4, 0, 8, None) == N.RC_ERR_ARG
    assert "rectangle" in N.last_error() or "NULL" in N.last_error()


def test_sanitized_build_is_the_one_loaded_when_asked():
    # RC_SANITIZED=1 runs the CPU tests against the build with AddressSanitizer and
    # UndefinedBehaviorSanitizer on its host code; make sure that library is the one in use
    if os.environ.get("RC_SANITIZED") != "1":
        pytest.skip("plain build")
    assert N.LIB_PATH.endswith("librcattn_san.so")
    assert "librcattn_san.so" in open("/proc/self/maps").read()
