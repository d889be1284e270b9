"""The C-ABI library on the CPU: it loads, exports every symbol include/rswa.h declares, and its
host-only paths (layout planning, validation, status strings) behave as documented. No call here
reaches the GPU."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rswa.h")
LIB = os.path.join(ROOT, "windowed_attention_amd", "librswa.so")


@pytest.fixture(scope="module")
def wa():
    if not os.path.exists(LIB):  # build once if nothing is built yet (without importing the
        import importlib.util    # package, which needs the library)
        spec = importlib.util.spec_from_file_location(
            "windowed_attention_amd_build", os.path.join(ROOT, "windowed_attention_amd", "_build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import windowed_attention_amd
    return windowed_attention_amd


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rswa_\w+)\s*\(", text)))


def test_exports_every_header_symbol(wa):
    names = header_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(LIB)
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(wa.EXPORTS) == names


def test_library_holds_gfx950_code_only():
    data = open(LIB, "rb").read()
    assert b"gfx950" in data
    for other in (b"amdgcn-amd-amdhsa--gfx942", b"amdgcn-amd-amdhsa--gfx90a"):
        assert other not in data


def test_status_strings(wa):
    for code, name in wa.STATUS.items():
        assert wa.status_str(code) == name
    assert wa.status_str(-99) == "RSWA_E_UNKNOWN"


def test_plan_layout_matches_row_counts(wa):
    m = [272, 0, 5155]
    n = [128, 5, 64]
    off, rows, nbytes = wa.rswa_cache_plan(m, n, num_heads=16, kv_dtype=torch.bfloat16)
    np.testing.assert_array_equal(rows, [400, 5, 5219])
    per_seq = 2 * 16 * rows.astype(np.int64) * 128  # K and V, elements
    np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(per_seq)[:-1]]))
    assert nbytes == int(per_seq.sum()) * 2 + 4096  # plus the tail the decode tiles may read
    # batched single-page decode: 64 sequences x (272 + 128) rows x 16 heads x 128 x K,V x bf16
    assert wa.rswa_cache_bytes([272] * 64, [128] * 64) == 64 * 400 * 16 * 128 * 2 * 2 + 4096
    # full causal: m + max_steps rows, fp32
    _, rows, nbytes = wa.rswa_cache_plan([7], None, [20], mode=wa.MODE_FULL_CAUSAL,
                                         num_heads=2, kv_dtype=torch.float32)
    assert rows.tolist() == [27] and nbytes == 2 * 2 * 27 * 128 * 4 + 4096


@pytest.mark.parametrize("kw,status", [
    (dict(prefix_len=[1], window=[0]), -1),
    (dict(prefix_len=[-1], window=[4]), -1),
    (dict(prefix_len=[4], window=[4], head_dim=64), -2),
    (dict(prefix_len=[4], window=[4], head_dim=0), -1),
    (dict(prefix_len=[4], window=[4], num_heads=0), -1),
    (dict(prefix_len=[4], window=None), -1),
    (dict(prefix_len=[4], window=[4], max_steps=None, mode=1), -1),
    (dict(prefix_len=[4], window=None, max_steps=[0], mode=1), -1),
    (dict(prefix_len=[4], window=[4], mode=7), -1),
])
def test_plan_rejects_invalid_descriptions(wa, kw, status):
    kw = dict(kw)
    args = (kw.pop("prefix_len"), kw.pop("window"), kw.pop("max_steps", None))
    with pytest.raises(wa.RswaError) as e:
        wa.rswa_cache_plan(*args, **kw)
    assert e.value.status == status
    assert wa.rswa_cache_bytes(*args, **kw) == 0


def test_null_arguments_are_rejected_before_any_device_work(wa):
    lib = wa._lib
    null = ctypes.c_void_p(None)
    assert lib.rswa_append_kv(null, null, null, null, null) == -1
    assert lib.rswa_decode_attn(null, null, null, 1, 0.0, null, null) == -1
    assert lib.rswa_cache_steps(null, None, null) == -1
    assert lib.rswa_cache_info(null, None, None, None) == -1
    assert lib.rswa_cache_set_decode_split(null, 64, 0) == -1
    assert lib.rswa_cache_destroy(null) == 0
    h = ctypes.c_void_p(None)
    assert lib.rswa_cache_create(None, null, null, null, ctypes.byref(h)) == -1
    assert h.value is None
    assert b"NULL" in lib.rswa_last_error() or b"null" in lib.rswa_last_error()
    # prefill: null pointers, bad head_dim, bad dtype
    one = ctypes.c_void_p(16)
    assert lib.rswa_prefill_attn(null, one, one, one, 1, one, one, one, 1, 16, 128, 8, 0, 0.0,
                                 null) == -1
    assert lib.rswa_prefill_attn(one, one, one, one, 1, one, one, one, 1, 16, 64, 8, 0, 0.0,
                                 null) == -2
    assert lib.rswa_prefill_attn(one, one, one, one, 3, one, one, one, 1, 16, 128, 8, 0, 0.0,
                                 null) == -1
    assert lib.rswa_prefill_attn(one, one, one, one, 1, one, one, one, 0, 16, 128, 8, 0, 0.0,
                                 null) == -1


def test_training_entry_points_reject_bad_arguments_before_any_device_work(wa):
    lib = wa._lib
    null, one = ctypes.c_void_p(None), ctypes.c_void_p(16)
    # forward with log-sum-exp: NULL lse, bad head_dim
    assert lib.rswa_prefill_fwd(one, one, one, one, 1, null, one, one, one, 1, 16, 128, 8, 0,
                                0.0, null) == -1
    assert lib.rswa_prefill_fwd(one, one, one, one, 1, one, one, one, one, 1, 16, 64, 8, 0,
                                0.0, null) == -2
    # backward: each gradient-side pointer NULL in turn, then a bad grad dtype and token count
    args = [one, one, one, one, 1, one, one, one, one, one, one, 1, one, one, one,
            1, 8, 16, 128, 8, 0, 0.0, null]
    for i in (5, 6, 7, 8, 9, 10):
        bad = list(args)
        bad[i] = null
        assert lib.rswa_prefill_bwd(*bad) == -1, i
    bad = list(args)
    bad[11] = 7
    assert lib.rswa_prefill_bwd(*bad) == -1
    bad = list(args)
    bad[16] = -1
    assert lib.rswa_prefill_bwd(*bad) == -1
    bad = list(args)
    bad[18] = 96
    assert lib.rswa_prefill_bwd(*bad) == -2
    assert b"head_dim" in lib.rswa_last_error()


def test_paged_plan_stores_only_output_rows(wa):
    m, n = np.array([300, 150, 0, 40]), np.array([32, 16, 8, 64])
    _, rows_c, bytes_c = wa.rswa_cache_plan(m, n)
    _, rows_p, bytes_p = wa.rswa_cache_plan(m, n, paged=True)
    np.testing.assert_array_equal(rows_c, m + n)
    np.testing.assert_array_equal(rows_p, n)
    assert bytes_p == 2 * 16 * 128 * 2 * int(n.sum()) + 4096
    assert bytes_c - bytes_p == 2 * 16 * 128 * 2 * int(m.sum())


def test_paged_create_checks_arguments_before_device_work(wa):
    lib = wa._lib
    null, one = ctypes.c_void_p(None), ctypes.c_void_p(16)
    d, keep = wa._desc(np.array([5, 3]), np.array([4, 4]), None, 16, 128, wa.torch.bfloat16,
                       wa.MODE_RSWA, paged=True)
    h = ctypes.c_void_p(None)
    # NULL pool / table with m > 0
    assert lib.rswa_cache_create_paged(ctypes.byref(d), null, one, 10, one, null,
                                       ctypes.byref(h)) == -1
    assert lib.rswa_cache_create_paged(ctypes.byref(d), one, one, 10, null, null,
                                       ctypes.byref(h)) == -1
    assert lib.rswa_cache_create_paged(ctypes.byref(d), one, one, 0, one, null,
                                       ctypes.byref(h)) == -1
    # a paged description given to the copying entry point, and the reverse
    assert lib.rswa_cache_create(ctypes.byref(d), one, one, null, ctypes.byref(h)) == -1
    assert b"prefix_paged" in lib.rswa_last_error()
    d.prefix_paged = 0
    assert lib.rswa_cache_create_paged(ctypes.byref(d), one, one, 10, one, null,
                                       ctypes.byref(h)) == -1
    d.prefix_paged = 2
    assert lib.rswa_cache_create(ctypes.byref(d), one, one, null, ctypes.byref(h)) == -1
    assert h.value is None


def test_prefill_fill_checks_arguments_before_device_work(wa):
    lib = wa._lib
    null, one = ctypes.c_void_p(None), ctypes.c_void_p(16)
    i32p = ctypes.POINTER(ctypes.c_int32)

    def create(d, k, v, cu):
        h = ctypes.c_void_p(None)
        arr = None if cu is None else np.asarray(cu, dtype=np.int32)
        st = lib.rswa_cache_create_from_prefill(
            ctypes.byref(d), k, v, None if arr is None else arr.ctypes.data_as(i32p), null,
            ctypes.byref(h))
        assert h.value is None
        return st

    d, keep = wa._desc(np.array([5, 3]), np.array([4, 4]), None, 16, 128, wa.torch.bfloat16,
                       wa.MODE_RSWA)
    assert create(d, one, one, None) == -1                 # no cu_seqlens
    assert create(d, one, one, [-1, 6, 10]) == -1          # negative start
    assert create(d, one, one, [0, 4, 10]) == -1           # segment 0 shorter than m_0 = 5
    assert b"shorter than its prefix" in lib.rswa_last_error()
    assert create(d, one, one, [0, 9, 8]) == -1            # decreasing offsets
    assert create(d, null, one, [0, 9, 15]) == -1          # rows but no K
    assert create(d, ctypes.c_void_p(8), one, [0, 9, 15]) == -1  # misaligned K
    d.prefix_paged = 1
    assert create(d, one, one, [0, 9, 15]) == -1
    assert b"prefix_paged" in lib.rswa_last_error()
    # full causal: a segment with more outputs than max_steps
    d, keep = wa._desc(np.array([5, 3]), None, np.array([4, 4]), 16, 128, wa.torch.bfloat16,
                       wa.MODE_FULL_CAUSAL)
    assert create(d, one, one, [0, 10, 15]) == -3
    assert b"max_steps" in lib.rswa_last_error()


def test_prefill_fill_binding_checks_the_row_count(wa):
    # the C call cannot see the size of k / v; the binding checks cu_seqlens against it first
    k = torch.zeros((10, 16, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="holds 10 rows"):
        wa.rswa_cache_create_from_prefill(k, k, [0, 6, 11], [4, 2], [8, 8])
    with pytest.raises(ValueError, match="3 entries"):
        wa.rswa_cache_create_from_prefill(k, k, [0, 6], [4, 2], [8, 8])


def test_prefill_binding_checks_sequences_fit_the_rows(wa):
    q = torch.zeros((10, 16, 128), dtype=torch.bfloat16)
    cu = torch.tensor([0, 6, 12], dtype=torch.int32)
    m = torch.tensor([2, 2], dtype=torch.int32)
    n = torch.tensor([4, 4], dtype=torch.int32)
    for fn in (wa.rswa_prefill_attn, wa.rswa_prefill_fwd):
        with pytest.raises(ValueError, match="hold 10 rows"):
            fn(q, q, q, cu, m, n)


def test_step_graph_arguments_are_checked_before_device_work(wa):
    lib = wa._lib
    null, one = ctypes.c_void_p(None), ctypes.c_void_p(16)
    h = ctypes.c_void_p(None)
    f = ctypes.c_float(0.0)
    assert lib.rswa_step_graph_create(null, 2, one, one, one, one, 1, f, ctypes.byref(h)) == -1
    assert lib.rswa_step_graph_create(one, 2, one, one, one, one, 1, f, None) == -1
    assert lib.rswa_step_graph_launch(null, null) == -1
    assert lib.rswa_step_graph_destroy(null) == 0
    assert h.value is None
