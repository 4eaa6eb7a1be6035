"""The C ABI without a GPU: the library loads, exports every declared entry
point, sizes workspaces, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import block_sparse_kv_amd as mage

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "mage.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mage_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = mage.lib()
    names = declared_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name


def test_hip_library_is_separate_from_the_oracle():
    # the product library must not link or embed the oracle
    data = open(mage.LIB_PATH, "rb").read()
    assert b"oracle_" not in data


def test_status_strings():
    lib = mage.lib()
    for st in range(5):
        assert lib.mage_status_string(st)


def dims(**kw):
    d = dict(num_seqs=1, block=32, num_q_heads=32, num_kv_heads=8, head_dim=128, scale=1.0)
    d.update(kw)
    return mage.Dims(**d)


def test_workspace_bytes():
    small = mage.workspace_bytes(dims(), 32768, 512)
    big = mage.workspace_bytes(dims(), 131072, 1024)
    assert 0 < small < big
    assert mage.workspace_bytes(dims(head_dim=96), 1024, 64) == 0
    assert mage.workspace_bytes(dims(num_q_heads=30), 1024, 64) == 0
    assert mage.workspace_bytes(dims(), 0, 64) == 0
    # R = 64 * 4 = 256 rows per KV head runs in two sub-groups on the same layout
    assert mage.workspace_bytes(dims(block=64), 131072, 1024) == big
    assert mage.workspace_bytes(dims(block=200), 1024, 64) == 0
    # a paged call over more than MAGE_MAX_SEQS sequences runs in groups of 256: the
    # size covers the whole shape and every group's
    many = mage.workspace_bytes(dims(num_seqs=300), 4096, 256)
    assert many >= mage.workspace_bytes(dims(num_seqs=256), 4096, 256) > mage.workspace_bytes(dims(num_seqs=44), 4096, 256)
    # every layout starts with the fixed 256 KiB arrival-counter region of the later steps
    tiny = mage.workspace_bytes(dims(block=1, num_q_heads=1, num_kv_heads=1, head_dim=64), 1, 1)
    assert tiny >= 16384 * 4 * 4


FAKE = ctypes.c_void_p(1 << 20)   # never dereferenced: every call below fails its checks first


def call_select(d, n=1024, k=64, ws_bytes=1 << 40, q=FAKE, o=FAKE, idx=FAKE):
    lib = mage.lib()
    return lib.mage_select_exact(ctypes.byref(d), q, FAKE, FAKE, n, k, o, None, idx, None, FAKE,
                                 ws_bytes, None, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), mage.ERR_UNSUPPORTED),
    (dict(num_q_heads=30), mage.ERR_INVALID_ARG),
    (dict(block=200), mage.ERR_UNSUPPORTED),          # B > 128 (R > 128 alone runs in sub-groups)
    (dict(num_seqs=0), mage.ERR_INVALID_ARG),
    (dict(scale=float("nan")), mage.ERR_INVALID_ARG),
    (dict(scale=-1.0), mage.ERR_INVALID_ARG),
])
def test_select_rejects_bad_dims(kw, status):
    assert call_select(dims(**kw)) == status


def test_select_rejects_bad_arguments():
    d = dims()
    assert call_select(d, n=0) == mage.ERR_INVALID_ARG
    assert call_select(d, k=0) == mage.ERR_INVALID_ARG
    assert call_select(d, q=None) == mage.ERR_INVALID_ARG
    assert call_select(d, idx=None) == mage.ERR_INVALID_ARG
    assert call_select(d, q=ctypes.c_void_p((1 << 20) + 2)) == mage.ERR_INVALID_ARG  # misaligned
    assert call_select(d, ws_bytes=16) == mage.ERR_WORKSPACE_TOO_SMALL
    assert b"workspace" in mage.lib().mage_last_error()
    assert call_select(mage.Dims(1, 1, 1, 1, 64, 1.0), ws_bytes=16) == mage.ERR_WORKSPACE_TOO_SMALL
    lib = mage.lib()
    assert lib.mage_select_exact(None, FAKE, FAKE, FAKE, 8, 4, FAKE, None, FAKE, None, FAKE, 1 << 30,
                                 None, None, None) == mage.ERR_INVALID_ARG


def test_sparse_rejects_bad_arguments():
    lib = mage.lib()
    d = dims()
    args = lambda n, idx, k, wsb: (ctypes.byref(d), FAKE, FAKE, FAKE, n, idx, k, FAKE, None, FAKE, wsb, None)
    assert lib.mage_sparse_attn(*args(1024, None, 64, 1 << 40)) == mage.ERR_INVALID_ARG
    assert lib.mage_sparse_attn(*args(1024, FAKE, 0, 1 << 40)) == mage.ERR_INVALID_ARG
    assert lib.mage_sparse_attn(*args(-5, FAKE, 64, 1 << 40)) == mage.ERR_INVALID_ARG
    assert lib.mage_sparse_attn(*args(1024, FAKE, 64, 100)) == mage.ERR_WORKSPACE_TOO_SMALL
    assert lib.mage_sparse_attn(*args(1 << 20, FAKE, mage.MAX_SPARSE_K + 1, 1 << 40)) == mage.ERR_UNSUPPORTED


def test_kernel_timer_arguments():
    """Arming checks its arguments on the host and is cleared by the next call."""
    lib = mage.lib()
    ev = (ctypes.c_void_p * 8)()
    assert lib.mage_arm_kernel_timers(ev, ev, mage.MAX_TIMED_LAUNCHES + 1) == mage.ERR_INVALID_ARG
    assert lib.mage_arm_kernel_timers(None, None, 2) == mage.ERR_INVALID_ARG
    assert lib.mage_arm_kernel_timers(None, None, 0) == mage.OK
    # a call that fails its checks launches nothing and reports no launches
    d = dims()
    assert lib.mage_sparse_attn(ctypes.byref(d), FAKE, FAKE, FAKE, 1024, None, 64, FAKE, None, FAKE,
                                1 << 40, None) == mage.ERR_INVALID_ARG
    assert lib.mage_last_launches(None, 0) == 0
    assert mage.last_launches() == []


def test_paged_rejects_bad_arguments():
    lib = mage.lib()
    d = dims(num_seqs=2)
    lens = (ctypes.c_int32 * 2)(100, 40)
    lp = ctypes.cast(lens, ctypes.POINTER(ctypes.c_int32))

    def kv(page_size=16, max_pages=8, table=FAKE.value):
        return mage.PagedKv(FAKE.value, FAKE.value, table, max_pages, page_size, lp)

    def sel(k):
        return lib.mage_select_exact_paged(ctypes.byref(d), FAKE, ctypes.byref(k), 64, FAKE, None,
                                           FAKE, None, FAKE, 1 << 40, None, None, None)
    assert sel(kv(page_size=12)) == mage.ERR_INVALID_ARG
    assert sel(kv(max_pages=4)) == mage.ERR_INVALID_ARG      # 100 > 4 * 16
    assert sel(kv(table=None)) == mage.ERR_INVALID_ARG
    lens[1] = 0
    assert sel(kv()) == mage.ERR_INVALID_ARG
    # 300 sequences run as groups of 256 and 44; a bad length in the second group
    # is found before the first group is launched (a launch here, with no GPU,
    # would return ERR_HIP)
    big = dims(num_seqs=300, num_kv_heads=8)
    lens300 = (ctypes.c_int32 * 300)(*([64] * 300))
    lens300[280] = 0
    k = mage.PagedKv(FAKE.value, FAKE.value, FAKE.value, 8, 16, ctypes.cast(lens300, ctypes.POINTER(ctypes.c_int32)))
    assert lib.mage_sparse_attn_paged(ctypes.byref(big), FAKE, ctypes.byref(k), FAKE, 64, FAKE, None,
                                      FAKE, 1 << 40, None) == mage.ERR_INVALID_ARG
    assert lib.mage_select_exact_paged(ctypes.byref(big), FAKE, ctypes.byref(k), 64, FAKE, None, FAKE, None,
                                       FAKE, 1 << 40, None, None, None) == mage.ERR_INVALID_ARG
    assert b"seq_lens" in lib.mage_last_error()


def test_topk_rejects_bad_arguments():
    lib = mage.lib()
    assert lib.mage_topk(0, FAKE, 10, None, 10, 4, FAKE, FAKE, 1 << 30, None) == mage.ERR_INVALID_ARG
    assert lib.mage_topk(2, FAKE, 5, None, 10, 4, FAKE, FAKE, 1 << 30, None) == mage.ERR_INVALID_ARG
    assert lib.mage_topk(2, FAKE, 10, None, 10, 4, FAKE, FAKE, 8, None) == mage.ERR_WORKSPACE_TOO_SMALL
    lens = (ctypes.c_int32 * 2)(3, 11)
    assert lib.mage_topk(2, FAKE, 10, ctypes.cast(lens, ctypes.POINTER(ctypes.c_int32)), 10, 4, FAKE,
                         FAKE, 1 << 30, None) == mage.ERR_INVALID_ARG


def test_calls_fail_loudly_without_a_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("GPU present")
    q = torch.zeros(1, 2, 1, 64, dtype=torch.bfloat16)
    with pytest.raises((ValueError, RuntimeError)):
        mage.sparse_attn(q, torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16),
                         torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16),
                         torch.zeros(1, 1, 4, dtype=torch.int32), 0.125)


def test_block_attn_argument_checks():
    lib = mage.lib()
    d = dims()
    ok = [ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None]
    # null inputs / output
    for i in (1, 2, 3, 4, 5, 6):
        args = list(ok)
        args[i] = None
        assert lib.mage_block_attn(*args) == mage.ERR_INVALID_ARG
    # misaligned bf16 input and fp32 output
    for i in (1, 4, 6):
        args = list(ok)
        args[i] = ctypes.c_void_p((1 << 20) + 4)
        assert lib.mage_block_attn(*args) == mage.ERR_INVALID_ARG
    # unsupported head dim, bad group
    assert lib.mage_block_attn(ctypes.byref(dims(head_dim=96)), *ok[1:]) == mage.ERR_UNSUPPORTED
    assert lib.mage_block_attn(ctypes.byref(dims(num_q_heads=30)), *ok[1:]) != mage.OK


def test_sparse_block_attn_argument_checks():
    lib = mage.lib()
    d = dims()
    # dims, q, k_cache, v_cache, seq_len, idx, k, k_blk, v_blk, o, lse, workspace, bytes, stream
    ok = [ctypes.byref(d), FAKE, FAKE, FAKE, 1024, FAKE, 64, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None]
    for i in (7, 8):
        args = list(ok)
        args[i] = None
        assert lib.mage_sparse_block_attn(*args) == mage.ERR_INVALID_ARG
        args[i] = ctypes.c_void_p((1 << 20) + 4)
        assert lib.mage_sparse_block_attn(*args) == mage.ERR_INVALID_ARG
    args = list(ok)
    args[6] = 0
    assert lib.mage_sparse_block_attn(*args) == mage.ERR_INVALID_ARG
    # paged: dims, q, kv, idx, k, k_blk, v_blk, o, lse, workspace, bytes, stream
    pk = mage.PagedKv()
    okp = [ctypes.byref(d), FAKE, ctypes.byref(pk), FAKE, 64, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None]
    for i in (5, 6):
        args = list(okp)
        args[i] = None
        assert lib.mage_sparse_block_attn_paged(*args) == mage.ERR_INVALID_ARG
    assert lib.mage_sparse_block_attn_paged(ctypes.byref(dims(head_dim=96)), *okp[1:]) == mage.ERR_UNSUPPORTED


def test_anchor_diagnostics_argument_checks():
    lib = mage.lib()
    d = dims()
    # dims, q, k_cache, v_cache, seq_len, k, idx, scores, workspace, bytes, stream
    ok = [ctypes.byref(d), FAKE, FAKE, FAKE, 1024, 64, FAKE, None, FAKE, 1 << 30, None]
    for i, bad in ((1, None), (6, None), (5, 0), (1, ctypes.c_void_p((1 << 20) + 2)),
                   (7, ctypes.c_void_p((1 << 20) + 2))):
        args = list(ok)
        args[i] = bad
        assert lib.mage_select_mean_query(*args) == mage.ERR_INVALID_ARG
    assert lib.mage_select_mean_query(ctypes.byref(dims(head_dim=96)), *ok[1:]) == mage.ERR_UNSUPPORTED
    pk = mage.PagedKv()
    okp = [ctypes.byref(d), FAKE, ctypes.byref(pk), 64, FAKE, None, FAKE, 1 << 30, None]
    assert lib.mage_select_mean_query_paged(*okp) == mage.ERR_INVALID_ARG      # empty paged cache
    args = list(okp)
    args[4] = None
    assert lib.mage_select_mean_query_paged(*args) == mage.ERR_INVALID_ARG
    # mean query alone
    assert lib.mage_mean_query(ctypes.byref(d), None, FAKE, None) == mage.ERR_INVALID_ARG
    assert lib.mage_mean_query(ctypes.byref(d), FAKE, None, None) == mage.ERR_INVALID_ARG
    assert lib.mage_mean_query(ctypes.byref(dims(num_q_heads=30)), FAKE, FAKE, None) == mage.ERR_INVALID_ARG
    # overlap: rows, k, a, b, common, count_a, count_b, stream
    assert lib.mage_idx_overlap(0, 4, FAKE, FAKE, FAKE, None, None, None) == mage.ERR_INVALID_ARG
    assert lib.mage_idx_overlap(4, 0, FAKE, FAKE, FAKE, None, None, None) == mage.ERR_INVALID_ARG
    assert lib.mage_idx_overlap(4, 4, None, FAKE, FAKE, None, None, None) == mage.ERR_INVALID_ARG
    assert lib.mage_idx_overlap(4, 4, FAKE, FAKE, None, None, None, None) == mage.ERR_INVALID_ARG
    assert lib.mage_idx_overlap(4, 4, FAKE, FAKE, FAKE, ctypes.c_void_p((1 << 20) + 2), None,
                                None) == mage.ERR_INVALID_ARG


def test_select_pages_argument_checks():
    lib = mage.lib()
    d = dims()
    # dims, q, k_cache, v_cache, seq_len, page_tokens, k_pages, o, lse, idx, page_idx, scores, ws, bytes,
    # attn stream, select stream, event
    ok = [ctypes.byref(d), FAKE, FAKE, FAKE, 1024, 16, 8, FAKE, None, FAKE, None, None, FAKE, 1 << 40, None,
          None, None]
    for i, bad, st in ((5, 0, mage.ERR_INVALID_ARG), (5, 5000, mage.ERR_INVALID_ARG), (6, 0, mage.ERR_INVALID_ARG),
                       (6, 1 << 20, mage.ERR_UNSUPPORTED), (10, ctypes.c_void_p((1 << 20) + 2), mage.ERR_INVALID_ARG),
                       (9, None, mage.ERR_INVALID_ARG), (1, None, mage.ERR_INVALID_ARG)):
        args = list(ok)
        args[i] = bad
        assert lib.mage_select_pages(*args) == st, (i, bad)
    args = list(ok)
    args[13] = 1024
    assert lib.mage_select_pages(*args) == mage.ERR_WORKSPACE_TOO_SMALL
    pk = mage.PagedKv()
    okp = [ctypes.byref(d), FAKE, ctypes.byref(pk), 16, 8, FAKE, None, FAKE, None, None, FAKE, 1 << 40, None, None,
           None]
    assert lib.mage_select_pages_paged(*okp) == mage.ERR_INVALID_ARG       # empty paged cache
    args = list(okp)
    args[3] = 0
    assert lib.mage_select_pages_paged(*args) == mage.ERR_INVALID_ARG


def test_adaptive_budget_argument_checks():
    lib = mage.lib()
    d = dims()
    # dims, q, k_cache, v_cache, seq_len, k, o, lse, idx, counts, ws, bytes, attn, select, event
    ok = [ctypes.byref(d), FAKE, FAKE, FAKE, 1024, 64, FAKE, None, FAKE, FAKE, FAKE, 1 << 40, None, None, None]
    for i, bad, st in ((9, None, mage.ERR_INVALID_ARG), (9, ctypes.c_void_p((1 << 20) + 2), mage.ERR_INVALID_ARG),
                       (5, 0, mage.ERR_INVALID_ARG), (5, 1 << 15, mage.ERR_UNSUPPORTED), (8, None, mage.ERR_INVALID_ARG)):
        args = list(ok)
        args[i] = bad
        assert lib.mage_select_adaptive(*args) == st, (i, bad)
    pk = mage.PagedKv()
    okp = [ctypes.byref(d), FAKE, ctypes.byref(pk), 64, FAKE, None, FAKE, FAKE, FAKE, 1 << 40, None, None, None]
    assert lib.mage_select_adaptive_paged(*okp) == mage.ERR_INVALID_ARG
    # counts step: dims, q, k_cache, v_cache, seq_len, idx, k_row, counts, k_seq, o, lse, ws, bytes, stream
    oks = [ctypes.byref(d), FAKE, FAKE, FAKE, 1024, FAKE, 64, FAKE, 512, FAKE, None, FAKE, 1 << 40, None]
    for i, bad in ((7, None), (8, 0), (6, 0), (5, None)):
        args = list(oks)
        args[i] = bad
        assert lib.mage_sparse_attn_counts(*args) == mage.ERR_INVALID_ARG, (i, bad)
    okps = [ctypes.byref(d), FAKE, ctypes.byref(pk), FAKE, 64, FAKE, 512, FAKE, None, FAKE, 1 << 40, None]
    assert lib.mage_sparse_attn_counts_paged(*okps) == mage.ERR_INVALID_ARG


def test_noalloc_rejects_a_plan_beyond_its_scratch():
    # 32 units of one 32-row block, k = 1024: 8 chunks per unit, 256 partial slots of
    # 64 KiB (16 MiB) > the 8 MiB scratch; rejected before any HIP call
    lib = mage.lib()
    d = dims(num_seqs=4, block=8, num_q_heads=32, num_kv_heads=8)
    st = lib.mage_sparse_attn_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, 4096, FAKE, 1024, FAKE, None, None)
    assert st == mage.ERR_UNSUPPORTED
    assert b"scratch" in lib.mage_last_error()
    # and argument checks come first: null q
    assert lib.mage_sparse_attn_noalloc(ctypes.byref(dims()), None, FAKE, FAKE, 4096, FAKE, 64, FAKE, None,
                                        None) == mage.ERR_INVALID_ARG
