"""Python binding of libmage.so: block-shared top-k sparse KV attention (MAGE) on MI355X.

Argument marshalling only. Every step of the path runs in the HIP kernels of
``libmage.so`` (C ABI in ``include/mage.h``); PyTorch provides device memory
and streams. There is no CPU fallback: importing works without a GPU, but
each call raises if the library or a GPU is missing.

Entry points mirror the C ABI:

* :func:`select_exact` / :func:`select_exact_paged` -- step 1 of a block:
  exact O and lse on the caller's stream, the block-averaged scores and the
  top-k index set on a second stream.
* :func:`sparse_attn` / :func:`sparse_attn_paged` -- a later step over the
  reused index set.
* :func:`topk` -- the selection on its own, over caller-provided scores.
* :func:`arm_kernel_timers` / :func:`last_launches` -- per-kernel GPU timing
  of the next call (HIP events attached to the kernel launches).
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmage.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE_TOO_SMALL, ERR_HIP = range(5)
MAX_SEQS = 256
MAX_ROWS = 128
MAX_SPARSE_K = 131072
MAX_TIMED_LAUNCHES = 12


class MageError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        super().__init__(f"{func}: status {status} ({detail})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("block", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("scale", ctypes.c_float)]


class PagedKv(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("seq_lens", ctypes.POINTER(ctypes.c_int32))]


_lib = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t


def lib():
    """Load libmage.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m block_sparse_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.mage_workspace_bytes.argtypes = [P(Dims), _i32, _i32]
        L.mage_workspace_bytes.restype = _sz
        L.mage_workspace_init.argtypes = [_vp, _sz, _vp]
        L.mage_workspace_check.argtypes = [_vp, _sz, _vp, _vp]
        L.mage_select_exact.argtypes = [P(Dims), _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp,
                                        _vp, _sz, _vp, _vp, _vp]
        L.mage_select_exact_paged.argtypes = [P(Dims), _vp, P(PagedKv), _i32, _vp, _vp, _vp, _vp,
                                              _vp, _sz, _vp, _vp, _vp]
        L.mage_exact_attn.argtypes = [P(Dims), _vp, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp]
        L.mage_exact_attn_paged.argtypes = [P(Dims), _vp, P(PagedKv), _vp, _vp, _vp, _sz, _vp]
        L.mage_sparse_attn.argtypes = [P(Dims), _vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _sz,
                                       _vp]
        L.mage_sparse_attn_paged.argtypes = [P(Dims), _vp, P(PagedKv), _vp, _i32, _vp, _vp, _vp,
                                             _sz, _vp]
        L.mage_sparse_attn_noalloc.argtypes = [P(Dims), _vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _vp]
        L.mage_topk.argtypes = [_i32, _vp, ctypes.c_int64, P(_i32), _i32, _i32, _vp, _vp, _sz, _vp]
        L.mage_block_attn.argtypes = [P(Dims), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.mage_sparse_block_attn.argtypes = [P(Dims), _vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp,
                                             _vp, _sz, _vp]
        L.mage_sparse_block_attn_paged.argtypes = [P(Dims), _vp, P(PagedKv), _vp, _i32, _vp, _vp, _vp,
                                                   _vp, _vp, _sz, _vp]
        L.mage_select_mean_query.argtypes = [P(Dims), _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _sz, _vp]
        L.mage_select_mean_query_paged.argtypes = [P(Dims), _vp, P(PagedKv), _i32, _vp, _vp, _vp, _sz, _vp]
        L.mage_idx_overlap.argtypes = [_i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]
        L.mage_mean_query.argtypes = [P(Dims), _vp, _vp, _vp]
        L.mage_select_adaptive.argtypes = [P(Dims), _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp,
                                           _vp, _vp]
        L.mage_select_adaptive_paged.argtypes = [P(Dims), _vp, P(PagedKv), _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp,
                                                 _vp, _vp]
        L.mage_sparse_attn_counts.argtypes = [P(Dims), _vp, _vp, _vp, _i32, _vp, _i32, _vp, _i32, _vp, _vp, _vp,
                                              _sz, _vp]
        L.mage_sparse_attn_counts_paged.argtypes = [P(Dims), _vp, P(PagedKv), _vp, _i32, _vp, _i32, _vp, _vp, _vp,
                                                    _sz, _vp]
        L.mage_select_pages.argtypes = [P(Dims), _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _sz, _vp, _vp, _vp]
        L.mage_select_pages_paged.argtypes = [P(Dims), _vp, P(PagedKv), _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                              _sz, _vp, _vp, _vp]
        for f in ("mage_workspace_init", "mage_workspace_check", "mage_select_exact", "mage_select_exact_paged",
                  "mage_exact_attn", "mage_exact_attn_paged",
                  "mage_sparse_attn", "mage_sparse_attn_paged", "mage_sparse_attn_noalloc", "mage_topk", "mage_block_attn",
                  "mage_sparse_block_attn", "mage_sparse_block_attn_paged", "mage_select_mean_query",
                  "mage_select_mean_query_paged", "mage_idx_overlap", "mage_mean_query",
                  "mage_select_pages", "mage_select_pages_paged", "mage_select_adaptive",
                  "mage_select_adaptive_paged", "mage_sparse_attn_counts", "mage_sparse_attn_counts_paged"):
            getattr(L, f).restype = ctypes.c_int
        L.mage_status_string.argtypes = [ctypes.c_int]
        L.mage_status_string.restype = ctypes.c_char_p
        L.mage_last_error.argtypes = []
        L.mage_last_error.restype = ctypes.c_char_p
        L.mage_arm_kernel_timers.argtypes = [P(_vp), P(_vp), _i32]
        L.mage_arm_kernel_timers.restype = ctypes.c_int
        L.mage_last_launches.argtypes = [P(ctypes.c_char_p), _i32]
        L.mage_last_launches.restype = _i32
        _lib = L
    return _lib


def _check(status: int, func: str):
    if status != OK:
        raise MageError(status, func, lib().mage_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(s):
    if s is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(s.cuda_stream)


def make_dims(q: torch.Tensor, num_kv_heads: int, scale: float) -> Dims:
    S, B, Hq, d = q.shape
    return Dims(S, B, Hq, num_kv_heads, d, float(scale))


def workspace_bytes(dims: Dims, max_seq_len: int, k: int) -> int:
    return int(lib().mage_workspace_bytes(ctypes.byref(dims), int(max_seq_len), int(k)))


def _capturing(stream) -> bool:
    """True while `stream` (a torch stream, None = the current one) is being captured into a graph."""
    if stream is None or stream == torch.cuda.current_stream(stream.device):
        return torch.cuda.is_current_stream_capturing()
    with torch.cuda.stream(stream):
        return torch.cuda.is_current_stream_capturing()


class Workspace:
    """A device workspace; grows when a call needs more.

    Every new buffer is zeroed (mage_workspace_init) on the stream of the call
    that needs it: the sparse calls keep arrival counters in it, which must
    start at zero and which every call leaves at zero.

    Calls through one Workspace are ordered, whatever streams they run on: a
    call notes the streams it used (its stream and, for step 1, its select
    stream); when the next call runs on another stream, an event is recorded
    on each of those streams (after everything queued there, the previous call
    included) and the new call's stream waits for it. A buffer that is
    replaced by a larger one goes back to the allocator only after the work
    queued on every stream that used it (record_stream). Under graph capture
    nothing is recorded or waited for: the graph's own edges order the
    captured calls.
    """

    def __init__(self, device=None):
        self.device = torch.device(device or "cuda")
        self.buf = None
        self.pending = []          # streams the previous call used
        self._users = set()        # streams (handles) the current buffer was used on
        self._events = {}          # one reusable event per stream handle

    def _order_after_pending(self, st):
        for s in self.pending or []:
            if s.cuda_stream != st.cuda_stream:
                ev = self._events.get(s.cuda_stream)
                if ev is None:
                    ev = self._events[s.cuda_stream] = torch.cuda.Event()
                ev.record(s)
                st.wait_event(ev)

    def get(self, nbytes: int, stream=None) -> torch.Tensor:
        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        if not _capturing(st):
            self._order_after_pending(st)
            self.pending = []
        if self.buf is None or self.buf.numel() < nbytes:
            with torch.cuda.stream(st):
                self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
            self._users = {st.cuda_stream}
            _check(lib().mage_workspace_init(_ptr(self.buf), self.buf.numel(), _stream(st)),
                   "mage_workspace_init")
        return self.buf

    def done(self, stream=None, *others):
        """Note that the call just issued used this workspace on `stream`
        (None = the current stream) and on `others` (None entries ignored)."""
        first = stream if stream is not None else torch.cuda.current_stream(self.device)
        sts = [first] + [s for s in others if s is not None]
        if _capturing(first):
            return
        out = []
        for s in sts:
            if any(s.cuda_stream == x.cuda_stream for x in out):
                continue
            out.append(s)
            if s.cuda_stream not in self._users:
                self.buf.record_stream(s)
                self._users.add(s.cuda_stream)
        self.pending = out

    def mark(self, stream):
        """Record that work using this workspace is still running on `stream`."""
        self.done(stream)

    def check(self, stream=None) -> int:
        """Number of non-zero arrival counters (0 for a healthy workspace);
        waits for `stream`."""
        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        if self.buf is None:
            return 0
        self._order_after_pending(st)
        out = torch.empty(1, dtype=torch.int32, device=self.device)
        _check(lib().mage_workspace_check(_ptr(self.buf), self.buf.numel(), _ptr(out), _stream(st)),
               "mage_workspace_check")
        return int(out.item())


_default_ws = {}


def _ws_obj(workspace, device):
    if workspace is None:
        workspace = _default_ws.setdefault(str(device), Workspace(device))
    return workspace


def _bf16_ptr(t, name):
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor")
    return _ptr(t)


def _out(t, shape, dtype, device):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"output must be contiguous {dtype} of shape {tuple(shape)}")
    return t


def select_exact(q, k_cache, v_cache, k: int, scale: float, *, o=None, lse=None, idx=None,
                 scores=None, want_scores=True, workspace=None, stream=None, select_stream=None,
                 idx_ready=None):
    """Step 1: exact attention + block-averaged scores + top-k, contiguous cache.

    q bf16 [S][B][Hq][d]; k_cache, v_cache bf16 [S][Hkv][N][d].
    Returns (o fp32 [S][B][Hq][d], lse fp32 [S][B][Hq], idx int32 [S][Hkv][k],
    scores fp32 [S][Hkv][N] or None). idx/scores are ready on select_stream
    (recorded into idx_ready, a torch.cuda.Event, if given).
    """
    S, B, Hq, d = q.shape
    _, Hkv, N, _ = k_cache.shape
    dims = make_dims(q, Hkv, scale)
    dev = q.device
    o = _out(o, (S, B, Hq, d), torch.float32, dev)
    lse = _out(lse, (S, B, Hq), torch.float32, dev)
    idx = _out(idx, (S, Hkv, k), torch.int32, dev)
    if want_scores:
        scores = _out(scores, (S, Hkv, N), torch.float32, dev)
    wso = _ws_obj(workspace, dev)
    ws = wso.get(workspace_bytes(dims, N, k), stream)
    _check(lib().mage_select_exact(ctypes.byref(dims), _bf16_ptr(q, "q"),
                                   _bf16_ptr(k_cache, "k_cache"), _bf16_ptr(v_cache, "v_cache"),
                                   N, int(k), _ptr(o), _ptr(lse), _ptr(idx), _ptr(scores),
                                   _ptr(ws), ws.numel(), _stream(stream),
                                   None if select_stream is None else _stream(select_stream),
                                   None), "mage_select_exact")
    wso.done(stream, select_stream)
    if idx_ready is not None:
        idx_ready.record(select_stream if select_stream is not None else torch.cuda.current_stream())
    return o, lse, idx, scores


def _paged(k_pool, v_pool, page_table, seq_lens):
    lens = [int(x) for x in (seq_lens.tolist() if torch.is_tensor(seq_lens) else seq_lens)]
    arr = (ctypes.c_int32 * len(lens))(*lens)
    if page_table.dtype != torch.int32 or not page_table.is_cuda or not page_table.is_contiguous():
        raise ValueError("page_table must be a contiguous int32 CUDA tensor")
    kv = PagedKv(_bf16_ptr(k_pool, "k_pool").value, _bf16_ptr(v_pool, "v_pool").value,
                 page_table.data_ptr(), page_table.shape[1], k_pool.shape[2],
                 ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)))
    return kv, arr, lens


def select_exact_paged(q, k_pool, v_pool, page_table, seq_lens, k: int, scale: float, *, o=None,
                       lse=None, idx=None, scores=None, want_scores=True, workspace=None,
                       stream=None, select_stream=None, idx_ready=None):
    """Step 1 over a paged cache (pools bf16 [P][Hkv][page][d], host seq_lens).

    scores is fp32 [S][Hkv][max(seq_lens)]; entries past N_s are left untouched.
    """
    S, B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    dims = make_dims(q, Hkv, scale)
    kv, keep, lens = _paged(k_pool, v_pool, page_table, seq_lens)
    maxn = max(lens)
    dev = q.device
    o = _out(o, (S, B, Hq, d), torch.float32, dev)
    lse = _out(lse, (S, B, Hq), torch.float32, dev)
    idx = _out(idx, (S, Hkv, k), torch.int32, dev)
    if want_scores:
        scores = _out(scores, (S, Hkv, maxn), torch.float32, dev)
    wso = _ws_obj(workspace, dev)
    ws = wso.get(workspace_bytes(dims, maxn, k), stream)
    _check(lib().mage_select_exact_paged(ctypes.byref(dims), _bf16_ptr(q, "q"), ctypes.byref(kv),
                                         int(k), _ptr(o), _ptr(lse), _ptr(idx), _ptr(scores),
                                         _ptr(ws), ws.numel(), _stream(stream),
                                         None if select_stream is None else _stream(select_stream),
                                         None), "mage_select_exact_paged")
    wso.done(stream, select_stream)
    if idx_ready is not None:
        idx_ready.record(select_stream if select_stream is not None else torch.cuda.current_stream())
    return o, lse, idx, scores


def select_pages(q, k_cache, v_cache, page_tokens: int, k_pages: int, scale: float, *, o=None, lse=None,
                 idx=None, page_idx=None, scores=None, want_scores=False, workspace=None, stream=None):
    """Step 1 with page-granular selection. Returns (o, lse, idx int32
    [S][Hkv][k_pages * page_tokens] positions, page_idx int32 [S][Hkv][k_pages],
    scores or None); everything on `stream`."""
    S, B, Hq, d = q.shape
    _, Hkv, N, _ = k_cache.shape
    dims = make_dims(q, Hkv, scale)
    dev = q.device
    k = k_pages * page_tokens
    o = _out(o, (S, B, Hq, d), torch.float32, dev)
    lse = _out(lse, (S, B, Hq), torch.float32, dev)
    idx = _out(idx, (S, Hkv, k), torch.int32, dev)
    page_idx = _out(page_idx, (S, Hkv, k_pages), torch.int32, dev)
    if want_scores or scores is not None:
        scores = _out(scores, (S, Hkv, N), torch.float32, dev)
    wso = _ws_obj(workspace, dev)
    ws = wso.get(workspace_bytes(dims, N, k), stream)
    _check(lib().mage_select_pages(ctypes.byref(dims), _bf16_ptr(q, "q"), _bf16_ptr(k_cache, "k_cache"),
                                   _bf16_ptr(v_cache, "v_cache"), N, int(page_tokens), int(k_pages), _ptr(o),
                                   _ptr(lse), _ptr(idx), _ptr(page_idx), _ptr(scores), _ptr(ws), ws.numel(),
                                   _stream(stream), None, None), "mage_select_pages")
    wso.done(stream)
    return o, lse, idx, page_idx, scores


def select_pages_paged(q, k_pool, v_pool, page_table, seq_lens, page_tokens: int, k_pages: int, scale: float, *,
                       o=None, lse=None, idx=None, page_idx=None, scores=None, want_scores=False, workspace=None,
                       stream=None):
    """select_pages over a paged cache; scores fp32 [S][Hkv][max(seq_lens)]."""
    S, B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    dims = make_dims(q, Hkv, scale)
    kv, keep, lens = _paged(k_pool, v_pool, page_table, seq_lens)
    dev = q.device
    k = k_pages * page_tokens
    o = _out(o, (S, B, Hq, d), torch.float32, dev)
    lse = _out(lse, (S, B, Hq), torch.float32, dev)
    idx = _out(idx, (S, Hkv, k), torch.int32, dev)
    page_idx = _out(page_idx, (S, Hkv, k_pages), torch.int32, dev)
    if want_scores or scores is not None:
        scores = _out(scores, (S, Hkv, max(lens)), torch.float32, dev)
    wso = _ws_obj(workspace, dev)
    ws = wso.get(workspace_bytes(dims, max(lens), k), stream)
    _check(lib().mage_select_pages_paged(ctypes.byref(dims), _bf16_ptr(q, "q"), ctypes.byref(kv), int(page_tokens),
                                         int(k_pages), _ptr(o), _ptr(lse), _ptr(idx), _ptr(page_idx), _ptr(scores),
                                         _ptr(ws), ws.numel(), _stream(stream), None, None),
           "mage_select_pages_paged")
    wso.done(stream)
    return o, lse, idx, page_idx, scores


def select_adaptive(q, k_cache, v_cache, k: int, scale: float, *, o=None, lse=None, idx=None, counts=None,
                    workspace=None, stream=None):
    """Step 1 with head-adaptive budgets (k * Hkv positions per sequence shared by
    its KV heads). Returns (o, lse, idx int32 [S][Hkv][k * Hkv], counts int32
    [S][Hkv]); everything on `stream`."""
    S, B, Hq, d = q.shape
    _, Hkv, N, _ = k_cache.shape
    dims = make_dims(q, Hkv, scale)
    dev = q.device
    K = k * Hkv
    o = _out(o, (S, B, Hq, d), torch.float32, dev)
    lse = _out(lse, (S, B, Hq), torch.float32, dev)
    idx = _out(idx, (S, Hkv, K), torch.int32, dev)
    counts = _out(counts, (S, Hkv), torch.int32, dev)
    wso = _ws_obj(workspace, dev)
    ws = wso.get(workspace_bytes(dims, N, K), stream)
    _check(lib().mage_select_adaptive(ctypes.byref(dims), _bf16_ptr(q, "q"), _bf16_ptr(k_cache, "k_cache"),
                                      _bf16_ptr(v_cache, "v_cache"), N, int(k), _ptr(o), _ptr(lse), _ptr(idx),
                                      _ptr(counts), _ptr(ws), ws.numel(), _stream(stream), None, None),
           "mage_select_adaptive")
    wso.done(stream)
    return o, lse, idx, counts


def select_adaptive_paged(q, k_pool, v_pool, page_table, seq_lens, k: int, scale: float, *, o=None, lse=None,
                          idx=None, counts=None, workspace=None, stream=None):
    """select_adaptive over a paged cache."""
    S, B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    dims = make_dims(q, Hkv, scale)
    kv, keep, lens = _paged(k_pool, v_pool, page_table, seq_lens)
    dev = q.device
    K = k * Hkv
    o = _out(o, (S, B, Hq, d), torch.float32, dev)
    lse = _out(lse, (S, B, Hq), torch.float32, dev)
    idx = _out(idx, (S, Hkv, K), torch.int32, dev)
    counts = _out(counts, (S, Hkv), torch.int32, dev)
    wso = _ws_obj(workspace, dev)
    ws = wso.get(workspace_bytes(dims, max(lens), K), stream)
    _check(lib().mage_select_adaptive_paged(ctypes.byref(dims), _bf16_ptr(q, "q"), ctypes.byref(kv), int(k),
                                            _ptr(o), _ptr(lse), _ptr(idx), _ptr(counts), _ptr(ws), ws.numel(),
                                            _stream(stream), None, None), "mage_select_adaptive_paged")
    wso.done(stream)
    return o, lse, idx, counts


def _counts_arg(counts, S, Hkv):
    if counts.dtype != torch.int32 or not counts.is_cuda or not counts.is_contiguous() or \
            tuple(counts.shape) != (S, Hkv):
        raise ValueError("counts must be a contiguous int32 CUDA tensor [S][Hkv]")
    return _ptr(counts)


def sparse_attn_counts(q, k_cache, v_cache, idx, counts, k_seq: int, scale: float, *, o=None, lse=None,
                       workspace=None, stream=None):
    """A later step over idx[s][h][:counts[s][h]] (head-adaptive budgets); k_seq
    bounds the entries of a sequence summed over its heads."""
    S, B, Hq, d = q.shape
    _, Hkv, N, _ = k_cache.shape
    k_row = idx.shape[-1]
    if idx.dtype != torch.int32 or not idx.is_contiguous() or tuple(idx.shape[:2]) != (S, Hkv):
        raise ValueError("idx must be contiguous int32 [S][Hkv][k_row]")
    cp = _counts_arg(counts, S, Hkv)
    dims = make_dims(q, Hkv, scale)
    dev = q.device
    o = _out(o, (S, B, Hq, d), torch.float32, dev)
    lse = _out(lse, (S, B, Hq), torch.float32, dev)
    wso = _ws_obj(workspace, dev)
    ws = wso.get(workspace_bytes(dims, N, k_row), stream)
    _check(lib().mage_sparse_attn_counts(ctypes.byref(dims), _bf16_ptr(q, "q"), _bf16_ptr(k_cache, "k_cache"),
                                         _bf16_ptr(v_cache, "v_cache"), N, _ptr(idx), int(k_row), cp, int(k_seq),
                                         _ptr(o), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)),
           "mage_sparse_attn_counts")
    wso.done(stream)
    return o, lse


def sparse_attn_counts_paged(q, k_pool, v_pool, page_table, seq_lens, idx, counts, k_seq: int, scale: float, *,
                             o=None, lse=None, workspace=None, stream=None):
    """sparse_attn_counts over a paged cache."""
    S, B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    k_row = idx.shape[-1]
    if idx.dtype != torch.int32 or not idx.is_contiguous() or tuple(idx.shape[:2]) != (S, Hkv):
        raise ValueError("idx must be contiguous int32 [S][Hkv][k_row]")
    cp = _counts_arg(counts, S, Hkv)
    dims = make_dims(q, Hkv, scale)
    kv, keep, lens = _paged(k_pool, v_pool, page_table, seq_lens)
    dev = q.device
    o = _out(o, (S, B, Hq, d), torch.float32, dev)
    lse = _out(lse, (S, B, Hq), torch.float32, dev)
    wso = _ws_obj(workspace, dev)
    ws = wso.get(workspace_bytes(dims, max(lens), k_row), stream)
    _check(lib().mage_sparse_attn_counts_paged(ctypes.byref(dims), _bf16_ptr(q, "q"), ctypes.byref(kv), _ptr(idx),
                                               int(k_row), cp, int(k_seq), _ptr(o), _ptr(lse), _ptr(ws),
                                               ws.numel(), _stream(stream)), "mage_sparse_attn_counts_paged")
    wso.done(stream)
    return o, lse


def mean_query(q, num_kv_heads: int, *, out=None, stream=None):
    """The block's mean query per KV head, rounded once to bf16: [S][1][Hkv][d]."""
    S, B, Hq, d = q.shape
    dims = make_dims(q, num_kv_heads, 1.0)
    out = _out(out, (S, 1, num_kv_heads, d), torch.bfloat16, q.device)
    _check(lib().mage_mean_query(ctypes.byref(dims), _bf16_ptr(q, "q"), _bf16_ptr(out, "out"), _stream(stream)),
           "mage_mean_query")
    return out


def select_mean_query(q, k_cache, v_cache, k: int, scale: float, *, idx=None, scores=None,
                      want_scores=False, workspace=None, stream=None):
    """Top-k by the probability under the block's mean query (one bf16 row per
    KV head). Returns (idx int32 [S][Hkv][k], scores fp32 [S][Hkv][N] or None)."""
    S, B, Hq, d = q.shape
    _, Hkv, N, _ = k_cache.shape
    dims = make_dims(q, Hkv, scale)
    dev = q.device
    idx = _out(idx, (S, Hkv, k), torch.int32, dev)
    if want_scores or scores is not None:
        scores = _out(scores, (S, Hkv, N), torch.float32, dev)
    wso = _ws_obj(workspace, dev)
    ws = wso.get(workspace_bytes(dims, N, k), stream)
    _check(lib().mage_select_mean_query(ctypes.byref(dims), _bf16_ptr(q, "q"), _bf16_ptr(k_cache, "k_cache"),
                                        _bf16_ptr(v_cache, "v_cache"), N, int(k), _ptr(idx), _ptr(scores),
                                        _ptr(ws), ws.numel(), _stream(stream)), "mage_select_mean_query")
    wso.done(stream)
    return idx, scores


def select_mean_query_paged(q, k_pool, v_pool, page_table, seq_lens, k: int, scale: float, *, idx=None,
                            scores=None, want_scores=False, workspace=None, stream=None):
    """select_mean_query over a paged cache; scores fp32 [S][Hkv][max(seq_lens)]."""
    S, B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    dims = make_dims(q, Hkv, scale)
    kv, keep, lens = _paged(k_pool, v_pool, page_table, seq_lens)
    dev = q.device
    idx = _out(idx, (S, Hkv, k), torch.int32, dev)
    if want_scores or scores is not None:
        scores = _out(scores, (S, Hkv, max(lens)), torch.float32, dev)
    wso = _ws_obj(workspace, dev)
    ws = wso.get(workspace_bytes(dims, max(lens), k), stream)
    _check(lib().mage_select_mean_query_paged(ctypes.byref(dims), _bf16_ptr(q, "q"), ctypes.byref(kv), int(k),
                                              _ptr(idx), _ptr(scores), _ptr(ws), ws.numel(), _stream(stream)),
           "mage_select_mean_query_paged")
    wso.done(stream)
    return idx, scores


def idx_overlap(a, b, *, stream=None):
    """Per row of two int32 index tensors [..., k] in idx form: (common, count_a,
    count_b) int32 tensors; the recall of a against b is common / count_b."""
    if a.shape != b.shape or a.dtype != torch.int32 or b.dtype != torch.int32:
        raise ValueError("a and b must be int32 tensors of one shape")
    if not (a.is_cuda and b.is_cuda and a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous CUDA tensors")
    k = a.shape[-1]
    rows = a.numel() // k
    common = torch.empty(a.shape[:-1], dtype=torch.int32, device=a.device)
    ca = torch.empty_like(common)
    cb = torch.empty_like(common)
    _check(lib().mage_idx_overlap(rows, k, _ptr(a), _ptr(b), _ptr(common), _ptr(ca), _ptr(cb),
                                  _stream(stream)), "mage_idx_overlap")
    return common, ca, cb


def exact_attn(q, k_cache, v_cache, scale: float, *, o=None, lse=None, workspace=None, stream=None):
    """Exact attention of the block over the whole contiguous prefix (no selection)."""
    S, B, Hq, d = q.shape
    _, Hkv, N, _ = k_cache.shape
    dims = make_dims(q, Hkv, scale)
    dev = q.device
    o = _out(o, (S, B, Hq, d), torch.float32, dev)
    lse = _out(lse, (S, B, Hq), torch.float32, dev)
    wso = _ws_obj(workspace, dev)
    ws = wso.get(workspace_bytes(dims, N, 1), stream)
    _check(lib().mage_exact_attn(ctypes.byref(dims), _bf16_ptr(q, "q"), _bf16_ptr(k_cache, "k_cache"),
                                 _bf16_ptr(v_cache, "v_cache"), N, _ptr(o), _ptr(lse), _ptr(ws),
                                 ws.numel(), _stream(stream)), "mage_exact_attn")
    wso.done(stream)
    return o, lse


def exact_attn_paged(q, k_pool, v_pool, page_table, seq_lens, scale: float, *, o=None, lse=None,
                     workspace=None, stream=None):
    """Exact attention over a paged cache (no selection)."""
    S, B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    dims = make_dims(q, Hkv, scale)
    kv, keep, lens = _paged(k_pool, v_pool, page_table, seq_lens)
    dev = q.device
    o = _out(o, (S, B, Hq, d), torch.float32, dev)
    lse = _out(lse, (S, B, Hq), torch.float32, dev)
    wso = _ws_obj(workspace, dev)
    ws = wso.get(workspace_bytes(dims, max(lens), 1), stream)
    _check(lib().mage_exact_attn_paged(ctypes.byref(dims), _bf16_ptr(q, "q"), ctypes.byref(kv),
                                       _ptr(o), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)),
           "mage_exact_attn_paged")
    wso.done(stream)
    return o, lse


def sparse_attn(q, k_cache, v_cache, idx, scale: float, *, o=None, lse=None, workspace=None,
                stream=None):
    """A later step: attention over k_cache/v_cache rows idx[s][h][:] (any order, -1 skipped)."""
    S, B, Hq, d = q.shape
    _, Hkv, N, _ = k_cache.shape
    k = idx.shape[-1]
    if idx.dtype != torch.int32 or not idx.is_contiguous() or tuple(idx.shape[:2]) != (S, Hkv):
        raise ValueError("idx must be contiguous int32 [S][Hkv][k]")
    dims = make_dims(q, Hkv, scale)
    dev = q.device
    o = _out(o, (S, B, Hq, d), torch.float32, dev)
    lse = _out(lse, (S, B, Hq), torch.float32, dev)
    wso = _ws_obj(workspace, dev)
    ws = wso.get(workspace_bytes(dims, N, k), stream)
    _check(lib().mage_sparse_attn(ctypes.byref(dims), _bf16_ptr(q, "q"),
                                  _bf16_ptr(k_cache, "k_cache"), _bf16_ptr(v_cache, "v_cache"), N,
                                  _ptr(idx), int(k), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(),
                                  _stream(stream)), "mage_sparse_attn")
    wso.done(stream)
    return o, lse


def sparse_attn_noalloc(q, k_cache, v_cache, idx, scale: float, *, o, lse=None, stream=None):
    """sparse_attn with the library's fixed scratch instead of a workspace: the
    call allocates nothing (o, and lse if given, are the caller's)."""
    S, B, Hq, d = q.shape
    _, Hkv, N, _ = k_cache.shape
    k = idx.shape[-1]
    if idx.dtype != torch.int32 or not idx.is_contiguous() or tuple(idx.shape[:2]) != (S, Hkv):
        raise ValueError("idx must be contiguous int32 [S][Hkv][k]")
    dims = make_dims(q, Hkv, scale)
    o = _out(o, (S, B, Hq, d), torch.float32, q.device)
    if lse is not None:
        lse = _out(lse, (S, B, Hq), torch.float32, q.device)
    _check(lib().mage_sparse_attn_noalloc(ctypes.byref(dims), _bf16_ptr(q, "q"), _bf16_ptr(k_cache, "k_cache"),
                                          _bf16_ptr(v_cache, "v_cache"), N, _ptr(idx), int(k), _ptr(o), _ptr(lse),
                                          _stream(stream)), "mage_sparse_attn_noalloc")
    return o, lse


def sparse_attn_paged(q, k_pool, v_pool, page_table, seq_lens, idx, scale: float, *, o=None,
                      lse=None, workspace=None, stream=None):
    """A later step over a paged cache; idx holds logical positions."""
    S, B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    k = idx.shape[-1]
    if idx.dtype != torch.int32 or not idx.is_contiguous() or tuple(idx.shape[:2]) != (S, Hkv):
        raise ValueError("idx must be contiguous int32 [S][Hkv][k]")
    dims = make_dims(q, Hkv, scale)
    kv, keep, lens = _paged(k_pool, v_pool, page_table, seq_lens)
    dev = q.device
    o = _out(o, (S, B, Hq, d), torch.float32, dev)
    lse = _out(lse, (S, B, Hq), torch.float32, dev)
    wso = _ws_obj(workspace, dev)
    ws = wso.get(workspace_bytes(dims, max(lens), k), stream)
    _check(lib().mage_sparse_attn_paged(ctypes.byref(dims), _bf16_ptr(q, "q"), ctypes.byref(kv),
                                        _ptr(idx), int(k), _ptr(o), _ptr(lse), _ptr(ws),
                                        ws.numel(), _stream(stream)), "mage_sparse_attn_paged")
    wso.done(stream)
    return o, lse


def _block_rows(q, Hkv, k_blk, v_blk):
    S, B, _, d = q.shape
    for t, name in ((k_blk, "k_blk"), (v_blk, "v_blk")):
        if tuple(t.shape) != (S, Hkv, B, d):
            raise ValueError(f"{name} must be [S][Hkv][B][d] = {(S, Hkv, B, d)}")
    return _bf16_ptr(k_blk, "k_blk"), _bf16_ptr(v_blk, "v_blk")


def sparse_block_attn(q, k_cache, v_cache, idx, k_blk, v_blk, scale: float, *, o=None, lse=None,
                      workspace=None, stream=None):
    """A later step over the idx rows of the prefix together with the block's own
    rows k_blk/v_blk [S][Hkv][B][d], in one pass."""
    S, B, Hq, d = q.shape
    _, Hkv, N, _ = k_cache.shape
    k = idx.shape[-1]
    if idx.dtype != torch.int32 or not idx.is_contiguous() or tuple(idx.shape[:2]) != (S, Hkv):
        raise ValueError("idx must be contiguous int32 [S][Hkv][k]")
    kb, vb = _block_rows(q, Hkv, k_blk, v_blk)
    dims = make_dims(q, Hkv, scale)
    dev = q.device
    o = _out(o, (S, B, Hq, d), torch.float32, dev)
    lse = _out(lse, (S, B, Hq), torch.float32, dev)
    wso = _ws_obj(workspace, dev)
    ws = wso.get(workspace_bytes(dims, N, k), stream)
    _check(lib().mage_sparse_block_attn(ctypes.byref(dims), _bf16_ptr(q, "q"),
                                        _bf16_ptr(k_cache, "k_cache"), _bf16_ptr(v_cache, "v_cache"), N,
                                        _ptr(idx), int(k), kb, vb, _ptr(o), _ptr(lse), _ptr(ws),
                                        ws.numel(), _stream(stream)), "mage_sparse_block_attn")
    wso.done(stream)
    return o, lse


def sparse_block_attn_paged(q, k_pool, v_pool, page_table, seq_lens, idx, k_blk, v_blk, scale: float, *,
                            o=None, lse=None, workspace=None, stream=None):
    """sparse_block_attn over a paged cache; idx holds logical positions."""
    S, B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    k = idx.shape[-1]
    if idx.dtype != torch.int32 or not idx.is_contiguous() or tuple(idx.shape[:2]) != (S, Hkv):
        raise ValueError("idx must be contiguous int32 [S][Hkv][k]")
    kb, vb = _block_rows(q, Hkv, k_blk, v_blk)
    dims = make_dims(q, Hkv, scale)
    kv, keep, lens = _paged(k_pool, v_pool, page_table, seq_lens)
    dev = q.device
    o = _out(o, (S, B, Hq, d), torch.float32, dev)
    lse = _out(lse, (S, B, Hq), torch.float32, dev)
    wso = _ws_obj(workspace, dev)
    ws = wso.get(workspace_bytes(dims, max(lens), k), stream)
    _check(lib().mage_sparse_block_attn_paged(ctypes.byref(dims), _bf16_ptr(q, "q"), ctypes.byref(kv),
                                              _ptr(idx), int(k), kb, vb, _ptr(o), _ptr(lse), _ptr(ws),
                                              ws.numel(), _stream(stream)), "mage_sparse_block_attn_paged")
    wso.done(stream)
    return o, lse


def block_attn(q, k_blk, v_blk, o_prefix, lse_prefix, scale: float, *, o=None, lse=None, stream=None):
    """The block's queries over the prefix part (o_prefix, lse_prefix from a
    prefix pass) together with the block's own keys k_blk/v_blk [S][Hkv][B][d];
    o / lse may be the prefix tensors themselves (in place)."""
    S, B, Hq, d = q.shape
    Hkv = k_blk.shape[1]
    if tuple(k_blk.shape) != (S, Hkv, B, d) or tuple(v_blk.shape) != (S, Hkv, B, d):
        raise ValueError("k_blk and v_blk must be [S][Hkv][B][d]")
    for t, shape, name in ((o_prefix, (S, B, Hq, d), "o_prefix"), (lse_prefix, (S, B, Hq), "lse_prefix")):
        if tuple(t.shape) != shape or t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous fp32 CUDA tensor of shape {shape}")
    dims = make_dims(q, Hkv, scale)
    dev = q.device
    o = _out(o, (S, B, Hq, d), torch.float32, dev)
    lse = _out(lse, (S, B, Hq), torch.float32, dev)
    _check(lib().mage_block_attn(ctypes.byref(dims), _bf16_ptr(q, "q"), _bf16_ptr(k_blk, "k_blk"),
                                 _bf16_ptr(v_blk, "v_blk"), _ptr(o_prefix), _ptr(lse_prefix), _ptr(o),
                                 _ptr(lse), _stream(stream)), "mage_block_attn")
    return o, lse


def topk(scores, k: int, lens=None, *, idx=None, workspace=None, stream=None):
    """Top-k per row of non-negative fp32 scores [rows][n]; ties to the lower position."""
    if scores.dtype != torch.float32 or not scores.is_cuda or scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be a 2-D fp32 CUDA tensor with unit column stride")
    rows, n = scores.shape
    idx = _out(idx, (rows, k), torch.int32, scores.device)
    keep = None
    lp = None
    if lens is not None:
        lens = [int(x) for x in (lens.tolist() if torch.is_tensor(lens) else lens)]
        keep = (ctypes.c_int32 * rows)(*lens)
        lp = ctypes.cast(keep, ctypes.POINTER(ctypes.c_int32))
    dims = Dims(rows, 1, 1, 1, 64, 1.0)
    wso = _ws_obj(workspace, scores.device)
    ws = wso.get(workspace_bytes(dims, n, k), stream)
    _check(lib().mage_topk(rows, _ptr(scores), scores.stride(0), lp, n, int(k), _ptr(idx),
                           _ptr(ws), ws.numel(), _stream(stream)), "mage_topk")
    wso.done(stream)
    return idx


def arm_kernel_timers(events):
    """Arm [(start, stop), ...] torch.cuda.Event pairs (timing enabled) for the
    kernels of the next call on this thread, in launch order."""
    n = len(events)
    if n > MAX_TIMED_LAUNCHES:
        raise ValueError(f"at most {MAX_TIMED_LAUNCHES} timed launches")
    starts = (ctypes.c_void_p * max(n, 1))()
    stops = (ctypes.c_void_p * max(n, 1))()
    for i, (a, b) in enumerate(events):
        for ev in (a, b):
            if ev.cuda_event == 0:   # torch creates the HIP event on first record
                ev.record()
        starts[i], stops[i] = a.cuda_event, b.cuda_event
    _check(lib().mage_arm_kernel_timers(starts, stops, n), "mage_arm_kernel_timers")


def last_launches() -> list:
    """Names of the kernels that the last call on this thread launched."""
    n = int(lib().mage_last_launches(None, 0))
    buf = (ctypes.c_char_p * max(n, 1))()
    lib().mage_last_launches(buf, n)
    return [buf[i].decode() for i in range(min(n, MAX_TIMED_LAUNCHES))]
