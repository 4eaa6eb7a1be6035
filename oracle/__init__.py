"""CPU oracle for block-shared top-k sparse KV attention (MAGE), fp64.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may use this package; the product path
(``block_sparse_kv_amd``) never imports it and has no CPU fallback.

The arithmetic lives in ``mage_oracle.cpp`` (plain C++17 + OpenMP, fp64,
full sort for top-k, gather-then-dense for the sparse step); this module only
marshals numpy/torch CPU arrays through ctypes and loops over sequences.
Every function follows the MAGE page ("MAGE: All-[MASK] Block Already Knows
Where to Look in Block Diffusion LLM", atlas.scime.ai summary): step-1 exact
attention of the all-[MASK] block and its per-block top-k subset
("Approach"), one subset shared by all block tokens ("Problem"), and reuse of
that subset at the later steps ("Approach").

Parity pins: every function here is pinned by tests/test_oracle_*.py against
closed forms, library routines and brute force (see those tests); none is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "mage_oracle.cpp")
_LIB_PATH = os.path.join(_DIR, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)


def build(force: bool = True) -> str:
    """Compile liboracle.so with g++ (no HIP headers, no shared sources)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["g++", "-O2", "-std=c++17", "-fopenmp", "-shared", "-fPIC",
                        "-o", tmp, _SRC], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_exact_seq.argtypes = [ctypes.c_int] * 4 + [ctypes.c_double, _u16p, _u16p, _u16p,
                                                             ctypes.c_int, _dp, _dp, _dp]
        lib.oracle_sparse_seq.argtypes = [ctypes.c_int] * 4 + [ctypes.c_double, _u16p, _u16p, _u16p,
                                                              ctypes.c_int, _i32p, ctypes.c_int, _dp, _dp]
        lib.oracle_topk.argtypes = [_dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p]
        lib.oracle_block_seq.argtypes = [ctypes.c_int] * 4 + [ctypes.c_double, _u16p, _u16p, _u16p,
                                                             ctypes.c_int, _i32p, ctypes.c_int, _u16p,
                                                             _u16p, _dp, _dp]
        lib.oracle_depage.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p,
                                      ctypes.c_int, _u16p]
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        for f in (lib.oracle_exact_seq, lib.oracle_sparse_seq, lib.oracle_topk, lib.oracle_depage,
                  lib.oracle_block_seq):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the oracle's OpenMP regions use."""
    return int(_load().oracle_num_threads())


def _u16(t) -> np.ndarray:
    """bf16 torch tensor (or uint16 array) -> contiguous uint16 numpy view."""
    if isinstance(t, torch.Tensor):
        assert t.dtype == torch.bfloat16 and t.device.type == "cpu"
        return np.ascontiguousarray(t.contiguous().view(torch.int16).numpy().view(np.uint16))
    return np.ascontiguousarray(t, dtype=np.uint16)


def _ptr(a: np.ndarray, typ):
    return a.ctypes.data_as(typ)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


def exact(q, k, v, scale: float, seq_lens=None):
    """Exact attention + block-averaged score, contiguous cache.

    q: bf16 [S][B][Hq][d]; k, v: bf16 [S][Hkv][N][d]. With ``seq_lens`` only
    the first N_s rows of sequence s take part (ragged batch in a padded
    array). Returns (O [S][B][Hq][d], lse [S][B][Hq], score list of
    [Hkv][N_s]) as float64 numpy arrays.
    """
    lib = _load()
    qn, kn, vn = _u16(q), _u16(k), _u16(v)
    S, B, Hq, d = qn.shape
    _, Hkv, N, _ = kn.shape
    O = np.zeros((S, B, Hq, d))
    lse = np.zeros((S, B, Hq))
    scores = []
    for s in range(S):
        n = N if seq_lens is None else int(seq_lens[s])
        ks = np.ascontiguousarray(kn[s, :, :n])
        vs = np.ascontiguousarray(vn[s, :, :n])
        qs = np.ascontiguousarray(qn[s])
        Os = np.zeros((B, Hq, d))
        ls = np.zeros((B, Hq))
        sc = np.zeros((Hkv, n))
        _check(lib.oracle_exact_seq(B, Hq, Hkv, d, float(scale), _ptr(qs, _u16p), _ptr(ks, _u16p),
                                    _ptr(vs, _u16p), n, _ptr(Os, _dp), _ptr(ls, _dp),
                                    _ptr(sc, _dp)), "exact")
        O[s], lse[s] = Os, ls
        scores.append(sc)
    return O, lse, scores


def topk(score_rows, k: int) -> np.ndarray:
    """Top-k per row under (score desc, position asc); ascending output, -1 padded.

    score_rows: [rows][N] array-like (fp32 inputs are widened exactly).
    """
    lib = _load()
    a = np.ascontiguousarray(np.asarray(score_rows, dtype=np.float64))
    if a.ndim == 1:
        a = a[None]
    rows, n = a.shape
    idx = np.zeros((rows, k), dtype=np.int32)
    _check(lib.oracle_topk(_ptr(a, _dp), rows, n, int(k), _ptr(idx, _i32p)), "topk")
    return idx


def select_exact(q, k, v, scale: float, topk_k: int, seq_lens=None):
    """Step 1 of a block: exact O, lse, per-(seq, KV head) score, and top-k idx.

    Returns (O, lse, scores, idx) with idx int32 [S][Hkv][topk_k].
    """
    O, lse, scores = exact(q, k, v, scale, seq_lens)
    idx = np.stack([topk(sc, topk_k) for sc in scores])
    return O, lse, scores, idx


def sparse(q, k, v, idx, scale: float, seq_lens=None):
    """Later-step attention over the gathered rows idx[s][h][:] (gather-then-dense)."""
    lib = _load()
    qn, kn, vn = _u16(q), _u16(k), _u16(v)
    S, B, Hq, d = qn.shape
    _, Hkv, N, _ = kn.shape
    idn = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    kk = idn.shape[-1]
    O = np.zeros((S, B, Hq, d))
    lse = np.zeros((S, B, Hq))
    for s in range(S):
        n = N if seq_lens is None else int(seq_lens[s])
        ks = np.ascontiguousarray(kn[s, :, :n])
        vs = np.ascontiguousarray(vn[s, :, :n])
        qs = np.ascontiguousarray(qn[s])
        ids = np.ascontiguousarray(idn[s])
        Os = np.zeros((B, Hq, d))
        ls = np.zeros((B, Hq))
        _check(lib.oracle_sparse_seq(B, Hq, Hkv, d, float(scale), _ptr(qs, _u16p), _ptr(ks, _u16p),
                                     _ptr(vs, _u16p), n, _ptr(ids, _i32p), kk, _ptr(Os, _dp),
                                     _ptr(ls, _dp)), "sparse")
        O[s], lse[s] = Os, ls
    return O, lse


def block(q, k, v, idx, k_blk, v_blk, scale: float, seq_lens=None):
    """Block attention: the block's queries over the prefix rows idx[s][h][:]
    (idx None: every prefix row) together with the block's own rows
    k_blk/v_blk [S][Hkv][B][d], as one softmax over the union."""
    lib = _load()
    qn, kn, vn = _u16(q), _u16(k), _u16(v)
    kbn, vbn = _u16(k_blk), _u16(v_blk)
    S, B, Hq, d = qn.shape
    _, Hkv, N, _ = kn.shape
    if kbn.shape != (S, Hkv, B, d) or vbn.shape != (S, Hkv, B, d):
        raise ValueError("k_blk and v_blk must be [S][Hkv][B][d]")
    idn = None if idx is None else np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    kk = 0 if idn is None else idn.shape[-1]
    O = np.zeros((S, B, Hq, d))
    lse = np.zeros((S, B, Hq))
    for s in range(S):
        n = N if seq_lens is None else int(seq_lens[s])
        ks = np.ascontiguousarray(kn[s, :, :n])
        vs = np.ascontiguousarray(vn[s, :, :n])
        ids = None if idn is None else np.ascontiguousarray(idn[s])
        Os = np.zeros((B, Hq, d))
        ls = np.zeros((B, Hq))
        _check(lib.oracle_block_seq(B, Hq, Hkv, d, float(scale), _ptr(np.ascontiguousarray(qn[s]), _u16p),
                                    _ptr(ks, _u16p), _ptr(vs, _u16p), n,
                                    None if ids is None else _ptr(ids, _i32p), kk,
                                    _ptr(np.ascontiguousarray(kbn[s]), _u16p),
                                    _ptr(np.ascontiguousarray(vbn[s]), _u16p), _ptr(Os, _dp), _ptr(ls, _dp)),
               "block")
        O[s], lse[s] = Os, ls
    return O, lse


def depage(pool, page_table, seq_lens, num_kv_heads: int | None = None):
    """Copy a page pool [P][Hkv][page][d] back to per-sequence [Hkv][N_s][d] uint16 arrays."""
    lib = _load()
    pn = _u16(pool)
    P, Hkv, page, d = pn.shape
    tab = np.ascontiguousarray(np.asarray(page_table, dtype=np.int32))
    out = []
    for s, n in enumerate(np.asarray(seq_lens).tolist()):
        o = np.zeros((Hkv, int(n), d), dtype=np.uint16)
        row = np.ascontiguousarray(tab[s])
        _check(lib.oracle_depage(_ptr(pn, _u16p), Hkv, page, d, _ptr(row, _i32p), int(n),
                                 _ptr(o, _u16p)), "depage")
        out.append(o)
    return out


def _padded(seqs):
    """Stack per-sequence [Hkv][N_s][d] arrays into [S][Hkv][maxN][d] (zero padded)."""
    S = len(seqs)
    Hkv, _, d = seqs[0].shape
    n = max(a.shape[1] for a in seqs)
    out = np.zeros((S, Hkv, n, d), dtype=np.uint16)
    for s, a in enumerate(seqs):
        out[s, :, :a.shape[1]] = a
    return out


def select_exact_paged(q, k_pool, v_pool, page_table, seq_lens, scale: float, topk_k: int):
    """Paged step 1: de-page, then the contiguous definition per sequence."""
    kc = _padded(depage(k_pool, page_table, seq_lens))
    vc = _padded(depage(v_pool, page_table, seq_lens))
    return select_exact(q, kc, vc, scale, topk_k, seq_lens=np.asarray(seq_lens))


def block_paged(q, k_pool, v_pool, page_table, seq_lens, idx, k_blk, v_blk, scale: float):
    """Block attention over a paged prefix: de-page, then as block()."""
    kc = _padded(depage(k_pool, page_table, seq_lens))
    vc = _padded(depage(v_pool, page_table, seq_lens))
    return block(q, kc, vc, idx, k_blk, v_blk, scale, seq_lens=np.asarray(seq_lens))


def sparse_paged(q, k_pool, v_pool, page_table, seq_lens, idx, scale: float):
    """Paged later step: de-page, then gather-then-dense per sequence."""
    kc = _padded(depage(k_pool, page_table, seq_lens))
    vc = _padded(depage(v_pool, page_table, seq_lens))
    return sparse(q, kc, vc, idx, scale, seq_lens=np.asarray(seq_lens))


# ---- anchor re-selection diagnostics: the mean-query score and set overlap ----
#
# Step-dLLM page (abstract): the sparse mask is refreshed at anchor steps and
# reused in between; the diagnostic measures how much of each step's own top-k
# set the set in use still covers. MAGE page ("Approach") motivates the block
# query with the block-average query; read literally, the probability under the
# mean query is an alternative to the averaged probability that the main path
# uses. Both functions below are exact (rational arithmetic, plain sets).

def _bf16_bits_of(x) -> int:
    """Round an exact rational to the nearest bf16 (8 significant bits, ties to
    even) and return its 16-bit pattern. x must be 0 or of magnitude in the
    normal range [2^-126, 2^128)."""
    from fractions import Fraction
    x = Fraction(x)
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    a = -x if x < 0 else x
    e = a.numerator.bit_length() - a.denominator.bit_length()   # 2^e <= a < 2^(e+2)
    if a < Fraction(2) ** e:
        e -= 1
    elif a >= Fraction(2) ** (e + 1):
        e += 1
    if not -126 <= e < 128:
        raise ValueError("value outside the bf16 normal range")
    ulp = Fraction(2) ** (e - 7)
    q, r = divmod(a, ulp)
    half = ulp / 2
    if r > half or (r == half and q % 2 == 1):
        q += 1
    v = float(q * ulp)                    # at most 9 significant bits: exact in fp32
    return sign | (int(np.array(v, dtype=np.float32).view(np.uint32)) >> 16)


def mean_query(q, num_kv_heads: int):
    """The block's mean query per (sequence, KV head): the exact mean of the
    B*G bf16 query rows that share KV head h (tokens b, heads h*G + g), rounded
    once to bf16 (nearest, ties to even). q: bf16 [S][B][Hq][d]; returns a bf16
    tensor [S][1][Hkv][d], the query of a one-token, one-head-per-group block."""
    from fractions import Fraction
    qn = _u16(q)
    S, B, Hq, d = qn.shape
    Hkv = int(num_kv_heads)
    G = Hq // Hkv
    vals = qn.astype(np.uint32) << 16
    f = vals.view(np.float32).astype(np.float64)          # exact widening
    out = np.zeros((S, 1, Hkv, d), dtype=np.uint16)
    for s in range(S):
        for h in range(Hkv):
            rows = f[s, :, h * G:(h + 1) * G, :].reshape(B * G, d)
            for e in range(d):
                tot = sum((Fraction(float(v)) for v in rows[:, e]), Fraction(0))
                out[s, 0, h, e] = _bf16_bits_of(tot / (B * G))
    return torch.from_numpy(out.view(np.int16)).view(torch.bfloat16)


def select_mean_query(q, k, v, scale: float, topk_k: int, seq_lens=None):
    """Top-k by the probability under the mean query: step-1 selection with the
    block replaced by its mean query (one row per KV head). Returns (scores,
    idx) as select_exact does."""
    Hkv = np.asarray(_u16(k)).shape[1]
    qm = mean_query(q, Hkv)
    _, _, scores, idx = select_exact(qm, k, v, scale, topk_k, seq_lens)
    return scores, idx


def select_mean_query_paged(q, k_pool, v_pool, page_table, seq_lens, scale: float, topk_k: int):
    kc = _padded(depage(k_pool, page_table, seq_lens))
    vc = _padded(depage(v_pool, page_table, seq_lens))
    return select_mean_query(q, kc, vc, scale, topk_k, seq_lens=np.asarray(seq_lens))


def idx_overlap(a, b):
    """Per row of two index lists [rows][k] (entries < 0 are padding): the size
    of the intersection of their valid entries, and the number of valid
    entries of each. Returns three int64 arrays (common, count_a, count_b);
    the recall of a against the reference b is common / count_b."""
    a = np.asarray(a).reshape(-1, np.asarray(a).shape[-1])
    b = np.asarray(b).reshape(-1, np.asarray(b).shape[-1])
    common, ca, cb = [], [], []
    for ra, rb in zip(a.tolist(), b.tolist()):
        sa = {x for x in ra if x >= 0}
        sb = {x for x in rb if x >= 0}
        common.append(len(sa & sb))
        ca.append(len(sa))
        cb.append(len(sb))
    return np.array(common), np.array(ca), np.array(cb)


# ---- page-granular selection ----
#
# The block-sparse view of the same selection (Step-dLLM page, abstract: a
# block-sparse mask; the KV cache's pages as the unit of a gather): positions
# are grouped into pages of P consecutive positions, a page's score is the
# sum of its positions' block-averaged scores, and the top pages by that score
# are kept whole.

def page_scores(score_row, page_tokens: int) -> np.ndarray:
    """Sum of the scores of each run of page_tokens consecutive positions (the
    last page holds what is left), fp64."""
    a = np.asarray(score_row, dtype=np.float64)
    n = a.shape[-1]
    npg = -(-n // page_tokens)
    pad = np.zeros(npg * page_tokens - n)
    return np.concatenate([a, pad]).reshape(npg, page_tokens).sum(axis=1)


def pages_to_positions(page_idx, page_tokens: int, n: int) -> np.ndarray:
    """Expand ascending page ids (negative: none) into their positions, page by
    page: row of len(page_idx) * page_tokens entries, -1 for positions past n
    or slots of a missing page."""
    out = []
    for pg in np.asarray(page_idx).tolist():
        for t in range(page_tokens):
            p = pg * page_tokens + t
            out.append(p if pg >= 0 and p < n else -1)
    return np.array(out, dtype=np.int32)


def select_pages(q, k, v, scale: float, page_tokens: int, k_pages: int, seq_lens=None):
    """Step 1 with page-granular selection. Returns (scores list of [Hkv][N_s],
    page_idx int32 [S][Hkv][k_pages] ascending with -1 padding, idx int32
    [S][Hkv][k_pages * page_tokens] of positions)."""
    _, _, scores, _ = select_exact(q, k, v, scale, 1, seq_lens)
    S = len(scores)
    Hkv = scores[0].shape[0]
    pidx = np.zeros((S, Hkv, k_pages), dtype=np.int32)
    idx = np.zeros((S, Hkv, k_pages * page_tokens), dtype=np.int32)
    for s in range(S):
        n = scores[s].shape[1]
        for h in range(Hkv):
            pidx[s, h] = topk(page_scores(scores[s][h], page_tokens), k_pages)[0]
            idx[s, h] = pages_to_positions(pidx[s, h], page_tokens, n)
    return scores, pidx, idx


def select_pages_paged(q, k_pool, v_pool, page_table, seq_lens, scale: float, page_tokens: int, k_pages: int):
    kc = _padded(depage(k_pool, page_table, seq_lens))
    vc = _padded(depage(v_pool, page_table, seq_lens))
    return select_pages(q, kc, vc, scale, page_tokens, k_pages, seq_lens=np.asarray(seq_lens))


# ---- head-adaptive budgets ----
#
# Step-dLLM page (abstract): one global budget per sequence, shared by its
# heads so that heads whose attention is concentrated are compressed harder.
# Read here: the sequence keeps the K = k * Hkv largest block-averaged scores
# over all of its (KV head, position) pairs, ties to the lower head, then the
# lower position; head h's budget k_h is how many of them are its own. Each
# head's scores sum to one, so a head whose mass sits on few positions wins
# few slots and a head with diffuse mass wins many.

def select_adaptive(q, k, v, scale: float, topk_k: int, seq_lens=None):
    """Step 1 with head-adaptive budgets. Returns (scores list of [Hkv][N_s],
    idx int32 [S][Hkv][k * Hkv] ascending positions then -1, counts int64
    [S][Hkv])."""
    _, _, scores, _ = select_exact(q, k, v, scale, 1, seq_lens)
    S = len(scores)
    Hkv, _ = scores[0].shape
    K = topk_k * Hkv
    idx = np.full((S, Hkv, K), -1, dtype=np.int32)
    counts = np.zeros((S, Hkv), dtype=np.int64)
    for s in range(S):
        n = scores[s].shape[1]
        flat = scores[s].reshape(-1)                       # (h, p) -> h * n + p
        chosen = topk(flat, min(K, flat.size))[0]
        chosen = chosen[chosen >= 0]
        for h in range(Hkv):
            mine = chosen[(chosen >= h * n) & (chosen < (h + 1) * n)] - h * n
            counts[s, h] = mine.size
            idx[s, h, :mine.size] = np.sort(mine)
    return scores, idx, counts


def select_adaptive_paged(q, k_pool, v_pool, page_table, seq_lens, scale: float, topk_k: int):
    kc = _padded(depage(k_pool, page_table, seq_lens))
    vc = _padded(depage(v_pool, page_table, seq_lens))
    return select_adaptive(q, kc, vc, scale, topk_k, seq_lens=np.asarray(seq_lens))
