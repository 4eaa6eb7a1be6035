"""Paged calls over more than MAGE_MAX_SEQS (256) sequences.

Such a call runs as consecutive groups of at most 256 sequences on its
stream. Every paged entry point is called on 300 sequences and must give,
bit for bit, what the same call gives on sequences 0..255 and 256..299
separately. The step-1 and later-step outputs must also equal the fp64
oracle. The same holds for the standalone top-k with per-row lengths.
"""
import numpy as np
import pytest
import torch

import block_sparse_kv_amd as mage
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-3
BAND = 1e-6
S_TOTAL = 300


def _inputs():
    rng = np.random.default_rng(300)
    lens = tuple(int(x) for x in rng.integers(24, 160, S_TOTAL))
    w = workloads.custom(lens, 4, 2, 64, 4, 20, paged=True, steps=2, seed=300, name="s300")
    return w, workloads.make_inputs(w, steps=2)


def _parts(n):
    return [slice(0, mage.MAX_SEQS), slice(mage.MAX_SEQS, n)]


def _equal(full, parts, lens=None, score_at=None):
    """Every output of the grouped call equals the groups' outputs, concatenated.
    The score output (index score_at; its rows are as long as the call's longest
    prefix) is compared over each sequence's prefix."""
    for j, a in enumerate(full):
        if a is None:
            continue
        pieces = [p[j] for p in parts]
        if j == score_at:
            s0 = 0
            for b in pieces:
                for s in range(b.shape[0]):
                    n = lens[s0 + s]
                    assert torch.equal(a[s0 + s, :, :n], b[s, :, :n]), (j, s0 + s)
                s0 += b.shape[0]
        else:
            assert torch.equal(a, torch.cat(pieces)), j


def test_paged_calls_over_more_than_256_sequences():
    w, inp = _inputs()
    lens = list(w.seq_lens)
    print(f"[case] {S_TOTAL} paged sequences, lens {min(lens)}..{max(lens)}", flush=True)
    q1, q2 = inp.q1.to(DEV), inp.q_steps[0].to(DEV)
    kp, vp, tab = inp.k_pool.to(DEV), inp.v_pool.to(DEV), inp.page_table.to(DEV)
    sl = _parts(S_TOTAL)

    def both(fn, *per_seq, **kw):
        """fn over all sequences, then over each group's sequences."""
        full = fn(*(x for x in per_seq), tab, lens, **kw)
        parts = [fn(*(x[s] for x in per_seq), tab[s], lens[s], **kw) for s in sl]
        torch.cuda.synchronize()
        return full, parts

    # step 1 with selection: grouped == split, and == the oracle
    sel = lambda q, t, n: mage.select_exact_paged(q, kp, vp, t, n, w.k, w.scale)   # noqa: E731
    full, parts = both(sel, q1)
    _equal(full, parts, lens, score_at=3)
    o, lse, idx, sc = full
    O, LSE, SC, IDX = oracle.select_exact_paged(inp.q1, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens,
                                                w.scale, w.k)
    assert np.abs(o.cpu().double().numpy() - O).max() <= TOL
    assert np.abs(lse.cpu().double().numpy() - LSE).max() <= TOL
    g_idx, g_sc = idx.cpu().numpy(), sc.cpu().double().numpy()
    for s, n in enumerate(lens):
        for h in range(w.num_kv_heads):
            assert abs(g_sc[s, h, :n].sum() - 1.0) < 1e-5
            assert np.abs(g_sc[s, h, :n] - SC[s][h]).max() <= 1e-5 * SC[s][h].max() + 1e-9
            kth = np.sort(SC[s][h])[::-1][min(w.k, n) - 1]
            diff = set(g_idx[s, h][g_idx[s, h] >= 0].tolist()) ^ set(IDX[s, h][IDX[s, h] >= 0].tolist())
            assert all(abs(SC[s][h][p] - kth) <= BAND for p in diff), (s, h)

    # the later step over that index set: grouped == split, and == the oracle
    sp = lambda q, i, t, n: mage.sparse_attn_paged(q, kp, vp, t, n, i, w.scale)   # noqa: E731
    full, parts = both(sp, q2, idx)
    _equal(full, parts)
    O2, L2 = oracle.sparse_paged(inp.q_steps[0], inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens, g_idx,
                                 w.scale)
    assert np.abs(full[0].cpu().double().numpy() - O2).max() <= TOL
    assert np.abs(full[1].cpu().double().numpy() - L2).max() <= TOL

    # the other paged entry points: grouped == split
    g = torch.Generator().manual_seed(301)
    kb = torch.randn(S_TOTAL, w.num_kv_heads, w.block, w.head_dim, generator=g).to(torch.bfloat16).to(DEV)
    vb = torch.randn(S_TOTAL, w.num_kv_heads, w.block, w.head_dim, generator=g).to(torch.bfloat16).to(DEV)
    _equal(*both(lambda q, t, n: mage.exact_attn_paged(q, kp, vp, t, n, w.scale), q1))
    _equal(*both(lambda q, i, b, c, t, n: mage.sparse_block_attn_paged(q, kp, vp, t, n, i, b, c, w.scale),
                 q2, idx, kb, vb))
    _equal(*both(lambda q, t, n: mage.select_pages_paged(q, kp, vp, t, n, 4, 5, w.scale, want_scores=True), q1),
           lens, score_at=4)
    _equal(*both(lambda q, t, n: mage.select_mean_query_paged(q, kp, vp, t, n, w.k, w.scale, want_scores=True),
                 q1), lens, score_at=1)
    full, parts = both(lambda q, t, n: mage.select_adaptive_paged(q, kp, vp, t, n, w.k, w.scale), q1)
    _equal(full, parts)
    k_seq = w.k * w.num_kv_heads
    _equal(*both(lambda q, i, c, t, n: mage.sparse_attn_counts_paged(q, kp, vp, t, n, i, c, k_seq, w.scale),
                 q2, full[2], full[3]))


def test_topk_with_lengths_over_more_than_256_rows():
    rows, n, k = S_TOTAL, 3000, 40
    sc = workloads.random_scores(rows, n, seed=302, ties="many")
    lens = [int(x) for x in np.random.default_rng(303).integers(1, n + 1, rows)]
    idx = mage.topk(sc.to(DEV), k, lens=lens)
    parts = [mage.topk(sc[s].to(DEV), k, lens=lens[s]) for s in _parts(rows)]
    torch.cuda.synchronize()
    assert torch.equal(idx, torch.cat(parts))
    got = idx.cpu().numpy()
    for r, m in enumerate(lens):
        assert np.array_equal(got[r], oracle.topk(sc[r, :m].numpy().astype(np.float64), k)[0]), r


def test_sequence_groups_with_split_head_groups():
    # 260 sequences (groups of 256 and 4) whose head groups hold R = 16 * 16 = 256 rows
    # per KV head (two sub-groups each): step 1 and the later step, grouped == split,
    # and the later step == the oracle
    rng = np.random.default_rng(310)
    lens = [int(x) for x in rng.integers(20, 90, 260)]
    w = workloads.custom(tuple(lens), 16, 1, 64, 16, 12, paged=True, steps=2, seed=310, name="s260_r256")
    inp = workloads.make_inputs(w, steps=2)
    print(f"[case] 260 paged sequences, R = {w.block * w.num_q_heads // w.num_kv_heads}", flush=True)
    q1, q2 = inp.q1.to(DEV), inp.q_steps[0].to(DEV)
    kp, vp, tab = inp.k_pool.to(DEV), inp.v_pool.to(DEV), inp.page_table.to(DEV)
    parts = _parts(len(lens))
    full = mage.select_exact_paged(q1, kp, vp, tab, lens, w.k, w.scale)
    split = [mage.select_exact_paged(q1[s], kp, vp, tab[s], lens[s], w.k, w.scale) for s in parts]
    torch.cuda.synchronize()
    _equal(full, split, lens, score_at=3)
    idx = full[2]
    o, lse = mage.sparse_attn_paged(q2, kp, vp, tab, lens, idx, w.scale)
    split = [mage.sparse_attn_paged(q2[s], kp, vp, tab[s], lens[s], idx[s], w.scale) for s in parts]
    torch.cuda.synchronize()
    _equal((o, lse), split)
    O2, L2 = oracle.sparse_paged(inp.q_steps[0], inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens,
                                 idx.cpu().numpy(), w.scale)
    assert np.abs(o.cpu().double().numpy() - O2).max() <= TOL
    assert np.abs(lse.cpu().double().numpy() - L2).max() <= TOL


def test_grouped_selection_with_a_select_stream():
    # a grouped step-1 call with a select stream: idx_ready (recorded on the select
    # stream after every group) is all a consumer waits for; the results equal the
    # same call on one stream bit for bit
    w, inp = _inputs()
    lens = list(w.seq_lens)
    q1 = inp.q1.to(DEV)
    kp, vp, tab = inp.k_pool.to(DEV), inp.v_pool.to(DEV), inp.page_table.to(DEV)
    ref = mage.select_exact_paged(q1, kp, vp, tab, lens, w.k, w.scale)
    torch.cuda.synchronize()
    side, consumer = torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)
    ready = torch.cuda.Event()
    o, lse, idx, sc = mage.select_exact_paged(q1, kp, vp, tab, lens, w.k, w.scale, select_stream=side,
                                              idx_ready=ready)
    consumer.wait_event(ready)
    with torch.cuda.stream(consumer):
        idx_copy = idx.clone()
        sc_copy = sc.clone()
    torch.cuda.synchronize()
    assert torch.equal(idx_copy, ref[2])
    _equal((sc_copy,), [(ref[3],)], lens, score_at=0)
    assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1])
