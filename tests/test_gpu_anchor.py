"""Anchor re-selection diagnostics on the GPU against the oracle: the block's
mean query (bit-exact), selection by the probability under it (index sets
within the 1e-6 tie band, scores to 1e-5 relative), the overlap of two index
sets (bit-exact counts), and the recall of a step-1 set against later steps'
own sets (Step-dLLM page, abstract: sets chosen at anchor steps and reused in
between).
"""
import numpy as np
import pytest
import torch

import block_sparse_kv_amd as mage
import oracle
import workloads
from test_gpu_parity import DEV, SMALL, check_idx, dev_inputs, gpu_select, ora_select

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("S,B,Hq,Hkv,d,seed", [
    (1, 32, 32, 8, 128, 1),     # R = 128
    (2, 5, 8, 2, 64, 2),        # R = 20: a divisor that is not a power of two
    (1, 33, 2, 2, 128, 3),      # R = 33
    (3, 1, 4, 4, 64, 4),        # R = 1: the query itself
    (1, 16, 16, 1, 64, 5),      # R = 256 > 128 rows per KV head (the mean needs no row blocks)
])
def test_mean_query_bits_match_oracle(S, B, Hq, Hkv, d, seed):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(S, B, Hq, d, generator=g) * 0.3).to(torch.bfloat16)
    got = mage.mean_query(q.to(DEV), Hkv)
    torch.cuda.synchronize()
    want = oracle.mean_query(q, Hkv)
    assert np.array_equal(_bits(got), _bits(want))


def test_mean_query_of_a_planted_workload_matches_oracle():
    w = workloads.custom((512,), 32, 8, 128, 32, 64, name="mq")
    inp = workloads.make_inputs(w)
    got = mage.mean_query(inp.q1.to(DEV), 8)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(got), _bits(oracle.mean_query(inp.q1, 8)))


MQ_CASES = [SMALL[i] for i in (0, 2, 3, 4, 6, 8, 12)] + [w for w in SMALL if w.name.endswith("_groups")]   # R > 128


@pytest.mark.parametrize("w", MQ_CASES, ids=[w.name for w in MQ_CASES])
def test_select_mean_query_matches_oracle(w):
    inp = workloads.make_inputs(w)
    d = dev_inputs(inp)
    print(f"[case] mean query {w.name} lens={w.seq_lens} B={w.block} k={w.k}", flush=True)
    if w.paged:
        idx, sc = mage.select_mean_query_paged(d["q1"], d["k_pool"], d["v_pool"], d["table"], d["lens"], w.k,
                                               w.scale, want_scores=True)
        SC, IDX = oracle.select_mean_query_paged(inp.q1, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens,
                                                 w.scale, w.k)
    else:
        idx, sc = mage.select_mean_query(d["q1"], d["k"], d["v"], w.k, w.scale, want_scores=True)
        SC, IDX = oracle.select_mean_query(inp.q1, inp.k, inp.v, w.scale, w.k)
    torch.cuda.synchronize()
    lens = w.seq_lens
    for s in range(w.num_seqs):
        for h in range(w.num_kv_heads):
            g = sc[s, h, :lens[s]].cpu().double().numpy()
            ref = SC[s][h]
            assert abs(g.sum() - 1.0) < 1e-5
            assert np.abs(g - ref).max() <= 1e-5 * ref.max() + 1e-9
    check_idx(idx, IDX, SC, w.k, lens)


def test_mean_query_selection_of_a_one_row_block_is_the_main_selection():
    # B = 1 and G = 1: the mean query is the query, so both selections run the
    # same kernels on the same bits
    w = workloads.custom((3000,), 4, 4, 128, 1, 200, name="one_row")
    inp = workloads.make_inputs(w)
    d = dev_inputs(inp)
    _, _, idx, sc = gpu_select(inp, d)
    idx2, sc2 = mage.select_mean_query(d["q1"], d["k"], d["v"], w.k, w.scale, want_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(sc, sc2)


def _idx_rows(rng, rows, k, n):
    out = np.full((rows, k), -1, dtype=np.int32)
    for r in range(rows):
        m = int(rng.integers(0, k + 1))
        out[r, :m] = np.sort(rng.choice(n, m, replace=False))
    return out


@pytest.mark.parametrize("rows,k,n", [(1, 1, 3), (7, 64, 100), (64, 1024, 131072), (3, 5000, 6000),
                                      (200, 40, 41)])
def test_idx_overlap_matches_oracle(rows, k, n):
    rng = np.random.default_rng(rows * 31 + k)
    a = _idx_rows(rng, rows, k, n)
    b = _idx_rows(rng, rows, k, n)
    b[0] = a[0]                                   # an identical pair
    if rows > 1:
        b[1, :] = -1                              # an empty reference row
    c, ca, cb = mage.idx_overlap(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV))
    torch.cuda.synchronize()
    C, CA, CB = oracle.idx_overlap(a, b)
    assert np.array_equal(c.cpu().numpy(), C)
    assert np.array_equal(ca.cpu().numpy(), CA) and np.array_equal(cb.cpu().numpy(), CB)


def test_recall_of_the_step_one_set_matches_oracle():
    # every later step's own set from its own queries (the main selection), and
    # the overlap of the step-1 set with each: GPU against oracle end to end
    w = workloads.custom((4000,), 16, 4, 128, 16, 128, steps=4, name="recall")
    inp = workloads.make_inputs(w, steps=4)
    d = dev_inputs(inp)
    qs = [inp.q1] + list(inp.q_steps)
    own_gpu, own_ora = [], []
    for t, q in enumerate(qs):
        _, _, idx, _ = mage.select_exact(q.to(DEV), d["k"], d["v"], w.k, w.scale)
        torch.cuda.synchronize()
        _, _, SC, IDX = oracle.select_exact(q, inp.k, inp.v, w.scale, w.k)
        nd = check_idx(idx, IDX, SC, w.k, w.seq_lens)
        print(f"[case] step {t + 1}: {nd} positions differ inside the tie band", flush=True)
        own_gpu.append(idx)
        own_ora.append((IDX, nd))
    for t in range(1, len(qs)):
        c, _, cb = mage.idx_overlap(own_gpu[0], own_gpu[t])
        torch.cuda.synchronize()
        C, _, CB = oracle.idx_overlap(own_ora[0][0], own_ora[t][0])
        slack = own_ora[0][1] + own_ora[t][1]     # tie-band swaps can move a count by one each
        assert np.abs(c.cpu().numpy().ravel() - C).max() <= slack
        assert np.array_equal(cb.cpu().numpy().ravel(), CB)
