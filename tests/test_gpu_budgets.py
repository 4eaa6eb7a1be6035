"""Head-adaptive budgets on the GPU against the oracle: the kept (KV head,
position) pairs of each sequence within the 1e-6 tie band of the global K-th
score, per-head counts and rows consistent with them, and the later step over
per-head counts within 2e-3 (work planned from the counts, not the row
length).
"""
import numpy as np
import pytest
import torch

import block_sparse_kv_amd as mage
import oracle
import workloads
from test_gpu_parity import BAND, DEV, TOL, dev_inputs, maxabs, ora_select, ora_sparse

pytestmark = pytest.mark.gpu


def gpu_adaptive(inp, d):
    w = inp.w
    if w.paged:
        return mage.select_adaptive_paged(d["q1"], d["k_pool"], d["v_pool"], d["table"], d["lens"], w.k, w.scale)
    return mage.select_adaptive(d["q1"], d["k"], d["v"], w.k, w.scale)


def ora_adaptive(inp):
    w = inp.w
    if w.paged:
        return oracle.select_adaptive_paged(inp.q1, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens, w.scale,
                                            w.k)
    return oracle.select_adaptive(inp.q1, inp.k, inp.v, w.scale, w.k)


def gpu_counts_step(inp, d, q, idx, counts, k_seq):
    w = inp.w
    if w.paged:
        return mage.sparse_attn_counts_paged(q, d["k_pool"], d["v_pool"], d["table"], d["lens"], idx, counts, k_seq,
                                             w.scale)
    return mage.sparse_attn_counts(q, d["k"], d["v"], idx, counts, k_seq, w.scale)


CASES = [
    workloads.custom((3000,), 32, 8, 128, 32, 64, name="gqa"),
    workloads.custom((2000,), 16, 16, 128, 8, 40, keys="clusters", name="mha_clusters"),
    workloads.custom((5000,), 8, 2, 64, 16, 300, name="d64_split"),
    workloads.custom((150,), 8, 4, 128, 8, 64, name="budget_over_one_head"),
    workloads.custom((53, 200, 1000), 8, 2, 64, 4, 64, paged=True, name="paged_ragged"),
    workloads.custom((17, 4096, 900), 32, 8, 128, 32, 256, paged=True, name="paged_r128"),
    workloads.custom((3000, 3000), 32, 8, 128, 32, 2000, name="wide_counts"),   # 1024-entry chunks
    # R > 128 rows per KV head: two sub-groups (scores summed over all rows), paged R = 192
    workloads.custom((3000,), 16, 2, 128, 32, 300, name="r256_budgets"),
    workloads.custom((900, 2500), 24, 2, 64, 16, 128, paged=True, name="paged_r192_budgets"),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_select_adaptive_matches_oracle(w):
    inp = workloads.make_inputs(w)
    d = dev_inputs(inp)
    print(f"[case] adaptive {w.name} lens={w.seq_lens} Hkv={w.num_kv_heads} k={w.k}", flush=True)
    o, lse, idx, counts = gpu_adaptive(inp, d)
    torch.cuda.synchronize()
    SC, IDX, CNT = ora_adaptive(inp)
    O, LSE, _, _ = ora_select(inp)
    assert maxabs(o, O) <= TOL and maxabs(lse, LSE) <= TOL
    g_i, g_c = idx.cpu().numpy(), counts.cpu().numpy()
    Hkv = w.num_kv_heads
    for s in range(w.num_seqs):
        n = w.seq_lens[s]
        K = min(w.k * Hkv, n * Hkv)
        assert g_c[s].sum() == K
        flat = np.concatenate([SC[s][h] for h in range(Hkv)])
        kth = np.sort(flat)[::-1][K - 1]
        mine, ref = set(), set()
        for h in range(Hkv):
            row = g_i[s, h]
            c = int(g_c[s, h])
            assert (row[c:] == -1).all() and (np.diff(row[:c]) > 0).all()
            assert c == 0 or (row[0] >= 0 and row[c - 1] < n)
            mine |= {(h, int(p)) for p in row[:c]}
            ref |= {(h, int(p)) for p in IDX[s, h, :CNT[s, h]]}
        diff = mine ^ ref
        bad = [(h, p) for (h, p) in diff if abs(SC[s][h][p] - kth) > BAND]
        assert not bad, f"(s={s}) kept pairs differ outside the tie band at {bad[:10]}"
        assert np.abs(g_c[s] - CNT[s]).sum() <= len(diff)
    # a later step over the GPU's own rows and counts, the same rows on the oracle side
    k_seq = w.k * Hkv
    o2, lse2 = gpu_counts_step(inp, d, d["q"][0], idx, counts, k_seq)
    torch.cuda.synchronize()
    O2, L2 = ora_sparse(inp, inp.q_steps[0], g_i)
    assert maxabs(o2, O2) <= TOL and maxabs(lse2, L2) <= TOL


def test_counts_step_edges():
    # counts of 0 (O = 0, lse = -inf), counts above the row length (capped),
    # entries past a count ignored even when valid, and the same rows through
    # the plain step (rows cut to the counts with -1) agree
    w = workloads.custom((4000,), 16, 4, 128, 16, 64, name="edges")
    inp = workloads.make_inputs(w)
    d = dev_inputs(inp)
    rng = np.random.default_rng(5)
    k_row = 700
    idx = np.stack([np.stack([np.sort(rng.choice(4000, k_row, replace=False)) for _ in range(4)])]).astype(np.int32)
    counts = np.array([[0, 700, 5000, 129]], dtype=np.int32)
    cut = idx.copy()
    for h in range(4):
        cut[0, h, min(counts[0, h], k_row):] = -1
    o, lse = mage.sparse_attn_counts(d["q"][0], d["k"], d["v"], torch.from_numpy(idx).to(DEV),
                                     torch.from_numpy(counts).to(DEV), 2 * k_row + 129, w.scale)
    o_ref, l_ref = mage.sparse_attn(d["q"][0], d["k"], d["v"], torch.from_numpy(cut).to(DEV), w.scale)
    torch.cuda.synchronize()
    G = 4
    assert (o[0, :, :G] == 0).all() and torch.isinf(lse[0, :, :G]).all() and (lse[0, :, :G] < 0).all()
    assert (o[:, :, G:] - o_ref[:, :, G:]).abs().max().item() <= 1e-5
    assert (lse[:, :, G:] - l_ref[:, :, G:]).abs().max().item() <= 1e-5
    O, L = ora_sparse(inp, inp.q_steps[0], cut)
    assert maxabs(o[:, :, G:], O[:, :, G:]) <= TOL and maxabs(lse[:, :, G:], L[:, :, G:]) <= TOL
