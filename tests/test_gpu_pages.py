"""Page-granular selection on the GPU against the oracle: page ids within the
1e-6 tie band of the k-th page score, positions equal to the expansion of the
chosen pages (bit-exact), O and lse of step 1 and of a later step over the
chosen pages within 2e-3, and one-position pages equal to the position
selection bit for bit.
"""
import numpy as np
import pytest
import torch

import block_sparse_kv_amd as mage
import oracle
import workloads
from test_gpu_parity import BAND, DEV, TOL, dev_inputs, gpu_select, gpu_sparse, maxabs, ora_select, ora_sparse

pytestmark = pytest.mark.gpu


def gpu_pages(inp, d, P, kp):
    w = inp.w
    if w.paged:
        return mage.select_pages_paged(d["q1"], d["k_pool"], d["v_pool"], d["table"], d["lens"], P, kp, w.scale,
                                       want_scores=True)
    return mage.select_pages(d["q1"], d["k"], d["v"], P, kp, w.scale, want_scores=True)


def ora_pages(inp, P, kp):
    w = inp.w
    if w.paged:
        return oracle.select_pages_paged(inp.q1, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens, w.scale, P,
                                         kp)
    return oracle.select_pages(inp.q1, inp.k, inp.v, w.scale, P, kp)


CASES = [
    (workloads.custom((3000,), 8, 2, 128, 16, 64, name="p16"), 16, 8),
    (workloads.custom((2999,), 8, 2, 64, 4, 64, name="p7_ragged_tail"), 7, 20),
    (workloads.custom((5000,), 32, 8, 128, 32, 64, name="p64"), 64, 4),
    (workloads.custom((100,), 4, 1, 64, 8, 8, name="more_pages_than_exist"), 16, 9),
    (workloads.custom((3000,), 16, 2, 128, 32, 64, name="r256_pages"), 16, 8),   # R = 256: two sub-groups
    (workloads.custom((700, 1800), 24, 2, 64, 16, 64, paged=True, name="paged_r192_pages"), 16, 6),   # R = 192
    (workloads.custom((53, 200, 1000), 8, 2, 64, 4, 64, paged=True, name="paged_ragged"), 16, 4),
    (workloads.custom((17, 4096, 900), 32, 8, 128, 32, 512, paged=True, name="paged_p4"), 4, 100),
]


@pytest.mark.parametrize("w,P,kp", CASES, ids=[c[0].name for c in CASES])
def test_select_pages_matches_oracle(w, P, kp):
    inp = workloads.make_inputs(w)
    d = dev_inputs(inp)
    print(f"[case] pages {w.name} lens={w.seq_lens} P={P} k_pages={kp}", flush=True)
    o, lse, idx, pidx, sc = gpu_pages(inp, d, P, kp)
    torch.cuda.synchronize()
    SC, PIDX, IDX = ora_pages(inp, P, kp)
    O, LSE, _, _ = ora_select(inp)
    assert maxabs(o, O) <= TOL and maxabs(lse, LSE) <= TOL
    g_p = pidx.cpu().numpy()
    g_i = idx.cpu().numpy()
    for s in range(w.num_seqs):
        n = w.seq_lens[s]
        npg = -(-n // P)
        keff = min(kp, npg)
        for h in range(w.num_kv_heads):
            ps = oracle.page_scores(SC[s][h], P)
            gp = g_p[s, h]
            assert (gp[keff:] == -1).all() and (np.diff(gp[:keff]) > 0).all()
            assert gp[:keff].min() >= 0 and gp[:keff].max() < npg
            kth = np.sort(ps)[::-1][keff - 1]
            diff = set(gp[:keff].tolist()) ^ set(PIDX[s, h, :keff].tolist())
            bad = [g for g in diff if abs(ps[g] - kth) > BAND]
            assert not bad, f"(s={s}, h={h}) pages differ outside the tie band at {bad[:10]}"
            # positions: the expansion of the GPU's own pages
            assert np.array_equal(g_i[s, h], oracle.pages_to_positions(gp, P, n))
            # the GPU's position scores (the page scores' inputs) match the oracle's
            g = sc[s, h, :n].cpu().double().numpy()
            assert np.abs(g - SC[s][h]).max() <= 1e-5 * SC[s][h].max() + 1e-9
    # a later step over the chosen pages, the same index rows on both sides
    o2, lse2 = gpu_sparse(inp, d, d["q"][0], idx)
    torch.cuda.synchronize()
    O2, L2 = ora_sparse(inp, inp.q_steps[0], g_i)
    assert maxabs(o2, O2) <= TOL and maxabs(lse2, L2) <= TOL


@pytest.mark.parametrize("paged", [False, True])
def test_one_position_pages_are_the_position_selection(paged):
    w = workloads.custom((700, 1500) if paged else (2000,), 16, 4, 128, 16, 96, paged=paged, name="p1")
    inp = workloads.make_inputs(w)
    d = dev_inputs(inp)
    _, _, idx, _ = gpu_select(inp, d)
    _, _, idx1, pidx1, _ = gpu_pages(inp, d, 1, w.k)
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx) and torch.equal(pidx1, idx)
