"""Parity at the full workload sizes, in the launch configuration bench.py times.

The whole batch runs on the GPU through the C ABI (default plan, default
workspace); the fp64 oracle recomputes every (sequence, KV head) unit one by
one (each is a plain, independent definition per unit). Bars as in
test_gpu_parity: O and lse max-abs <= 2e-3, idx equal outside the 1e-6 tie
band of the k-th oracle score, scores relative 1e-5; every unit's GPU scores
also sum to 1 and its idx row is ascending inside [0, N_s), then -1.
"""
import numpy as np
import pytest
import torch

import block_sparse_kv_amd as mage
import oracle
import workloads

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

DEV = "cuda:0"
TOL = 2e-3
BAND = 1e-6

# every (seq, KV head) unit of each large workload: 8, 8, 16 and 64 units
CASES = ["gqa32k", "head128k", "mha64k", "ragged"]


def unit_inputs(inp, s, h):
    """One unit's CPU inputs: q [1][B][G][d], k, v [1][1][N_s][d] (bf16 or their bits)."""
    w = inp.w
    G = w.group
    q1 = inp.q1[s:s + 1, :, h * G:(h + 1) * G].contiguous()
    q2 = inp.q_steps[0][s:s + 1, :, h * G:(h + 1) * G].contiguous()
    if w.paged:
        n = w.seq_lens[s]
        kk = oracle.depage(inp.k_pool, inp.page_table[s:s + 1], [n])[0][h:h + 1][None]
        vv = oracle.depage(inp.v_pool, inp.page_table[s:s + 1], [n])[0][h:h + 1][None]
        k = np.ascontiguousarray(kk)  # uint16 bf16 bit patterns; the oracle takes either
        v = np.ascontiguousarray(vv)
    else:
        k = inp.k[s:s + 1, h:h + 1].contiguous()
        v = inp.v[s:s + 1, h:h + 1].contiguous()
    return q1, q2, k, v


@pytest.mark.parametrize("name", CASES)
def test_full_size_every_unit(name):
    w = workloads.CONFIG_BY_NAME[name]
    units = [(s, h) for s in range(w.num_seqs) for h in range(w.num_kv_heads)]
    print(f"[case] {name} lens={w.seq_lens[:3]}... {len(units)} units", flush=True)
    inp = workloads.make_inputs(w, steps=2)
    q1 = inp.q1.to(DEV)
    q2 = inp.q_steps[0].to(DEV)
    side = torch.cuda.Stream(device=DEV)
    ready = torch.cuda.Event()
    if w.paged:
        kp, vp = inp.k_pool.to(DEV), inp.v_pool.to(DEV)
        tab, lens = inp.page_table.to(DEV), inp.seq_lens.tolist()
        o, lse, idx, sc = mage.select_exact_paged(q1, kp, vp, tab, lens, w.k, w.scale,
                                                  select_stream=side, idx_ready=ready)
        torch.cuda.current_stream().wait_event(ready)
        o2, lse2 = mage.sparse_attn_paged(q2, kp, vp, tab, lens, idx, w.scale)
    else:
        kc, vc = inp.k.to(DEV), inp.v.to(DEV)
        o, lse, idx, sc = mage.select_exact(q1, kc, vc, w.k, w.scale, select_stream=side,
                                            idx_ready=ready)
        torch.cuda.current_stream().wait_event(ready)
        o2, lse2 = mage.sparse_attn(q2, kc, vc, idx, w.scale)
    torch.cuda.synchronize()
    G = w.group
    # invariants of every unit's GPU output, before the oracle runs
    sc_cpu, idx_cpu = sc.cpu().double().numpy(), idx.cpu().numpy()
    for s, h in units:
        n = w.seq_lens[s]
        keff = min(w.k, n)
        row = sc_cpu[s, h, :n]
        assert (row >= 0).all() and abs(row.sum() - 1.0) <= 1e-5, (name, s, h, row.sum())
        gi = idx_cpu[s, h]
        assert (gi[keff:] == -1).all() and (np.diff(gi[:keff]) > 0).all(), (name, s, h)
        assert gi[0] >= 0 and gi[keff - 1] < n, (name, s, h)
    worst = 0.0
    for s, h in units:
        n = w.seq_lens[s]
        keff = min(w.k, n)
        uq1, uq2, uk, uv = unit_inputs(inp, s, h)
        O, LSE, SC, IDX = oracle.select_exact(uq1, uk, uv, w.scale, w.k)
        go = o[s:s + 1, :, h * G:(h + 1) * G].cpu().double().numpy()
        gl = lse[s:s + 1, :, h * G:(h + 1) * G].cpu().double().numpy()
        assert np.abs(go - O).max() <= TOL, (name, s, h)
        assert np.abs(gl - LSE).max() <= TOL, (name, s, h)
        gs = sc[s, h, :n].cpu().double().numpy()
        ref = SC[0][0]
        assert np.abs(gs - ref).max() <= 1e-5 * ref.max() + 1e-9
        gi = idx[s, h].cpu().numpy()
        assert (gi[keff:] == -1).all() and (np.diff(gi[:keff]) > 0).all()
        kth = np.sort(ref)[::-1][keff - 1]
        diff = set(gi[:keff].tolist()) ^ set(IDX[0, 0, :keff].tolist())
        bad = [p for p in diff if abs(ref[p] - kth) > BAND]
        assert not bad, (name, s, h, bad[:10])
        worst = max(worst, float(np.abs(go - O).max()))
        # later step over the GPU's own index set, both sides
        O2, L2 = oracle.sparse(uq2, uk, uv, gi[None, None], w.scale)
        g2 = o2[s:s + 1, :, h * G:(h + 1) * G].cpu().double().numpy()
        assert np.abs(g2 - O2).max() <= TOL, (name, s, h)
        assert np.abs(lse2[s:s + 1, :, h * G:(h + 1) * G].cpu().double().numpy() - L2).max() <= TOL
        worst = max(worst, float(np.abs(g2 - O2).max()))
    print(f"   {len(units)} units: worst O max-abs error {worst:.2e}", flush=True)


def _band_check(g_sel, ref_scores, ref_sel, keff, what):
    kth = np.sort(ref_scores)[::-1][keff - 1]
    diff = set(g_sel.tolist()) ^ set(ref_sel.tolist())
    bad = [p for p in diff if abs(ref_scores[p] - kth) > BAND]
    assert not bad, (what, bad[:10])
    return len(diff)


# (config, sampled (seq, KV head) units, the sequence checked whole for adaptive budgets)
NEXT_CASES = [("head128k", [(0, 6)], 0), ("ragged", [(0, 1), (6, 4)], 0)]


@pytest.mark.parametrize("name,units,whole", NEXT_CASES, ids=[c[0] for c in NEXT_CASES])
def test_full_size_next_rows(name, units, whole):
    """The block rows fused into a later step, mean-query and page-granular
    selection on sampled units, and head-adaptive budgets over one whole
    sequence, at the workload's full size."""
    w = workloads.CONFIG_BY_NAME[name]
    print(f"[case] next rows {name} units={units} whole={whole}", flush=True)
    inp = workloads.make_inputs(w, steps=2)
    g = torch.Generator().manual_seed(17)
    S, Hkv, G, B, d = w.num_seqs, w.num_kv_heads, w.group, w.block, w.head_dim
    kb = torch.randn(S, Hkv, B, d, generator=g).to(torch.bfloat16)
    vb = torch.randn(S, Hkv, B, d, generator=g).to(torch.bfloat16)
    q1 = inp.q1.to(DEV)
    q2 = inp.q_steps[0].to(DEV)
    P, kp = 16, w.k // 16
    if w.paged:
        kc, vc = inp.k_pool.to(DEV), inp.v_pool.to(DEV)
        tab, lens = inp.page_table.to(DEV), inp.seq_lens.tolist()
        _, _, idx, _ = mage.select_exact_paged(q1, kc, vc, tab, lens, w.k, w.scale)
        ob, lb = mage.sparse_block_attn_paged(q2, kc, vc, tab, lens, idx, kb.to(DEV), vb.to(DEV), w.scale)
        mq_idx, mq_sc = mage.select_mean_query_paged(q1, kc, vc, tab, lens, w.k, w.scale, want_scores=True)
        _, _, pidx_pos, pidx, psc = mage.select_pages_paged(q1, kc, vc, tab, lens, P, kp, w.scale, want_scores=True)
        _, _, aidx, acnt = mage.select_adaptive_paged(q1, kc, vc, tab, lens, w.k, w.scale)
    else:
        kc, vc = inp.k.to(DEV), inp.v.to(DEV)
        _, _, idx, _ = mage.select_exact(q1, kc, vc, w.k, w.scale)
        ob, lb = mage.sparse_block_attn(q2, kc, vc, idx, kb.to(DEV), vb.to(DEV), w.scale)
        mq_idx, mq_sc = mage.select_mean_query(q1, kc, vc, w.k, w.scale, want_scores=True)
        _, _, pidx_pos, pidx, psc = mage.select_pages(q1, kc, vc, P, kp, w.scale, want_scores=True)
        _, _, aidx, acnt = mage.select_adaptive(q1, kc, vc, w.k, w.scale)
    torch.cuda.synchronize()
    for s, h in units:
        n = w.seq_lens[s]
        uq1, uq2, uk, uv = unit_inputs(inp, s, h)
        gi = idx[s, h].cpu().numpy()
        # block rows fused into the later step over the GPU's own index set
        O, L = oracle.block(uq2, uk, uv, gi[None, None], kb[s:s + 1, h:h + 1], vb[s:s + 1, h:h + 1], w.scale)
        assert np.abs(ob[s:s + 1, :, h * G:(h + 1) * G].cpu().double().numpy() - O).max() <= TOL, (name, s, h)
        assert np.abs(lb[s:s + 1, :, h * G:(h + 1) * G].cpu().double().numpy() - L).max() <= TOL, (name, s, h)
        # mean-query selection
        msc, midx = oracle.select_mean_query(uq1, uk, uv, w.scale, w.k)
        keff = min(w.k, n)
        gm = mq_idx[s, h].cpu().numpy()
        assert (gm[keff:] == -1).all() and (np.diff(gm[:keff]) > 0).all()
        np.testing.assert_allclose(mq_sc[s, h, :n].cpu().double().numpy(), msc[0][0], rtol=0,
                                   atol=1e-5 * msc[0][0].max() + 1e-9)
        nd_m = _band_check(gm[:keff], msc[0][0], midx[0, 0, :keff], keff, (name, s, h, "mean query"))
        # page selection
        ssc, spidx, spos = oracle.select_pages(uq1, uk, uv, w.scale, P, kp)
        npg = -(-n // P)
        kpe = min(kp, npg)
        gp = pidx[s, h].cpu().numpy()
        nd_p = _band_check(gp[:kpe], oracle.page_scores(ssc[0][0], P), spidx[0, 0, :kpe], kpe, (name, s, h, "pages"))
        assert np.array_equal(pidx_pos[s, h].cpu().numpy(), oracle.pages_to_positions(gp, P, n))
        print(f"   unit ({s},{h}): block O err ok, mean-query diff {nd_m}, page diff {nd_p} (in band)", flush=True)
    # head-adaptive budgets over every KV head of one sequence
    s = whole
    n = w.seq_lens[s]
    if w.paged:
        kk = oracle.depage(inp.k_pool, inp.page_table[s:s + 1], [n])[0][None]
        vv = oracle.depage(inp.v_pool, inp.page_table[s:s + 1], [n])[0][None]
    else:
        kk, vv = inp.k[s:s + 1], inp.v[s:s + 1]
    SC, IDX, CNT = oracle.select_adaptive(inp.q1[s:s + 1].contiguous(), kk, vv, w.scale, w.k)
    ga, gc = aidx[s].cpu().numpy(), acnt[s].cpu().numpy()
    K = min(w.k * Hkv, n * Hkv)
    assert gc.sum() == K
    flat = np.concatenate([SC[0][h] for h in range(Hkv)])
    kth = np.sort(flat)[::-1][K - 1]
    mine = {(h, int(p)) for h in range(Hkv) for p in ga[h, :gc[h]]}
    ref = {(h, int(p)) for h in range(Hkv) for p in IDX[0, h, :CNT[0, h]]}
    diff = mine ^ ref
    bad = [(h, p) for (h, p) in diff if abs(SC[0][h][p] - kth) > BAND]
    assert not bad, (name, "adaptive", bad[:10])
    print(f"   adaptive budgets, sequence {s}: counts {gc.tolist()}, {len(diff)} pairs differ (in band)", flush=True)
