"""The later step's in-launch merge: when a step splits each (sequence, KV
head)'s index list into several chunks, the last work-group of each
(unit, row block) to finish merges the chunks' partials, found through an
arrival counter in the workspace that every call leaves at zero.

These tests run back-to-back calls of different chunk counts, unit counts and
layouts on one workspace. Each result must equal the oracle and must be
bit-identical to the same call on a fresh workspace. The counter region at the
start of the workspace must read zero afterwards.
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
ARRIVAL_BYTES = 16384 * 4 * 4   # capacity of the counter region: 16384 units x 4 row blocks


def _case(seq_lens, Hq, Hkv, d, B, k, paged, seed):
    w = workloads.custom(seq_lens, Hq, Hkv, d, B, k, paged=paged, steps=2, seed=seed, name=f"h{seed}")
    inp = workloads.make_inputs(w, steps=2)
    rng = np.random.default_rng(seed)
    idx = np.full((w.num_seqs, Hkv, k), -1, dtype=np.int32)
    for s, n in enumerate(w.seq_lens):
        ke = min(k, n)
        for h in range(Hkv):
            idx[s, h, :ke] = np.sort(rng.choice(n, ke, replace=False))
    return w, inp, torch.from_numpy(idx)


CASES = [
    # (seq_lens, Hq, Hkv, d, B, k, paged): chunk counts from 2 to 16 and different unit counts
    ((8192,), 32, 8, 128, 32, 1024, False),
    ((3000, 5000), 16, 4, 128, 16, 300, True),
    ((53, 900, 4000), 8, 2, 64, 8, 2048, True),
    ((20000,), 16, 16, 64, 64, 256, False),
    ((6000,), 32, 8, 128, 32, 4096, False),
    ((5000,), 4, 1, 128, 8, 4096, False),    # one unit, 32 rows: 32 chunks, merged in four batches
]


def _run(w, inp, idx, ws):
    q = inp.q_steps[0].to(DEV)
    if w.paged:
        return mage.sparse_attn_paged(q, inp.k_pool.to(DEV), inp.v_pool.to(DEV), inp.page_table.to(DEV),
                                      inp.seq_lens.tolist(), idx.to(DEV), w.scale, workspace=ws)
    return mage.sparse_attn(q, inp.k.to(DEV), inp.v.to(DEV), idx.to(DEV), w.scale, workspace=ws)


def _oracle(w, inp, idx):
    q = inp.q_steps[0]
    if w.paged:
        return oracle.sparse_paged(q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens, idx.numpy(), w.scale)
    return oracle.sparse(q, inp.k, inp.v, idx.numpy(), w.scale)


def test_back_to_back_calls_share_one_workspace():
    cases = [(_case(*c, seed=70 + i)) for i, c in enumerate(CASES)]
    fresh = []
    for w, inp, idx in cases:
        o, lse = _run(w, inp, idx, mage.Workspace(DEV))
        torch.cuda.synchronize()
        Or, lr = _oracle(w, inp, idx)
        assert np.abs(o.cpu().double().numpy() - Or).max() <= TOL, w.name
        assert np.abs(lse.cpu().double().numpy() - lr).max() <= TOL, w.name
        fresh.append((o.cpu(), lse.cpu()))
    ws = mage.Workspace(DEV)
    order = [0, 1, 2, 3, 4, 5, 4, 0, 5, 2, 1, 3, 0, 0]
    for rep, i in enumerate(order):
        w, inp, idx = cases[i]
        o, lse = _run(w, inp, idx, ws)
        torch.cuda.synchronize()
        assert torch.equal(o.cpu(), fresh[i][0]) and torch.equal(lse.cpu(), fresh[i][1]), (rep, w.name)
    head = ws.buf[:ARRIVAL_BYTES].view(torch.int32)
    assert int(head.count_nonzero()) == 0


def test_handoff_under_graph_replay_with_new_indices():
    w, inp, idx = _case((9000,), 32, 8, 128, 32, 1024, False, seed=81)
    k, v = inp.k.to(DEV), inp.v.to(DEV)
    q = inp.q_steps[0].to(DEV)
    rng = np.random.default_rng(5)
    sets = [idx]
    for _ in range(3):
        nxt = np.stack([np.stack([np.sort(rng.choice(w.seq_lens[0], w.k, replace=False)) for _ in range(8)])])
        sets.append(torch.from_numpy(nxt.astype(np.int32)))
    ws = mage.Workspace(DEV)
    idx_static = sets[0].to(DEV).clone()
    o = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=DEV)
    mage.sparse_attn(q, k, v, idx_static, w.scale, o=o, lse=lse, workspace=ws)   # sizes the workspace
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mage.sparse_attn(q, k, v, idx_static, w.scale, o=o, lse=lse, workspace=ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep, ix in enumerate(sets + sets[:1]):
        idx_static.copy_(ix.to(DEV))
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = o.cpu().double().numpy(), lse.cpu().double().numpy()
        Or, lr = _oracle(w, inp, ix)
        assert np.abs(got_o - Or).max() <= TOL, rep
        assert np.abs(got_l - lr).max() <= TOL, rep
    assert int(ws.buf[:ARRIVAL_BYTES].view(torch.int32).count_nonzero()) == 0


def test_one_launch_merge_equals_the_merge_launch():
    # the same split (8 chunks of 128 entries per KV head) merged inside the
    # launch (uniform index lists) and by the merge kernel (per-head counts,
    # here all equal to the row length): the merge arithmetic is shared, so
    # O and lse must agree bit for bit
    w, inp, idx = _case((4000,), 8, 2, 128, 32, 1024, False, seed=91)
    q, k, v = inp.q_steps[0].to(DEV), inp.k.to(DEV), inp.v.to(DEV)
    ix = idx.to(DEV)
    mage.last_launches()
    o1, l1 = mage.sparse_attn(q, k, v, ix, w.scale)
    names1 = mage.last_launches()
    counts = torch.full((1, 2), 1024, dtype=torch.int32, device=DEV)
    o2, l2 = mage.sparse_attn_counts(q, k, v, ix, counts, 2048, w.scale)
    names2 = mage.last_launches()
    torch.cuda.synchronize()
    assert names1 == ["sparse_attn_kernel"], names1
    assert names2 == ["sparse_attn_kernel", "exact_merge_kernel[sparse]"], names2
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    Or, lr = _oracle(w, inp, idx)
    assert np.abs(o1.cpu().double().numpy() - Or).max() <= TOL
    assert np.abs(l1.cpu().double().numpy() - lr).max() <= TOL
