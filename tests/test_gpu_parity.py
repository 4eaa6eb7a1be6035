"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Bars: O and lse max-abs <= 2e-3 against the fp64 oracle (bf16 K/V, fp32
accumulation); index sets equal to the oracle's except at positions whose
oracle score lies within 1e-6 of the k-th score; the stand-alone top-k,
paged-vs-contiguous and run-to-run checks are bit-exact.
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


def maxabs(gpu, ref):
    g = gpu.detach().cpu().double().numpy() if torch.is_tensor(gpu) else np.asarray(gpu, np.float64)
    return float(np.abs(g - ref).max())


def check_idx(gpu_idx, ora_idx, ora_scores, k, lens):
    """Index-set parity with the tie band; returns the number of differing positions."""
    g_all = gpu_idx.cpu().numpy() if torch.is_tensor(gpu_idx) else gpu_idx
    ndiff = 0
    S, Hkv, _ = g_all.shape
    for s in range(S):
        for h in range(Hkv):
            n = int(lens[s])
            keff = min(k, n)
            g = g_all[s, h]
            assert (g[keff:] == -1).all()
            gs = g[:keff]
            assert (np.diff(gs) > 0).all(), "not strictly ascending"
            assert gs.min() >= 0 and gs.max() < n
            sc = ora_scores[s][h]
            kth = np.sort(sc)[::-1][keff - 1]
            diff = set(gs.tolist()) ^ set(ora_idx[s, h, :keff].tolist())
            bad = [p for p in diff if abs(sc[p] - kth) > BAND]
            assert not bad, f"(s={s}, h={h}) idx differs outside the tie band at {bad[:10]}"
            ndiff += len(diff)
    return ndiff


def dev_inputs(inp):
    d = {"q1": inp.q1.to(DEV), "q": [t.to(DEV) for t in inp.q_steps]}
    if inp.w.paged:
        d.update(k_pool=inp.k_pool.to(DEV), v_pool=inp.v_pool.to(DEV),
                 table=inp.page_table.to(DEV), lens=inp.seq_lens.tolist())
    else:
        d.update(k=inp.k.to(DEV), v=inp.v.to(DEV))
    return d


def gpu_select(inp, d, **kw):
    w = inp.w
    if w.paged:
        return mage.select_exact_paged(d["q1"], d["k_pool"], d["v_pool"], d["table"], d["lens"],
                                       w.k, w.scale, **kw)
    return mage.select_exact(d["q1"], d["k"], d["v"], w.k, w.scale, **kw)


def gpu_sparse(inp, d, q, idx, **kw):
    w = inp.w
    if w.paged:
        return mage.sparse_attn_paged(q, d["k_pool"], d["v_pool"], d["table"], d["lens"], idx,
                                      w.scale, **kw)
    return mage.sparse_attn(q, d["k"], d["v"], idx, w.scale, **kw)


def ora_select(inp):
    w = inp.w
    if w.paged:
        return oracle.select_exact_paged(inp.q1, inp.k_pool, inp.v_pool, inp.page_table,
                                         inp.seq_lens, w.scale, w.k)
    return oracle.select_exact(inp.q1, inp.k, inp.v, w.scale, w.k)


def ora_sparse(inp, q, idx):
    w = inp.w
    if w.paged:
        return oracle.sparse_paged(q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens, idx, w.scale)
    return oracle.sparse(q, inp.k, inp.v, idx, w.scale)


SMALL = [
    workloads.CONFIG_BY_NAME["tiny"],                                  # R = 16, d = 64
    workloads.custom((300,), 4, 1, 64, 3, 40, name="r12"),             # R = 12, ragged tile
    workloads.custom((1000,), 8, 2, 128, 16, 100, name="r64"),         # R = 64
    workloads.custom((777,), 32, 8, 128, 32, 129, name="r128"),        # R = 128, ragged k and N
    workloads.custom((5000,), 16, 4, 128, 24, 256, name="r96_split"),  # R = 96, many splits
    workloads.custom((1,), 4, 2, 64, 2, 8, name="n1"),                 # N = 1 < k
    workloads.custom((600, 600), 8, 2, 64, 4, 50, name="two_seqs"),
    workloads.custom((20000,), 32, 8, 128, 32, 1024, name="two_topk_chunks"),
    workloads.custom((53, 200, 1000), 8, 2, 64, 4, 64, paged=True, name="paged_ragged"),
    workloads.custom((17, 4096, 900), 32, 8, 128, 32, 512, paged=True, name="paged_r128"),
    # tile and chunk edges: exact pass tails of 63/64/65 keys, shifted last tiles,
    # chunk boundaries inside pages, pages smaller than and larger than a tile
    workloads.custom((64,), 8, 2, 64, 16, 32, name="n64"),
    workloads.custom((65,), 8, 2, 128, 16, 32, name="n65"),
    workloads.custom((63, 64, 65, 129, 577), 8, 2, 128, 16, 64, paged=True, name="paged_edges"),
    workloads.custom((100, 1000), 8, 2, 128, 16, 64, paged=True, page_size=4, name="paged_p4"),
    workloads.custom((100, 3000), 8, 2, 128, 16, 64, paged=True, page_size=256, name="paged_p256"),
    # head groups of more than 128 rows (B * G): run as sub-groups of query heads
    workloads.custom((3000,), 16, 2, 128, 32, 300, name="r256_two_groups"),
    workloads.custom((900, 2500), 24, 2, 64, 16, 128, paged=True, name="paged_r192_two_groups"),
    workloads.custom((700,), 6, 2, 64, 100, 64, name="r300_three_groups"),
    # long later-step chunks: four 512-entry chunks merged in the launch, the
    # last one ragged (464 entries); and one unsplit 640-entry chunk per (unit,
    # row block), 160 entries per wave, paged
    workloads.custom((2500, 2500), 32, 8, 128, 32, 2000, name="wide_split"),
    workloads.custom((700, 1000, 650, 2000), 32, 16, 64, 64, 600, paged=True, name="wide_paged_d64"),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_select_exact_and_sparse_match_oracle(w):
    inp = workloads.make_inputs(w)
    d = dev_inputs(inp)
    print(f"[case] {w.name} lens={w.seq_lens} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"d={w.head_dim} B={w.block} k={w.k}", flush=True)
    side = torch.cuda.Stream(device=DEV)
    ready = torch.cuda.Event()
    o, lse, idx, sc = gpu_select(inp, d, select_stream=side, idx_ready=ready)
    torch.cuda.current_stream().wait_event(ready)
    torch.cuda.synchronize()
    O, LSE, SC, IDX = ora_select(inp)
    assert maxabs(o, O) <= TOL
    assert maxabs(lse, LSE) <= TOL
    lens = w.seq_lens
    for s in range(w.num_seqs):
        for h in range(w.num_kv_heads):
            g = sc[s, h, :lens[s]].cpu().double().numpy()
            ref = SC[s][h]
            assert abs(g.sum() - 1.0) < 1e-5
            assert np.abs(g - ref).max() <= 1e-5 * ref.max() + 1e-9
    check_idx(idx, IDX, SC, w.k, lens)
    # later step with the GPU's own idx on both sides
    q2 = inp.q_steps[0]
    o2, lse2 = gpu_sparse(inp, d, d["q"][0], idx)
    torch.cuda.synchronize()
    O2, L2 = ora_sparse(inp, q2, idx.cpu().numpy())
    assert maxabs(o2, O2) <= TOL
    assert maxabs(lse2, L2) <= TOL


@pytest.mark.parametrize("w", SMALL[:6], ids=[w.name for w in SMALL[:6]])
def test_sparse_with_oracle_idx(w):
    inp = workloads.make_inputs(w)
    d = dev_inputs(inp)
    _, _, _, IDX = ora_select(inp)
    idx = torch.from_numpy(IDX).to(DEV)
    o2, lse2 = gpu_sparse(inp, d, d["q"][0], idx)
    torch.cuda.synchronize()
    O2, L2 = ora_sparse(inp, inp.q_steps[0], IDX)
    assert maxabs(o2, O2) <= TOL and maxabs(lse2, L2) <= TOL


def test_sparse_all_positions_equals_exact():
    w = workloads.custom((700,), 32, 8, 128, 32, 700, name="k_eq_n")
    inp = workloads.make_inputs(w)
    d = dev_inputs(inp)
    o, lse, idx, _ = gpu_select(inp, d)
    assert (idx.cpu().numpy() == np.arange(700)).all()
    o2, lse2 = gpu_sparse(inp, d, d["q1"], idx)
    torch.cuda.synchronize()
    assert maxabs(o2, o.cpu().double().numpy()) <= TOL
    assert maxabs(lse2, lse.cpu().double().numpy()) <= TOL


def test_sparse_idx_order_padding_and_out_of_range():
    w = workloads.custom((900,), 32, 8, 128, 32, 256, name="scramble")
    inp = workloads.make_inputs(w)
    d = dev_inputs(inp)
    _, _, _, IDX = ora_select(inp)
    rng = np.random.default_rng(3)
    scr = np.ascontiguousarray(IDX[:, :, rng.permutation(256)])
    pad = np.concatenate([scr[:, :, :100], np.full((1, 8, 7), -1, np.int32), scr[:, :, 100:],
                          np.full((1, 8, 3), 5000, np.int32)], axis=-1)
    O2, L2 = ora_sparse(inp, inp.q_steps[0], IDX)
    for arr in (scr, pad):
        o2, l2 = gpu_sparse(inp, d, d["q"][0], torch.from_numpy(np.ascontiguousarray(arr)).to(DEV))
        torch.cuda.synchronize()
        assert maxabs(o2, O2) <= TOL and maxabs(l2, L2) <= TOL
    empty = torch.full((1, 8, 64), -1, dtype=torch.int32, device=DEV)
    o3, l3 = gpu_sparse(inp, d, d["q"][0], empty)
    torch.cuda.synchronize()
    assert (o3 == 0).all() and torch.isneginf(l3).all()


@pytest.mark.parametrize("k", [300, 2000])   # 2000: 512-entry later-step chunks
def test_paged_equals_contiguous_bit_exact(k):
    w = workloads.custom((3000, 3000), 32, 8, 128, 32, k, name="pc")
    inp = workloads.make_inputs(w)
    kp, vp, table, lens = workloads.to_paged(inp.k, inp.v, 16, seed=11)
    q, kc, vc = inp.q1.to(DEV), inp.k.to(DEV), inp.v.to(DEV)
    kp, vp, table = kp.to(DEV), vp.to(DEV), table.to(DEV)
    a = mage.select_exact(q, kc, vc, w.k, w.scale)
    b = mage.select_exact_paged(q, kp, vp, table, lens, w.k, w.scale)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    q2 = inp.q_steps[0].to(DEV)
    s1 = mage.sparse_attn(q2, kc, vc, a[2], w.scale)
    s2 = mage.sparse_attn_paged(q2, kp, vp, table, lens, a[2], w.scale)
    for x, y in zip(s1, s2):
        assert torch.equal(x, y)


@pytest.mark.parametrize("d", [128, 64])
def test_paged_equals_contiguous_long_chunks(d):
    # about 800 keys per exact-pass chunk: the steady loop of both forms (full
    # tiles before the last, issued from per-lane offsets or from one batch of
    # page ids) runs for several unrolled rounds; each unit's last chunk ends
    # mid-tile
    w = workloads.custom((50700, 50700), 8, 2, d, 32, 300, name=f"pcl{d}")
    print(f"[case] paged vs contiguous, long chunks, d={d}", flush=True)
    inp = workloads.make_inputs(w, steps=2)
    kp, vp, table, lens = workloads.to_paged(inp.k, inp.v, 16, seed=12)
    q, kc, vc = inp.q1.to(DEV), inp.k.to(DEV), inp.v.to(DEV)
    kp, vp, table = kp.to(DEV), vp.to(DEV), table.to(DEV)
    a = mage.select_exact(q, kc, vc, w.k, w.scale)
    b = mage.select_exact_paged(q, kp, vp, table, lens, w.k, w.scale)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    ea = mage.exact_attn(q, kc, vc, w.scale)
    eb = mage.exact_attn_paged(q, kp, vp, table, lens, w.scale)
    for x, y in zip(ea, eb):
        assert torch.equal(x, y)


def test_runs_are_bit_identical():
    w = workloads.custom((5000,), 32, 8, 128, 32, 512, name="det")
    inp = workloads.make_inputs(w)
    d = dev_inputs(inp)
    a = gpu_select(inp, d)
    b = gpu_select(inp, d)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    s1 = gpu_sparse(inp, d, d["q"][0], a[2])
    s2 = gpu_sparse(inp, d, d["q"][0], a[2])
    for x, y in zip(s1, s2):
        assert torch.equal(x, y)


def test_equal_keys_pick_lowest_positions_and_constant_v():
    g = torch.Generator().manual_seed(1)
    q = (torch.randn(1, 32, 32, 128, generator=g) / 11.3).to(torch.bfloat16)
    k = torch.randn(1, 8, 1, 128, generator=g).expand(1, 8, 2000, 128).contiguous().to(torch.bfloat16)
    v = torch.full((1, 8, 2000, 128), 0.75).to(torch.bfloat16)
    o, lse, idx, sc = mage.select_exact(q.to(DEV), k.to(DEV), v.to(DEV), 100, 1.0)
    torch.cuda.synchronize()
    assert (idx.cpu().numpy() == np.arange(100)).all()
    assert torch.allclose(o.cpu(), torch.full_like(o.cpu(), 0.75), atol=1e-6, rtol=0)
    assert torch.allclose(sc.cpu(), torch.full_like(sc.cpu(), 1 / 2000), rtol=1e-5, atol=0)


@pytest.mark.parametrize("ties", ["none", "many", "all", "zeros"])
@pytest.mark.parametrize("n,k", [(1, 1), (5, 3), (100, 100), (1000, 17), (16384, 1024),
                                 (16385, 1024), (40000, 2048), (50000, 20000), (9, 30), (200000, 6000),
                                 (1 << 20, 8192),
                                 (24576, 100), (24577, 100)])   # register capacity of the final pass's overflow tier
def test_topk_bit_exact(ties, n, k):
    sc = workloads.random_scores(3, n, seed=n * 7 + k, ties=ties)
    idx = mage.topk(sc.to(DEV), k)
    torch.cuda.synchronize()
    ref = oracle.topk(sc.numpy().astype(np.float64), k)
    assert np.array_equal(idx.cpu().numpy(), ref)


def test_topk_ragged_rows():
    sc = workloads.random_scores(4, 40000, seed=5, ties="many")
    lens = [40000, 1, 17000, 999]
    idx = mage.topk(sc.to(DEV), 1024, lens=lens)
    torch.cuda.synchronize()
    for r, n in enumerate(lens):
        ref = oracle.topk(sc[r, :n].numpy().astype(np.float64), 1024)[0]
        assert np.array_equal(idx[r].cpu().numpy(), ref)


def test_kernel_timers_time_each_launch():
    """Armed events mark each kernel of the next call; results are unchanged by timing."""
    w = workloads.custom((20000,), 8, 2, 128, 16, 256)
    inp = workloads.make_inputs(w, steps=2)
    d = dev_inputs(inp)
    _, _, idx, _ = gpu_select(inp, d)
    ref, _ = gpu_sparse(inp, d, d["q"][0], idx)
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    pairs = [(mk(), mk()) for _ in range(mage.MAX_TIMED_LAUNCHES)]
    mage.arm_kernel_timers(pairs)
    o, _ = gpu_sparse(inp, d, d["q"][0], idx)
    names = mage.last_launches()
    torch.cuda.synchronize()
    assert names[0] == "sparse_attn_kernel"
    assert set(names[1:]) <= {"exact_merge_kernel[sparse]"}
    ms = [a.elapsed_time(b) for a, b in pairs[:len(names)]]
    assert all(0 < t < 100 for t in ms)
    assert torch.equal(o, ref)
    # the next call is untimed but still reports its launches
    gpu_sparse(inp, d, d["q"][0], idx)
    assert mage.last_launches() == names
    mage.arm_kernel_timers(pairs)
    gpu_select(inp, d)
    names = mage.last_launches()
    torch.cuda.synchronize()
    assert names == ["exact_chunk_kernel", "exact_merge_kernel[exact]", "score_kernel", "topk_select_kernel"]
    span = pairs[0][0].elapsed_time(pairs[len(names) - 1][1])
    assert span >= max(a.elapsed_time(b) for a, b in pairs[:len(names)]) > 0


# ---- block attention: the block's queries over the prefix part and the block's own rows ----

def _block_inputs(S, B, Hq, Hkv, d, N, k, seed):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(S, B, Hq, d, generator=g) / d ** 0.5).to(torch.bfloat16)
    kk = torch.randn(S, Hkv, N, d, generator=g).to(torch.bfloat16)
    vv = torch.randn(S, Hkv, N, d, generator=g).to(torch.bfloat16)
    kb = torch.randn(S, Hkv, B, d, generator=g).to(torch.bfloat16)
    vb = torch.randn(S, Hkv, B, d, generator=g).to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    idx = np.stack([np.stack([np.sort(rng.choice(N, size=k, replace=False)).astype(np.int32)
                              for _ in range(Hkv)]) for _ in range(S)])
    idx[0, 0, -1] = -1                       # a skipped entry
    if Hkv > 1:
        idx[-1, -1, :] = -1                  # a head with no prefix row: lse_prefix = -inf
    return q, kk, vv, kb, vb, idx


@pytest.mark.parametrize("S,B,Hq,Hkv,d,N,k", [
    (1, 32, 32, 8, 128, 3000, 256),    # the 128K workload's block shape (prefix shortened)
    (2, 5, 8, 2, 64, 700, 100),        # ragged rows: R = 20, one 32-row block, 5 block keys
    (1, 64, 16, 16, 128, 2048, 300),   # MHA, B = 64: two 32-key tiles
    (1, 128, 8, 8, 64, 500, 64),       # B = 128: four 32-key tiles, four row blocks
    (1, 33, 2, 1, 128, 90, 90),        # B = 33: a second tile with one key
    (1, 32, 16, 2, 128, 700, 100),     # R = 256: two sub-groups of query heads
    (2, 100, 6, 2, 64, 700, 64),       # R = 300: three sub-groups of 100 rows
])
def test_block_attn_matches_oracle(S, B, Hq, Hkv, d, N, k):
    scale = 1.0
    q, kk, vv, kb, vb, idx = _block_inputs(S, B, Hq, Hkv, d, N, k, seed=S * 1000 + B * 7 + d)
    Op, lp = oracle.sparse(q, kk, vv, idx, scale)          # the prefix part, from the oracle
    O_ref, l_ref = oracle.block(q, kk, vv, idx, kb, vb, scale)
    o_pre = torch.from_numpy(Op.astype(np.float32)).to(DEV)
    lse_pre = torch.from_numpy(lp.astype(np.float32)).to(DEV)
    o, lse = mage.block_attn(q.to(DEV), kb.to(DEV), vb.to(DEV), o_pre, lse_pre, scale)
    torch.cuda.synchronize()
    assert np.abs(o.cpu().numpy() - O_ref).max() <= 2e-3
    assert np.abs(lse.cpu().numpy() - l_ref).max() <= 2e-3
    # in place: the prefix tensors receive the result
    o2, lse2 = mage.block_attn(q.to(DEV), kb.to(DEV), vb.to(DEV), o_pre, lse_pre, scale, o=o_pre, lse=lse_pre)
    torch.cuda.synchronize()
    assert torch.equal(o2.cpu(), o.cpu()) and torch.equal(lse2.cpu(), lse.cpu())


def test_block_attn_after_the_gpu_prefix_pass():
    # the end-to-end use: a sparse step's (o, lse) on the GPU merged with the
    # block rows (the index set is the oracle's, so every expected value is too)
    w = workloads.custom((2000,), 8, 2, 128, 16, 128, steps=2, seed=21)
    inp = workloads.make_inputs(w, steps=2)
    d = dev_inputs(inp)
    idx = ora_select(inp)[3]
    qt = d["q"][0]
    o_pre, lse_pre = gpu_sparse(inp, d, qt, torch.from_numpy(np.ascontiguousarray(idx)).to(DEV))
    g = torch.Generator().manual_seed(5)
    kb = torch.randn(1, 2, 16, 128, generator=g).to(torch.bfloat16)
    vb = torch.randn(1, 2, 16, 128, generator=g).to(torch.bfloat16)
    o, lse = mage.block_attn(qt, kb.to(DEV), vb.to(DEV), o_pre, lse_pre, w.scale)
    torch.cuda.synchronize()
    O_ref, l_ref = oracle.block(inp.q_steps[0], inp.k, inp.v, idx, kb, vb, w.scale)
    assert np.abs(o.cpu().numpy() - O_ref).max() <= 2e-3
    assert np.abs(lse.cpu().numpy() - l_ref).max() <= 2e-3


# ---- the fused later step: index rows and the block's own rows in one pass ----

@pytest.mark.parametrize("S,B,Hq,Hkv,d,N,k", [
    (1, 32, 32, 8, 128, 3000, 256),    # the 128K workload's block shape (prefix shortened)
    (1, 32, 32, 8, 128, 6000, 1024),   # several index chunks, then the block chunk
    (2, 5, 8, 2, 64, 700, 100),        # ragged rows; one sequence's head has no prefix row
    (1, 64, 16, 16, 128, 2048, 300),   # MHA, B = 64: 16 block rows per wave
    (1, 128, 8, 8, 64, 500, 64),       # B = 128: 32 block rows per wave, four row blocks
    (1, 33, 2, 1, 128, 90, 90),        # B = 33: waves with 9, 9, 9 and 6 block rows
    (1, 2, 4, 1, 128, 300, 40),        # B = 2: two waves without block rows
    (2, 32, 32, 8, 128, 2500, 2000),   # 4 index chunks of 512, block rows in the last
    (4, 64, 32, 16, 64, 1000, 600),    # one 640-entry chunk (256 row-block pairs), 16 block rows per wave
    (1, 32, 16, 2, 128, 2000, 300),    # R = 256: two sub-groups, each with the block rows
    (2, 100, 6, 2, 64, 700, 64),       # R = 300: three sub-groups of 100 rows
])
def test_sparse_block_attn_matches_oracle(S, B, Hq, Hkv, d, N, k):
    scale = 1.0
    q, kk, vv, kb, vb, idx = _block_inputs(S, B, Hq, Hkv, d, N, k, seed=S * 1000 + B * 7 + d + k)
    O_ref, l_ref = oracle.block(q, kk, vv, idx, kb, vb, scale)
    o, lse = mage.sparse_block_attn(q.to(DEV), kk.to(DEV), vv.to(DEV), torch.from_numpy(idx).to(DEV),
                                    kb.to(DEV), vb.to(DEV), scale)
    torch.cuda.synchronize()
    assert np.abs(o.cpu().numpy() - O_ref).max() <= 2e-3
    assert np.abs(lse.cpu().numpy() - l_ref).max() <= 2e-3


@pytest.mark.parametrize("k,Hq,B", [
    (64, 8, 4), (700, 8, 4),   # 700: six index chunks merged in the launch, some only padding
    (100, 32, 16),             # R = 16 * 16 = 256 rows per KV head: two sub-groups, each with the block rows
])
def test_sparse_block_attn_paged_matches_oracle(k, Hq, B):
    # ragged paged prefix, shuffled 16-token pages; the oracle's own index set
    w = workloads.custom((53, 200, 1000), Hq, 2, 64, B, k, paged=True, steps=2, name="paged_ragged", seed=31)
    inp = workloads.make_inputs(w, steps=2)
    d = dev_inputs(inp)
    idx = np.ascontiguousarray(ora_select(inp)[3])
    g = torch.Generator().manual_seed(9)
    S = len(w.seq_lens)
    kb = torch.randn(S, 2, B, 64, generator=g).to(torch.bfloat16)
    vb = torch.randn(S, 2, B, 64, generator=g).to(torch.bfloat16)
    qt = d["q"][0]
    o, lse = mage.sparse_block_attn_paged(qt, d["k_pool"], d["v_pool"], d["table"], d["lens"],
                                          torch.from_numpy(idx).to(DEV), kb.to(DEV), vb.to(DEV), w.scale)
    torch.cuda.synchronize()
    O_ref, l_ref = oracle.block_paged(inp.q_steps[0], inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens,
                                      idx, kb, vb, w.scale)
    assert np.abs(o.cpu().numpy() - O_ref).max() <= 2e-3
    assert np.abs(lse.cpu().numpy() - l_ref).max() <= 2e-3


def test_sparse_block_attn_equals_sparse_then_block():
    # the fused pass and the two-pass composition agree to rounding on the same inputs
    q, kk, vv, kb, vb, idx = _block_inputs(1, 32, 32, 8, 128, 4000, 512, seed=77)
    args = [t.to(DEV) for t in (q, kk, vv)] + [torch.from_numpy(idx).to(DEV)]
    o1, l1 = mage.sparse_block_attn(*args, kb.to(DEV), vb.to(DEV), 0.09)
    op, lp = mage.sparse_attn(*args, 0.09)
    o2, l2 = mage.block_attn(args[0], kb.to(DEV), vb.to(DEV), op, lp, 0.09)
    torch.cuda.synchronize()
    assert (o1 - o2).abs().max().item() <= 1e-4
    assert (l1 - l2).abs().max().item() <= 1e-4
