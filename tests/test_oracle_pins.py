"""Pins of the fp64 CPU oracle to things other than itself.

Each check is independent of the oracle's code: torch's own attention routine
(scaled_dot_product_attention) and logsumexp in float64, closed forms worked
out from the definition, brute-force rank counting, and invariants. The
definitions pinned are those of the MAGE page ("MAGE: All-[MASK] Block
Already Knows Where to Look in Block Diffusion LLM", atlas.scime.ai summary):
exact step-1 attention of the all-[MASK] block, the block-shared top-k subset
("Problem", "Approach"), and reuse of that subset at later steps ("Approach").
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

pytestmark = pytest.mark.filterwarnings("ignore")


def bf16(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def rand_case(S, B, Hq, Hkv, d, N, seed, kscale=1.0):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(S, B, Hq, d, generator=g) / math.sqrt(d)).to(torch.bfloat16)
    k = (kscale * torch.randn(S, Hkv, N, d, generator=g)).to(torch.bfloat16)
    v = torch.randn(S, Hkv, N, d, generator=g).to(torch.bfloat16)
    return q, k, v


def sdpa_ref(q, k, v, scale, mask=None):
    """torch's attention in float64; q [S][B][Hq][d], k/v [S][Hkv][N][d]."""
    qq = q.double().permute(0, 2, 1, 3)          # [S][Hq][B][d]
    o = F.scaled_dot_product_attention(qq, k.double(), v.double(), attn_mask=mask,
                                       scale=scale, enable_gqa=True)
    return o.permute(0, 2, 1, 3)                 # [S][B][Hq][d]


def lse_ref(q, k, scale):
    Hq, Hkv = q.shape[2], k.shape[1]
    kk = k.double().repeat_interleave(Hq // Hkv, dim=1)     # [S][Hq][N][d]
    x = torch.einsum("sbjd,sjnd->sbjn", q.double(), kk) * scale
    return torch.logsumexp(x, dim=-1)


def probs_ref(q, k, scale):
    """Attention probabilities via torch's attention routine with V = identity."""
    S, Hkv, N, d = k.shape
    eye = torch.eye(N, dtype=torch.float64).expand(S, Hkv, N, N)
    return sdpa_ref(q, k, eye, scale)            # [S][B][Hq][N]


SHAPES = [  # (S, B, Hq, Hkv, d, N)
    (1, 1, 1, 1, 64, 1), (1, 3, 1, 1, 64, 2), (1, 1, 4, 1, 64, 3), (2, 3, 4, 1, 128, 17),
    (1, 16, 1, 1, 64, 64), (1, 3, 8, 2, 128, 64), (1, 2, 4, 4, 64, 1024),
]


@pytest.mark.parametrize("S,B,Hq,Hkv,d,N", SHAPES)
def test_exact_matches_torch_attention(S, B, Hq, Hkv, d, N):
    q, k, v = rand_case(S, B, Hq, Hkv, d, N, seed=N * 31 + d)
    scale = 1.0 / math.sqrt(d) * 3.0
    O, lse, scores = oracle.exact(q, k, v, scale)
    np.testing.assert_allclose(O, sdpa_ref(q, k, v, scale).numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref(q, k, scale).numpy(), rtol=0, atol=1e-12)
    # score: mean over the B tokens and the G heads of the group of the probabilities
    P = probs_ref(q, k, scale)                   # [S][B][Hq][N]
    G = Hq // Hkv
    for s in range(S):
        for h in range(Hkv):
            ref = P[s, :, h * G:(h + 1) * G].reshape(-1, N).mean(0).numpy()
            np.testing.assert_allclose(scores[s][h], ref, rtol=0, atol=1e-14)


def test_two_keys_logistic_closed_form():
    # q = a e0, k0 = c0 e0, k1 = c1 e0: x_p = scale a c_p, P0 = 1/(1+exp(x1-x0))
    d, scale = 64, 0.125
    a, c0, c1 = 1.5, 2.0, -0.75
    q = np.zeros((1, 1, 1, d)); q[..., 0] = a
    k = np.zeros((1, 1, 2, d)); k[0, 0, 0, 0] = c0; k[0, 0, 1, 0] = c1
    v = np.zeros((1, 1, 2, d)); v[0, 0, 0, :] = 1.0; v[0, 0, 1, :] = -2.0
    O, lse, sc = oracle.exact(bf16(q), bf16(k), bf16(v), scale)
    x0, x1 = scale * a * c0, scale * a * c1
    p0 = 1.0 / (1.0 + math.exp(x1 - x0))
    assert abs(sc[0][0, 0] - p0) < 1e-15 and abs(sc[0][0, 1] - (1 - p0)) < 1e-15
    np.testing.assert_allclose(O[0, 0, 0], p0 * 1.0 + (1 - p0) * -2.0, atol=1e-15)
    assert abs(lse[0, 0, 0] - (x0 + math.log1p(math.exp(x1 - x0)))) < 1e-14


def test_zero_keys_give_mean_of_v():
    q, _, v = rand_case(1, 3, 4, 2, 64, 37, seed=3)
    k = torch.zeros(1, 2, 37, 64, dtype=torch.bfloat16)
    O, lse, sc = oracle.exact(q, k, v, 0.3)
    mean_v = v.double().mean(2)                                  # [S][Hkv][d]
    for j in range(4):
        np.testing.assert_allclose(O[0, :, j], mean_v[0, j // 2].expand(3, 64).numpy(), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(37), atol=1e-14)
    np.testing.assert_allclose(np.stack(sc[0]), 1 / 37, atol=1e-16)


def test_constant_v_and_single_key():
    q, k, _ = rand_case(1, 4, 2, 1, 128, 50, seed=4, kscale=3.0)
    v = torch.full((1, 1, 50, 128), -1.25, dtype=torch.bfloat16)
    O, _, _ = oracle.exact(q, k, v, 1.0)
    np.testing.assert_allclose(O, -1.25, atol=1e-14)
    q, k, v = rand_case(1, 4, 2, 1, 64, 1, seed=5)
    O, lse, sc = oracle.exact(q, k, v, 0.7)
    np.testing.assert_allclose(O[0, :, :], v.double()[0, 0, 0].expand(4, 2, 64).numpy(), atol=0)
    x = 0.7 * torch.einsum("bjd,d->bj", q.double()[0], k.double()[0, 0, 0])
    np.testing.assert_allclose(lse[0], x.numpy(), atol=1e-14)
    assert sc[0][0, 0] == 1.0


def test_gqa_group_mapping():
    # KV head h has constant V = h + 1, so query head j must read back j // G + 1.
    Hq, Hkv = 8, 2
    q, k, _ = rand_case(1, 3, Hq, Hkv, 64, 20, seed=6)
    v = torch.stack([torch.full((20, 64), float(h + 1)) for h in range(Hkv)])[None].to(torch.bfloat16)
    O, _, _ = oracle.exact(q, k, v, 0.5)
    for j in range(Hq):
        np.testing.assert_allclose(O[0, :, j], j // (Hq // Hkv) + 1, atol=1e-14)


def test_probability_rows_and_scores_sum_to_one():
    N, d = 64, 64
    q, k, _ = rand_case(1, 5, 4, 2, d, N, seed=8, kscale=2.0)
    eye = torch.eye(N).expand(1, 2, N, N).to(torch.bfloat16)   # V = I gives the P rows as O
    O, _, sc = oracle.exact(q, k, eye, 0.4)
    np.testing.assert_allclose(O.sum(-1), 1.0, atol=1e-13)
    assert (O >= 0).all()
    np.testing.assert_allclose(O, probs_ref(q, k, 0.4).numpy(), atol=1e-13)
    for h in range(2):
        assert abs(sc[0][h].sum() - 1.0) < 1e-12
        assert (sc[0][h] >= 0).all() and (sc[0][h] <= 1).all()


def test_dominant_key_selects_its_value_row():
    q, k, v = rand_case(1, 4, 1, 1, 128, 300, seed=9)
    m = q.double()[0, :, 0].mean(0)
    kk = k.double()
    kk[0, 0, 123] = 400.0 * m / m.norm()
    k = kk.to(torch.bfloat16)
    O, _, sc = oracle.exact(q, k, v, 1.0)
    x = torch.einsum("bd,nd->bn", q.double()[0, :, 0], k.double()[0, 0])
    gap = (x[:, 123:124] - torch.cat([x[:, :123], x[:, 124:]], 1)).min().item()
    assert gap > 20
    # O - v* = sum_p P_p (v_p - v*), and every P_p (p != 123) is below exp(-gap)
    tol = 299 * math.exp(-gap) * 2 * v.double().abs().max().item()
    np.testing.assert_allclose(O[0, :, 0], v.double()[0, 0, 123].expand(4, 128).numpy(),
                               rtol=0, atol=tol + 1e-15)
    assert int(np.argmax(sc[0][0])) == 123


def rank_topk(score, k):
    """O(N^2) brute force: rank(p) = #{q: s_q > s_p or (s_q == s_p and q < p)}."""
    s = np.asarray(score, dtype=np.float64)
    n = len(s)
    ranks = np.array([np.sum((s > s[p]) | ((s == s[p]) & (np.arange(n) < p))) for p in range(n)])
    sel = np.sort(np.nonzero(ranks < min(k, n))[0])
    return np.concatenate([sel, -np.ones(k - len(sel), dtype=np.int64)])


@pytest.mark.parametrize("ties", ["none", "many", "all", "zeros"])
@pytest.mark.parametrize("n,k", [(1, 1), (5, 3), (64, 64), (300, 17), (1000, 100), (7, 20)])
def test_topk_matches_rank_counting(ties, n, k):
    sc = workloads.random_scores(3, n, seed=n + k, ties=ties).numpy()
    idx = oracle.topk(sc, k)
    for r in range(3):
        np.testing.assert_array_equal(idx[r], rank_topk(sc[r], k))


def test_topk_special_cases():
    n = 100
    assert oracle.topk(np.full(n, 0.01), 10)[0].tolist() == list(range(10))
    assert oracle.topk(np.arange(n) * 1e-3, 200)[0].tolist() == list(range(n)) + [-1] * 100
    # strictly decreasing scores: the first k positions
    assert oracle.topk(1.0 - np.arange(n) * 1e-3, 5)[0].tolist() == [0, 1, 2, 3, 4]


def test_single_row_topk_is_topk_of_logits():
    # B * G = 1: the score is the softmax row, a monotone map of the raw logits,
    # so its top-k equals the top-k of the logits (stable: lower position first).
    q, k, v = rand_case(1, 1, 1, 1, 64, 500, seed=10, kscale=2.0)
    _, _, sc, idx = oracle.select_exact(q, k, v, 0.125, 40)
    x = (k.double()[0, 0] @ q.double()[0, 0, 0]).numpy()
    order = np.argsort(-x, kind="stable")[:40]
    np.testing.assert_array_equal(idx[0, 0], np.sort(order))


def test_permuting_positions_permutes_selection():
    q, k, v = rand_case(1, 4, 2, 1, 64, 256, seed=11, kscale=2.0)
    _, _, sc, idx = oracle.select_exact(q, k, v, 0.25, 32)
    perm = np.random.default_rng(0).permutation(256)
    _, _, sc2, idx2 = oracle.select_exact(q, k[:, :, perm], v[:, :, perm], 0.25, 32)
    # continuous random scores: no ties, so the selected set maps through perm
    np.testing.assert_allclose(sc2[0][0], sc[0][0][perm], rtol=1e-12, atol=0)
    assert set(perm[idx2[0, 0]].tolist()) == set(idx[0, 0].tolist())


def test_sparse_with_all_positions_equals_exact():
    q, k, v = rand_case(2, 3, 4, 2, 64, 77, seed=12, kscale=2.0)
    O, lse, _ = oracle.exact(q, k, v, 0.3)
    idx = np.broadcast_to(np.arange(77, dtype=np.int32), (2, 2, 77))
    Os, lses = oracle.sparse(q, k, v, idx, 0.3)
    np.testing.assert_allclose(Os, O, atol=1e-12)
    np.testing.assert_allclose(lses, lse, atol=1e-12)


def test_sparse_equals_masked_attention_and_ignores_order():
    S, B, Hq, Hkv, d, N, kk = 1, 3, 4, 2, 128, 200, 23
    q, k, v = rand_case(S, B, Hq, Hkv, d, N, seed=13, kscale=2.0)
    rng = np.random.default_rng(1)
    idx = np.stack([np.sort(rng.choice(N, kk, replace=False)) for _ in range(Hkv)])[None].astype(np.int32)
    mask = torch.zeros(S, Hq, B, N, dtype=torch.bool)
    for j in range(Hq):
        mask[0, j, :, idx[0, j // 2]] = True
    ref = sdpa_ref(q, k, v, 0.2, mask=mask).numpy()
    Os, lses = oracle.sparse(q, k, v, idx, 0.2)
    np.testing.assert_allclose(Os, ref, atol=1e-12)
    scrambled = idx[:, :, rng.permutation(kk)]
    Os2, lses2 = oracle.sparse(q, k, v, scrambled, 0.2)
    np.testing.assert_allclose(Os2, Os, atol=1e-13)
    np.testing.assert_allclose(lses2, lses, atol=1e-13)
    # -1 padding and out-of-range entries are skipped
    padded = np.concatenate([idx, np.full((1, Hkv, 5), -1, np.int32),
                             np.full((1, Hkv, 2), N + 3, np.int32)], axis=-1)
    Os3, _ = oracle.sparse(q, k, v, padded, 0.2)
    np.testing.assert_allclose(Os3, Os, atol=1e-13)
    Oe, le = oracle.sparse(q, k, v, np.full((1, Hkv, 4), -1, np.int32), 0.2)
    assert (Oe == 0).all() and np.isneginf(le).all()


def test_merge_of_disjoint_subsets_gives_union():
    # O over I1 u I2 equals the lse-weighted merge of the parts.
    q, k, v = rand_case(1, 2, 4, 1, 64, 90, seed=14, kscale=2.0)
    i1 = np.arange(0, 90, 2, dtype=np.int32)[None, None]
    i2 = np.arange(1, 90, 2, dtype=np.int32)[None, None]
    O1, l1 = oracle.sparse(q, k, v, i1, 0.3)
    O2, l2 = oracle.sparse(q, k, v, i2, 0.3)
    O, lse, _ = oracle.exact(q, k, v, 0.3)
    L = np.logaddexp(l1, l2)
    np.testing.assert_allclose(L, lse, atol=1e-12)
    merged = (np.exp(l1 - L)[..., None] * O1 + np.exp(l2 - L)[..., None] * O2)
    np.testing.assert_allclose(merged, O, atol=1e-12)


def test_paged_equals_contiguous_bit_exact():
    q, k, v = rand_case(2, 4, 4, 2, 64, 53, seed=15, kscale=2.0)   # ragged tail page
    kp, vp, table, lens = workloads.to_paged(k, v, 16, seed=3)
    O, lse, sc, idx = oracle.select_exact(q, k, v, 0.3, 9)
    Op, lsep, scp, idxp = oracle.select_exact_paged(q, kp, vp, table, lens, 0.3, 9)
    assert np.array_equal(O, Op) and np.array_equal(lse, lsep) and np.array_equal(idx, idxp)
    assert all(np.array_equal(a, b) for a, b in zip(sc, scp))
    Os, ls = oracle.sparse(q, k, v, idx, 0.3)
    Osp, lsp = oracle.sparse_paged(q, kp, vp, table, lens, idx, 0.3)
    assert np.array_equal(Os, Osp) and np.array_equal(ls, lsp)


def test_tiny_workload_plants_are_selected():
    inp = workloads.make_inputs(0, with_steps=False)
    w = inp.w
    _, _, sc, idx = oracle.select_exact(inp.q1, inp.k, inp.v, w.scale, w.k)
    assert set(inp.plants[(0, 0)].tolist()) <= set(idx[0, 0].tolist())
    assert abs(sc[0][0].sum() - 1) < 1e-12


# ---- block attention (the block's queries over prefix rows + its own rows) ----

def block_case(S, B, Hq, Hkv, d, N, seed):
    q, k, v = rand_case(S, B, Hq, Hkv, d, N, seed)
    g = torch.Generator().manual_seed(seed + 1)
    kb = torch.randn(S, Hkv, B, d, generator=g).to(torch.bfloat16)
    vb = torch.randn(S, Hkv, B, d, generator=g).to(torch.bfloat16)
    return q, k, v, kb, vb


@pytest.mark.parametrize("S,B,Hq,Hkv,d,N", [(1, 3, 4, 1, 64, 17), (2, 5, 8, 2, 128, 40), (1, 32, 4, 1, 64, 7)])
def test_block_attention_is_attention_over_the_concatenation(S, B, Hq, Hkv, d, N):
    q, k, v, kb, vb = block_case(S, B, Hq, Hkv, d, N, seed=S * 100 + B)
    O, lse = oracle.block(q, k, v, None, kb, vb, 0.7)
    kc, vc = torch.cat([k, kb], dim=2), torch.cat([v, vb], dim=2)
    ref = sdpa_ref(q, kc, vc, 0.7).numpy()
    assert np.abs(O - ref).max() < 1e-12
    assert np.abs(lse - lse_ref(q, kc, 0.7).numpy()).max() < 1e-12


def test_block_attention_with_a_selected_subset_is_masked_attention():
    S, B, Hq, Hkv, d, N = 1, 4, 4, 2, 64, 50
    q, k, v, kb, vb = block_case(S, B, Hq, Hkv, d, N, seed=9)
    idx = np.array([[[3, 7, 7, 49, -1, 60]], [[0, 1, 2, 3, 4, 5]]], dtype=np.int32).reshape(S, Hkv, 6)
    O, lse = oracle.block(q, k, v, idx, kb, vb, 1.3)
    # mask over the concatenated rows: the selected prefix rows (a repeated
    # index counts once per entry, as in the gather) and every block row
    kc = torch.cat([k, kb], dim=2)
    vc = torch.cat([v, vb], dim=2)
    G = Hq // Hkv
    mask = torch.full((S, Hq, B, N + B), -math.inf, dtype=torch.float64)
    mask[..., N:] = 0.0
    for h in range(Hkv):
        for p in idx[0, h]:
            if 0 <= p < N:
                for g in range(G):
                    if mask[0, h * G + g, 0, p] == -math.inf:
                        mask[0, h * G + g, :, p] = 0.0
                    else:   # a repeated row: double its weight
                        mask[0, h * G + g, :, p] += math.log(2.0)
    ref = sdpa_ref(q, kc, vc, 1.3, mask=mask).numpy()
    assert np.abs(O - ref).max() < 1e-12


def test_block_attention_merges_through_log_sum_exp():
    # the prefix part and the block-only part, merged by their lse, give the union
    S, B, Hq, Hkv, d, N = 1, 6, 4, 2, 128, 33
    q, k, v, kb, vb = block_case(S, B, Hq, Hkv, d, N, seed=4)
    idx = np.stack([np.arange(0, 33, 2, dtype=np.int32), np.arange(1, 34, 2, dtype=np.int32)])[None]
    Op, lp = oracle.sparse(q, k, v, idx, 0.9)
    empty = torch.zeros(S, Hkv, 0, d, dtype=torch.bfloat16)
    Ob, lb = oracle.block(q, empty, empty, None, kb, vb, 0.9)
    M = np.maximum(lp, lb)
    wp, wb = np.exp(lp - M), np.exp(lb - M)
    merged = (wp[..., None] * Op + wb[..., None] * Ob) / (wp + wb)[..., None]
    O, lse = oracle.block(q, k, v, idx, kb, vb, 0.9)
    assert np.abs(merged - O).max() < 1e-12
    assert np.abs(M + np.log(wp + wb) - lse).max() < 1e-12


def test_block_attention_closed_form_equal_logits():
    # zero queries give equal logits: O is the mean of the block's V rows
    S, B, Hq, Hkv, d = 1, 5, 2, 1, 64
    q = torch.zeros(S, B, Hq, d, dtype=torch.bfloat16)
    empty = torch.zeros(S, Hkv, 0, d, dtype=torch.bfloat16)
    g = torch.Generator().manual_seed(3)
    kb = torch.randn(S, Hkv, B, d, generator=g).to(torch.bfloat16)
    vb = torch.randn(S, Hkv, B, d, generator=g).to(torch.bfloat16)
    O, lse = oracle.block(q, empty, empty, None, kb, vb, 1.0)
    mean_v = vb.double().mean(dim=2).numpy()          # [S][Hkv][d]
    for b in range(B):
        for j in range(Hq):
            assert np.abs(O[0, b, j] - mean_v[0, 0]).max() < 1e-12
    assert np.abs(lse - math.log(B)).max() < 1e-12


# ---- anchor re-selection diagnostics: mean-query selection and set overlap ----

def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).astype(np.int64)


def test_bf16_rounding_matches_torch_single_rounding_from_fp32():
    # torch rounds fp32 -> bf16 to nearest, ties to even, in one step: for values
    # that fp32 holds exactly the oracle's exact rounding must agree bit for bit
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(4000) * 2.0 ** rng.integers(-40, 40, 4000)).astype(np.float32)
    ties = (x.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)      # exact midpoints
    near = (x.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x7FFF)      # just below
    for arr in (x, ties.view(np.float32), near.view(np.float32)):
        want = _bits(torch.from_numpy(arr).to(torch.bfloat16))
        got = np.array([oracle._bf16_bits_of(float(v)) for v in arr])
        assert np.array_equal(got, want)


def test_mean_query_special_cases():
    g = torch.Generator().manual_seed(4)
    # one row per group: the mean query is the query itself, bit for bit
    q = torch.randn(2, 1, 3, 16, generator=g).to(torch.bfloat16)
    assert torch.equal(oracle.mean_query(q, 3), q)
    # identical rows: their mean is that row
    row = torch.randn(1, 1, 1, 16, generator=g).to(torch.bfloat16)
    assert torch.equal(oracle.mean_query(row.expand(1, 5, 4, 16).contiguous(), 2)[0, 0, 0], row[0, 0, 0])
    # worked values: mean(1, 2) = 1.5; mean(1, 1, 1, 2^-8 + 1) = 1 + 2^-10 -> ties... below half: 1
    q = bf16([[[[1.0], [2.0]]]]).reshape(1, 2, 1, 1)
    assert oracle.mean_query(q, 1).float().item() == 1.5
    q = bf16([1.0, 1.0, 1.0, 1.0 + 2 ** -7]).reshape(1, 4, 1, 1)
    assert oracle.mean_query(q, 1).float().item() == 1.0            # 1 + 2^-9: below half an ulp
    q = bf16([1.0, 1.0 + 2 ** -7]).reshape(1, 2, 1, 1)
    assert oracle.mean_query(q, 1).float().item() == 1.0            # 1 + 2^-8: a tie, to even


def test_mean_query_matches_float64_mean_where_fp32_holds_it():
    # power-of-two row counts: the float64 mean is exact; where fp32 also holds
    # it exactly, torch's fp32 -> bf16 rounding is the single rounding required
    g = torch.Generator().manual_seed(5)
    q = torch.randn(2, 8, 8, 32, generator=g).to(torch.bfloat16)    # B*G = 8 * 4 = 32 rows per group
    got = oracle.mean_query(q, 2)
    m = q.double().reshape(2, 8, 2, 4, 32).mean(dim=(1, 3))          # [S][Hkv][d]
    m32 = m.float()
    exact = (m32.double() == m)
    assert exact.float().mean() > 0.9
    ref = m32.to(torch.bfloat16)
    assert torch.equal(got[:, 0][exact], ref[exact])
    # permuting the rows of a group does not change it
    perm = torch.randperm(8, generator=g)
    assert torch.equal(oracle.mean_query(q[:, perm].contiguous(), 2), got)


def test_mean_query_selection_is_top_k_of_the_mean_query_logits():
    # with one query row, the softmax is monotone in the logit: the top-k by
    # probability is the top-k of scale * qbar . k (lower position on ties)
    q, k, v = rand_case(2, 8, 8, 2, 32, 300, seed=6)
    qm = oracle.mean_query(q, 2)
    scale = 0.3
    scores, idx = oracle.select_mean_query(q, k, v, scale, 40)
    logits = torch.einsum("shd,shnd->shn", qm[:, 0].double(), k.double()) * scale
    for s in range(2):
        for h in range(2):
            order = sorted(range(300), key=lambda p: (-logits[s, h, p].item(), p))[:40]
            assert idx[s, h].tolist() == sorted(order)
            # the scores are that row's softmax probabilities
            np.testing.assert_allclose(scores[s][h], torch.softmax(logits[s, h], 0).numpy(), rtol=1e-12,
                                       atol=1e-15)
    # one row per group: identical to the main selection
    q1 = q[:, :1, ::4].contiguous()                                   # B = 1, G = 1
    assert np.array_equal(oracle.select_mean_query(q1, k, v, scale, 40)[1],
                          oracle.select_exact(q1, k, v, scale, 40)[3])


def test_idx_overlap_counts():
    a = [[0, 3, 5, 9, -1, -1], [1, 2, 3, 4, 5, 6], [-1] * 6, [7, 8, -1, -1, -1, -1]]
    b = [[3, 4, 5, 6, 9, -1], [1, 2, 3, 4, 5, 6], [0, 1, -1, -1, -1, -1], [9, 10, 11, -1, -1, -1]]
    c, ca, cb = oracle.idx_overlap(a, b)
    assert c.tolist() == [3, 6, 0, 0]
    assert ca.tolist() == [4, 6, 0, 2] and cb.tolist() == [5, 6, 2, 3]
    c2, _, _ = oracle.idx_overlap(b, a)
    assert c2.tolist() == c.tolist()                                  # symmetric
    rng = np.random.default_rng(7)
    for _ in range(20):
        n, k = 200, int(rng.integers(1, 60))
        ra = np.sort(rng.choice(n, k, replace=False))
        rb = np.sort(rng.choice(n, k, replace=False))
        c, _, _ = oracle.idx_overlap([ra], [rb])
        assert c[0] == np.intersect1d(ra, rb).size


# ---- page-granular selection ----

def test_page_scores_and_expansion_by_hand():
    np.testing.assert_array_equal(oracle.page_scores([1, 2, 3, 4, 5], 2), [3, 7, 5])
    np.testing.assert_array_equal(oracle.page_scores([0.5, 0.25], 4), [0.75])
    np.testing.assert_array_equal(oracle.pages_to_positions([0, 2, -1], 3, 8), [0, 1, 2, 6, 7, -1, -1, -1, -1])


def test_page_selection_with_one_token_pages_is_the_token_selection():
    q, k, v = rand_case(1, 8, 8, 2, 32, 257, seed=21)
    _, _, _, idx = oracle.select_exact(q, k, v, 0.5, 40)
    _, pidx, pos = oracle.select_pages(q, k, v, 0.5, 1, 40)
    assert np.array_equal(pidx, idx) and np.array_equal(pos, idx)


def test_page_selection_by_brute_force():
    # every page's score from the oracle's own position scores, ranked by
    # counting (score desc, page asc), on a ragged last page
    q, k, v = rand_case(1, 4, 4, 1, 32, 203, seed=22)
    P, kp = 16, 5
    scores, pidx, pos = oracle.select_pages(q, k, v, 0.7, P, kp)
    sc = scores[0][0]
    npg = -(-203 // P)
    ps = [sum(sc[p] for p in range(g * P, min(203, (g + 1) * P))) for g in range(npg)]
    rank = [sum(1 for h in range(npg) if ps[h] > ps[g] or (ps[h] == ps[g] and h < g)) for g in range(npg)]
    want = sorted(g for g in range(npg) if rank[g] < kp)
    assert pidx[0, 0].tolist() == want
    assert abs(sum(ps) - 1.0) < 1e-12                      # page scores still sum to one
    exp = [p for g in want for p in range(g * P, (g + 1) * P)]
    assert [p if p < 203 else -1 for p in exp] == pos[0, 0].tolist()


def test_page_selection_keeps_the_page_of_a_dominant_key():
    # one key far above the rest: its page must be chosen first
    q, k, v = rand_case(1, 4, 4, 1, 32, 512, seed=23)
    m = q.double()[0, :, :, :].mean(dim=(0, 1))
    k2 = k.clone()
    k2[0, 0, 333] = (m / m.norm() * 40).to(torch.bfloat16)
    _, pidx, _ = oracle.select_pages(q, k2, v, 1.0, 16, 1)
    assert pidx[0, 0, 0] == 333 // 16


# ---- head-adaptive budgets ----

def test_adaptive_budgets_of_identical_heads_are_equal():
    # every KV head sees the same keys and queries: the global top-(k * Hkv) is
    # the top k of each head
    q, k, v = rand_case(1, 8, 2, 1, 32, 300, seed=31)
    q4 = q.repeat(1, 1, 4, 1).contiguous()                  # 8 query heads, G = 2 per KV head
    k4 = k.repeat(1, 4, 1, 1).contiguous()
    v4 = v.repeat(1, 4, 1, 1).contiguous()
    _, idx, counts = oracle.select_adaptive(q4, k4, v4, 0.4, 30)
    _, _, _, ref = oracle.select_exact(q4, k4, v4, 0.4, 30)
    assert counts.tolist() == [[30, 30, 30, 30]]
    assert np.array_equal(idx[..., :30], ref)
    assert (idx[..., 30:] == -1).all()


def test_adaptive_budgets_by_brute_force():
    # the kept (head, position) pairs are exactly those ranked below K by
    # (score desc, head asc, position asc), counted pair against pair
    q, k, v = rand_case(1, 4, 6, 3, 32, 60, seed=32)
    scores, idx, counts = oracle.select_adaptive(q, k, v, 0.9, 7)
    sc = scores[0]
    pairs = [(h, p) for h in range(3) for p in range(60)]
    def ahead(a, b):
        return sc[a] > sc[b] or (sc[a] == sc[b] and a < b)
    kept = {a for a in pairs if sum(ahead(b, a) for b in pairs) < 21}
    for h in range(3):
        assert set(idx[0, h, :counts[0, h]].tolist()) == {p for (hh, p) in kept if hh == h}
        assert (np.diff(idx[0, h, :counts[0, h]]) > 0).all() and (idx[0, h, counts[0, h]:] == -1).all()
    assert counts.sum() == 21


def test_adaptive_budgets_favour_the_diffuse_head():
    # head 0: a few keys carry its mass; head 1: every key equal (uniform). The
    # concentrated head needs only its heavy keys, the rest goes to head 1
    d, n = 32, 400
    g = torch.Generator().manual_seed(33)
    q = torch.zeros(1, 1, 2, d)
    q[0, 0, 0, 0] = 1.0
    k = torch.zeros(1, 2, n, d)
    k[0, 0, :, 0] = -30.0
    k[0, 0, [5, 50, 77], 0] = 10.0                          # head 0: three dominant keys
    v = torch.randn(1, 2, n, d, generator=g)
    _, idx, counts = oracle.select_adaptive(q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16),
                                            1.0, 20)
    assert idx[0, 0, :3].tolist() == [5, 50, 77]
    assert counts[0, 0] == 3 and counts[0, 1] == 37         # head 1's uniform 1/400 beats head 0's tail
    assert idx[0, 1, :37].tolist() == list(range(37))         # equal scores: lowest positions


def test_adaptive_budget_of_one_head_is_the_top_k():
    q, k, v = rand_case(2, 4, 4, 1, 32, 250, seed=34)
    _, idx, counts = oracle.select_adaptive(q, k, v, 0.6, 33)
    _, _, _, ref = oracle.select_exact(q, k, v, 0.6, 33)
    assert (counts == 33).all() and np.array_equal(idx, ref)
