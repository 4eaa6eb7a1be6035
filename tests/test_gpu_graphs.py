"""The C ABI under HIP graph capture and on concurrent streams: the calls launch kernels and record and
wait on events only (no allocation, no memset node), so a captured step can
be replayed. Each graph is replayed several times with new inputs copied into
its static buffers, with eager work and synchronizations between replays, and
every replay must equal the eager call on the same inputs bit for bit.
"""
import pytest
import torch

import block_sparse_kv_amd as mage
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(steps):
    w = workloads.custom((3000,), 16, 4, 128, 16, 128, steps=steps, seed=41, name="graph")
    inp = workloads.make_inputs(w, steps=steps)
    return w, inp


def test_captured_sparse_step_replays_like_eager():
    w, inp = _inputs(4)
    k, v = inp.k.to(DEV), inp.v.to(DEV)
    qs = [t.to(DEV) for t in [inp.q1] + list(inp.q_steps)]
    ws = mage.Workspace(DEV)
    _, _, idx, _ = mage.select_exact(qs[0], k, v, w.k, w.scale, workspace=ws)
    q_static = qs[1].clone()
    o = torch.empty(q_static.shape, dtype=torch.float32, device=DEV)
    lse = torch.empty(q_static.shape[:-1], dtype=torch.float32, device=DEV)
    kb = torch.randn(1, 4, 16, 128, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16).to(DEV)
    vb = torch.randn(1, 4, 16, 128, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).to(DEV)
    ob = torch.empty_like(o)
    lb = torch.empty_like(lse)
    # eager calls first: the workspace reaches its size before capture
    mage.sparse_attn(q_static, k, v, idx, w.scale, o=o, lse=lse, workspace=ws)
    mage.sparse_block_attn(q_static, k, v, idx, kb, vb, w.scale, o=ob, lse=lb, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mage.sparse_attn(q_static, k, v, idx, w.scale, o=o, lse=lse, workspace=ws, stream=s)
            mage.sparse_block_attn(q_static, k, v, idx, kb, vb, w.scale, o=ob, lse=lb, workspace=ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep, q in enumerate(qs[1:] + qs[1:2]):
        q_static.copy_(q)
        g.replay()
        torch.cuda.synchronize()
        got = (o.clone(), lse.clone(), ob.clone(), lb.clone())
        _ = (torch.randn(1000, device=DEV) * 2).sum().item()       # eager work between replays
        e_o, e_l = mage.sparse_attn(q, k, v, idx, w.scale, workspace=ws)
        e_ob, e_lb = mage.sparse_block_attn(q, k, v, idx, kb, vb, w.scale, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(got[0], e_o) and torch.equal(got[1], e_l), rep
        assert torch.equal(got[2], e_ob) and torch.equal(got[3], e_lb), rep


def test_captured_step_one_with_a_select_stream_replays_like_eager():
    w, inp = _inputs(3)
    k, v = inp.k.to(DEV), inp.v.to(DEV)
    qs = [t.to(DEV) for t in [inp.q1] + list(inp.q_steps)]
    ws = mage.Workspace(DEV)
    q_static = qs[0].clone()
    S, B, Hq, d = q_static.shape
    o = torch.empty(S, B, Hq, d, dtype=torch.float32, device=DEV)
    lse = torch.empty(S, B, Hq, dtype=torch.float32, device=DEV)
    idx = torch.empty(S, 4, w.k, dtype=torch.int32, device=DEV)
    sc = torch.empty(S, 4, 3000, dtype=torch.float32, device=DEV)
    mage.select_exact(q_static, k, v, w.k, w.scale, o=o, lse=lse, idx=idx, scores=sc, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=DEV)
    side = torch.cuda.Stream(device=DEV)
    ready = torch.cuda.Event()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mage.select_exact(q_static, k, v, w.k, w.scale, o=o, lse=lse, idx=idx, scores=sc, workspace=ws,
                              stream=s, select_stream=side, idx_ready=ready)
            s.wait_event(ready)                                    # join the select stream
    torch.cuda.current_stream().wait_stream(s)
    ws.pending = None   # the select-stream event it holds was recorded inside the capture
    for rep, q in enumerate(qs + qs[:1]):
        q_static.copy_(q)
        g.replay()
        torch.cuda.synchronize()
        got = (o.clone(), lse.clone(), idx.clone(), sc.clone())
        _ = (torch.randn(1000, device=DEV) * 3).sum().item()
        e = mage.select_exact(q, k, v, w.k, w.scale, workspace=ws)
        torch.cuda.synchronize()
        for a, b in zip(got, e):
            assert torch.equal(a, b), rep


def test_concurrent_calls_on_distinct_workspaces_match_sequential():
    # two sequences' step 1 and later step on two streams at once, each with its
    # own workspace, against the same calls one after the other
    wa = workloads.custom((5000,), 32, 8, 128, 32, 256, steps=2, seed=51, name="ca")
    wb = workloads.custom((53, 200, 1000), 8, 2, 64, 4, 64, paged=True, steps=2, seed=52, name="cb")
    ia, ib = workloads.make_inputs(wa, steps=2), workloads.make_inputs(wb, steps=2)
    ka, va = ia.k.to(DEV), ia.v.to(DEV)
    kp, vp, tab, lens = ib.k_pool.to(DEV), ib.v_pool.to(DEV), ib.page_table.to(DEV), ib.seq_lens.tolist()
    qa1, qa2 = ia.q1.to(DEV), ia.q_steps[0].to(DEV)
    qb1, qb2 = ib.q1.to(DEV), ib.q_steps[0].to(DEV)

    def run_a(ws, stream):
        o, l, idx, _ = mage.select_exact(qa1, ka, va, wa.k, wa.scale, workspace=ws, stream=stream)
        o2, l2 = mage.sparse_attn(qa2, ka, va, idx, wa.scale, workspace=ws, stream=stream)
        return o, l, idx, o2, l2

    def run_b(ws, stream):
        o, l, idx, _ = mage.select_exact_paged(qb1, kp, vp, tab, lens, wb.k, wb.scale, workspace=ws, stream=stream)
        o2, l2 = mage.sparse_attn_paged(qb2, kp, vp, tab, lens, idx, wb.scale, workspace=ws, stream=stream)
        return o, l, idx, o2, l2

    ref_a = run_a(mage.Workspace(DEV), None)
    ref_b = run_b(mage.Workspace(DEV), None)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)
    wsa, wsb = mage.Workspace(DEV), mage.Workspace(DEV)
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        with torch.cuda.stream(sa):
            got_a = run_a(wsa, sa)
        with torch.cuda.stream(sb):
            got_b = run_b(wsb, sb)
        torch.cuda.synchronize()
        for x, y in zip(got_a, ref_a):
            assert torch.equal(x, y), ("a", rep)
        for x, y in zip(got_b, ref_b):
            assert torch.equal(x, y), ("b", rep)
