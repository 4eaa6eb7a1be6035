"""The workspace contract on the GPU: calls through one (default) workspace
from several streams are ordered by the binding, the arrival counters are
left at zero by every call, and mage_workspace_check reports a workspace
whose counters are not zero."""
import pytest
import torch

import block_sparse_kv_amd as mage
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(seed, n=6000, k=512):
    # k = 512 over 8 units of 4 row blocks: the later step splits its index list and
    # merges inside the launch through the arrival counters
    w = workloads.custom((n,), 32, 8, 128, 32, k, steps=3, seed=seed, name=f"ws{seed}")
    inp = workloads.make_inputs(w, steps=3)
    return w, inp.q1.to(DEV), [q.to(DEV) for q in inp.q_steps], inp.k.to(DEV), inp.v.to(DEV)


def test_default_workspace_orders_calls_on_two_streams():
    wa, qa, qas, ka, va = _case(61)
    wb, qb, qbs, kb, vb = _case(62, n=9000, k=1024)
    # sequential reference, fresh workspaces
    ref = []
    for w, q, qs, k, v in ((wa, qa, qas, ka, va), (wb, qb, qbs, kb, vb)):
        ws = mage.Workspace(DEV)
        _, _, idx, _ = mage.select_exact(q, k, v, w.k, w.scale, workspace=ws)
        ref.append([idx] + [mage.sparse_attn(qq, k, v, idx, w.scale, workspace=ws)[0] for qq in qs])
    torch.cuda.synchronize()
    # the same calls interleaved over two streams, all through the default workspace
    sa, sb = torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        _, _, ia, _ = mage.select_exact(qa, ka, va, wa.k, wa.scale, stream=sa)
        _, _, ib, _ = mage.select_exact(qb, kb, vb, wb.k, wb.scale, stream=sb)
        outs_a, outs_b = [], []
        for qq_a, qq_b in zip(qas, qbs):
            outs_a.append(mage.sparse_attn(qq_a, ka, va, ia, wa.scale, stream=sa)[0])
            outs_b.append(mage.sparse_attn(qq_b, kb, vb, ib, wb.scale, stream=sb)[0])
        torch.cuda.synchronize()
        assert torch.equal(ia, ref[0][0]) and torch.equal(ib, ref[1][0]), rep
        for x, y in zip(outs_a, ref[0][1:]):
            assert torch.equal(x, y), ("a", rep)
        for x, y in zip(outs_b, ref[1][1:]):
            assert torch.equal(x, y), ("b", rep)
    ws = mage._ws_obj(None, torch.device(DEV))
    assert ws.check() == 0


def test_workspace_check_reports_nonzero_counters():
    w, q, qs, k, v = _case(63)
    ws = mage.Workspace(DEV)
    _, _, idx, _ = mage.select_exact(q, k, v, w.k, w.scale, workspace=ws)
    o, _ = mage.sparse_attn(qs[0], k, v, idx, w.scale, workspace=ws)
    torch.cuda.synchronize()
    assert ws.check() == 0
    # plant three non-zero counters from the host side (a workspace written over by its owner)
    ws.buf.view(torch.int32)[[0, 5, 65535]] = 7
    assert ws.check() == 3
    ws.buf.view(torch.int32)[[0, 5, 65535]] = 0
    assert ws.check() == 0
    o2, _ = mage.sparse_attn(qs[0], k, v, idx, w.scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
