"""mage_sparse_attn_noalloc (the later step with the library's fixed scratch
instead of a workspace) against mage_sparse_attn on the same inputs: calls
of different shapes in a row (a smaller one after a larger one and the
reverse, one with its head group run as two sub-groups), each repeated, every result
bit-identical to the workspace call (same kernels and plan) and within the
2e-3 bar of the fp64 oracle. Both calls split their index lists, so the
arrival counters in the scratch are exercised and must be left at zero."""
import numpy as np
import pytest
import torch

import block_sparse_kv_amd as mage
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("first", [True, False])
def test_noalloc_matches_the_workspace_call(first):
    # the third: R = 16 * 16 = 256 rows per KV head, two sub-groups in turn on the scratch
    cases = [(20000, 32, 8, 128, 32, 1024, 71), (3000, 16, 4, 64, 16, 512, 72), (3000, 32, 2, 128, 16, 1024, 73)]
    if not first:
        cases = cases[::-1]
    for n, Hq, Hkv, d, B, k, seed in cases:
        print(f"[case] noalloc N={n} Hq={Hq} Hkv={Hkv} d={d} B={B} k={k}", flush=True)
        w = workloads.custom((n,), Hq, Hkv, d, B, k, steps=2, seed=seed)
        inp = workloads.make_inputs(w, steps=2)
        q1, q2 = inp.q1.to(DEV), inp.q_steps[0].to(DEV)
        kc, vc = inp.k.to(DEV), inp.v.to(DEV)
        _, _, idx, _ = mage.select_exact(q1, kc, vc, k, w.scale, workspace=mage.Workspace(DEV))
        ref_o, ref_l = mage.sparse_attn(q2, kc, vc, idx, w.scale, workspace=mage.Workspace(DEV))
        for rep in range(2):
            o = torch.full_like(ref_o, float("nan"))
            lse = torch.full_like(ref_l, float("nan"))
            mage.sparse_attn_noalloc(q2, kc, vc, idx, w.scale, o=o, lse=lse)
            torch.cuda.synchronize()
            assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), (n, k, rep)
        O2, L2 = oracle.sparse(inp.q_steps[0], inp.k, inp.v, idx.cpu().numpy(), w.scale)
        assert np.abs(o.cpu().double().numpy() - O2).max() <= 2e-3
        assert np.abs(lse.cpu().double().numpy() - L2).max() <= 2e-3
