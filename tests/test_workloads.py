"""The seeded input generator: determinism and the shapes of each workload."""
import hashlib

import numpy as np
import torch

import workloads


def _sha(t: torch.Tensor) -> str:
    return hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()


def test_same_seed_same_bytes():
    w = workloads.custom((300,), 8, 2, 64, 4, 16, steps=3, seed=5)
    a, b = workloads.make_inputs(w), workloads.make_inputs(w)
    for x, y in [(a.q1, b.q1), (a.k, b.k), (a.v, b.v)] + list(zip(a.q_steps, b.q_steps)):
        assert _sha(x) == _sha(y)
    c = workloads.make_inputs(workloads.custom((300,), 8, 2, 64, 4, 16, steps=3, seed=6))
    assert _sha(c.k) != _sha(a.k)


def test_tiny_workload_shape_and_plants():
    inp = workloads.make_inputs(0)
    w = inp.w
    assert inp.q1.shape == (1, 16, 1, 64) and inp.k.shape == (1, 1, 1024, 64)
    assert len(inp.q_steps) == 3 and inp.q1.dtype == torch.bfloat16
    assert len(inp.plants[(0, 0)]) == 16 and w.scale == 0.125


def test_paged_table_is_a_permutation():
    w = workloads.custom((40, 16, 1), 4, 2, 64, 2, 8, paged=True, seed=3)
    inp = workloads.make_inputs(w)
    tab = inp.page_table.numpy()
    ids = np.concatenate([tab[s, :(n + 15) // 16] for s, n in enumerate(w.seq_lens)])
    assert sorted(ids.tolist()) == list(range(inp.k_pool.shape[0]))
    assert (tab[2, 1:] == -1).all()


def test_paged_rows_match_their_draws():
    # logical row p of sequence s sits at slot p % 16 of page table[s][p // 16]
    w = workloads.custom((40,), 4, 2, 64, 2, 8, paged=True, seed=3)
    inp = workloads.make_inputs(w)
    wc = workloads.custom((40,), 4, 2, 64, 2, 8, paged=False, seed=3)
    ref = workloads.make_inputs(wc)
    for p in range(40):
        pg = int(inp.page_table[0, p // 16])
        assert torch.equal(inp.k_pool[pg, :, p % 16], ref.k[0, :, p])
        assert torch.equal(inp.v_pool[pg, :, p % 16], ref.v[0, :, p])


def test_oracle_reproduces_tiny_regression_fixture():
    """Regression fixture written by tests/golden/make_golden.py (oracle only)."""
    import json
    import os
    import oracle
    with open(os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.json")) as f:
        g = json.load(f)
    inp = workloads.make_inputs(0)
    w = inp.w
    O, lse, sc, idx = oracle.select_exact(inp.q1, inp.k, inp.v, w.scale, w.k)
    assert idx[0, 0].tolist() == g["idx"]
    np.testing.assert_allclose(lse[0, :, 0], g["lse_step1"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(O[0, :, 0].sum(-1), g["o_step1_row_sums"], rtol=0, atol=1e-12)
    Os, lses = oracle.sparse(inp.q_steps[0], inp.k, inp.v, idx, w.scale)
    np.testing.assert_allclose(lses[0, :, 0], g["lse_step2"], rtol=0, atol=1e-12)


def test_walk_queries_drift_from_q1():
    w = workloads.custom((64,), 8, 2, 128, 16, 8, steps=32, name="walk")
    q1 = workloads.make_inputs(w, with_steps=False).q1.float()
    walk = workloads.walk_queries(w)
    assert len(walk) == 31
    assert all(torch.equal(a, b) for a, b in zip(walk, workloads.walk_queries(w)))   # seeded
    # the drift from Q1 has standard deviation sigma half-way (step 17) and grows
    sd = [float((q.float() - q1).std()) for q in walk]
    assert abs(sd[15] - w.q_noise) < 0.1 * w.q_noise
    assert sd[-1] > sd[15] > sd[3]


def _torch_calls_on_worker_threads(fn):
    """Run fn() and return the torch functions entered on threads other than
    the calling one (Python frames of torch modules, or torch builtins)."""
    import threading
    main = threading.get_ident()
    seen = []

    def prof(frame, event, arg):
        if threading.get_ident() == main:
            return
        if event == "call":
            mod = frame.f_globals.get("__name__", "")
            if mod.startswith("torch"):
                seen.append(f"{mod}.{frame.f_code.co_name}")
        elif event == "c_call":
            owner = getattr(arg, "__module__", None) or getattr(getattr(arg, "__objclass__", None), "__module__", "")
            if str(owner).startswith("torch"):
                seen.append(f"{owner}.{getattr(arg, '__name__', arg)}")

    threading.setprofile(prof)
    try:
        fn()
    finally:
        threading.setprofile(None)
    return seen


def test_generator_worker_threads_never_enter_torch():
    # torch's CPU kernels start an OpenMP team per calling thread; on the GPU machine a
    # worker thread inside torch during the first CUDA initialisation crashed the
    # process, so the draws on worker threads are numpy only
    for w in (workloads.custom((700,), 8, 2, 64, 4, 16, seed=9),
              workloads.custom((300, 45), 8, 2, 64, 4, 16, paged=True, seed=10)):
        assert _torch_calls_on_worker_threads(lambda: workloads.make_inputs(w)) == []


def test_worker_thread_check_sees_a_torch_call(monkeypatch):
    # the detector itself: a generator whose workers call torch is caught
    real = workloads._bf16_bits

    def leaky(a):
        torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
        return real(a)
    monkeypatch.setattr(workloads, "_bf16_bits", leaky)
    w = workloads.custom((200,), 8, 2, 64, 4, 16, seed=11)
    assert _torch_calls_on_worker_threads(lambda: workloads.make_inputs(w))
