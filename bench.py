"""Benchmark of the MAGE hot path on one MI355X.

One bench step = one block of block-diffusion decoding for one layer: step 1
(exact attention + block-averaged scores + top-k on a second stream), then
T-1 sparse steps over the reused index set with fresh queries. Default
workload: 1 sequence, 32 query / 8 KV heads, d=128, N=131072 prefix, B=32,
k=1024, T=32 (the MAGE page's headline shape under "Key results").

Protocol: inputs are resident in HBM before timing. Before every timed call a
1 GiB scratch buffer is overwritten and then read back on the same stream
(outside the timed window) so that K/V rows come from HBM, not from L2 or the
256 MB MALL, and the caches hold clean lines: without the read-back the timed
kernel would also pay for writing back the dirty lines the flush itself left
in the MALL (--flush dirty measures that case; --flush none keeps caches). Each
kernel of a timed call is launched with HIP events attached to the launch
itself (mage_arm_kernel_timers, hipExtLaunchKernel), so kernel durations are
GPU start-to-end times on the stream the kernel runs on, the same quantity
rocprofv3's kernel trace reports. A call's GPU time is the sum of its kernels'
durations: on an uninstrumented stream the kernels of a call dispatch back to
back, while the attached events themselves open gaps of several microseconds
between kernels. The instrumented span (first start to last end) and an
ordinary event pair around each call are reported beside it. `value` is
sparse steps per second (cold).

    python bench.py [--steps K] [--warmup W] [--config head128k] [--no-cpu]
    python bench.py --summarize-trace DIR           (rocprofv3 kernel-trace CSVs)
    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR   (rocprofv3 --pmc CSVs)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

FLUSH_DESC = {
    "clean": "a 1 GiB write then a 1 GiB read of a scratch buffer",
    "dirty": "a 1 GiB write of a scratch buffer (leaves dirty MALL lines)",
    "none": "no flush",
}
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
METRIC = "sparse-step denoising steps/sec and HBM GB/s (% peak) at 128K ctx, k=1024, B=32"
COPY_MIB = 256                 # size of the copy used to calibrate FETCH_SIZE / WRITE_SIZE


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---- algorithmic bytes and flops -------------------------------------------------
def sparse_bytes(w: workloads.Workload) -> int:
    """One sparse step: k_eff rows of K and V per (seq, KV head), Q (bf16) read, O (fp32) written."""
    d = w.head_dim
    rows = sum(w.k_eff(s) for s in range(w.num_seqs)) * w.num_kv_heads
    q = w.num_seqs * w.block * w.num_q_heads * d * 2
    o = w.num_seqs * w.block * w.num_q_heads * d * 4
    return rows * d * 2 * 2 + q + o


def sparse_chunk_bytes(w: workloads.Workload) -> int:
    """The sparse step's gather kernel: the K/V rows and Q (O is written by the merge)."""
    d = w.head_dim
    return sparse_bytes(w) - w.num_seqs * w.block * w.num_q_heads * d * 4


def select_bytes(w: workloads.Workload) -> int:
    """Step 1: Q + K + V read once, O + lse written, scores written and read back once, idx written."""
    d, S, Hkv = w.head_dim, w.num_seqs, w.num_kv_heads
    ntot = sum(w.seq_lens)
    q = S * w.block * w.num_q_heads * d * 2
    kv = ntot * Hkv * d * 2 * 2
    o = S * w.block * w.num_q_heads * (d + 1) * 4
    sc = ntot * Hkv * 4 * 2
    idx = S * Hkv * w.k * 4
    return q + kv + o + sc + idx


def exact_pass_bytes(w: workloads.Workload) -> int:
    """The exact pass kernel: Q, K and V read once (its partials stay in the workspace)."""
    d = w.head_dim
    return w.num_seqs * w.block * w.num_q_heads * d * 2 + sum(w.seq_lens) * w.num_kv_heads * d * 4


def score_bytes(w: workloads.Workload) -> int:
    """The score sweep: K read again, Q read, scores written."""
    d = w.head_dim
    ntot = sum(w.seq_lens) * w.num_kv_heads
    return w.num_seqs * w.block * w.num_q_heads * d * 2 + ntot * d * 2 + ntot * 4


def block_bytes(w: workloads.Workload) -> int:
    """Block attention: q and the block's K/V rows in bf16, the prefix O/lse read and the
    merged O/lse written in fp32."""
    S, B, Hq, Hkv, d = w.num_seqs, w.block, w.num_q_heads, w.num_kv_heads, w.head_dim
    return S * B * (Hq * d * 2 + 2 * Hkv * d * 2 + 2 * Hq * (d + 1) * 4)


def exact_flops(w: workloads.Workload) -> float:
    return 4.0 * w.block * w.num_q_heads * w.head_dim * sum(w.seq_lens)


def source_digest() -> str:
    """Digest of every HIP source of the library (the counter records name the sources they were taken on)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_kv_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hpp", ".hip")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


# ---- the GPU side --------------------------------------------------------------
class KernelTimer:
    """Events attached to the kernels of one library call, plus an outer event pair."""

    def __init__(self, torch, n):
        mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        self.pairs = [(mk(), mk()) for _ in range(n)]
        self.outer = (mk(), mk())
        for a, b in self.pairs:   # torch creates the HIP events on first record
            a.record()
            b.record()
        self.names = []

    def kernels_ms(self):
        if len(self.names) > len(self.pairs):
            raise RuntimeError(f"{len(self.names)} launches but {len(self.pairs)} timer pairs")
        return [a.elapsed_time(b) for a, b in self.pairs[:len(self.names)]]

    def busy_ms(self):
        """Sum of the call's kernel durations: its GPU time on a stream that dispatches
        the kernels back to back."""
        return sum(self.kernels_ms())

    def span_ms(self):
        """First kernel's start to last kernel's end; includes the gaps that the attached
        events themselves add between kernels."""
        n = len(self.names)
        return self.pairs[0][0].elapsed_time(self.pairs[n - 1][1])

    def outer_ms(self):
        return self.outer[0].elapsed_time(self.outer[1])


class Runner:
    def __init__(self, torch, mage, w, inp, dev):
        self.torch, self.mage = torch, mage
        self.w, self.dev = w, dev
        self.q1 = inp.q1.to(dev)
        self.qs = [t.to(dev) for t in inp.q_steps]
        if w.paged:
            self.kp, self.vp = inp.k_pool.to(dev), inp.v_pool.to(dev)
            self.table, self.lens = inp.page_table.to(dev), inp.seq_lens.tolist()
        else:
            self.k, self.v = inp.k.to(dev), inp.v.to(dev)
        self.ws = mage.Workspace(dev)
        self.side = torch.cuda.Stream(device=dev)
        self.ready = torch.cuda.Event()
        S, B, Hq, d = self.q1.shape
        self.o = torch.empty(S, B, Hq, d, dtype=torch.float32, device=dev)
        self.lse = torch.empty(S, B, Hq, dtype=torch.float32, device=dev)
        self.o2 = torch.empty_like(self.o)
        self.lse2 = torch.empty_like(self.lse)
        self.idx = torch.empty(S, w.num_kv_heads, w.k, dtype=torch.int32, device=dev)
        self.scores = torch.empty(S, w.num_kv_heads, w.max_seq_len, dtype=torch.float32, device=dev)
        g = torch.Generator().manual_seed(w.seed + 7)
        kb = torch.randn(S, w.num_kv_heads, B, d, generator=g).to(torch.bfloat16)
        self.kb, self.vb = kb.to(dev), torch.randn(kb.shape, generator=g).to(torch.bfloat16).to(dev)
        self.o3 = torch.empty_like(self.o)
        self.lse3 = torch.empty_like(self.lse)

    def _call(self, timer, fn):
        cur = self.torch.cuda.current_stream()
        if timer is not None:
            self.mage.arm_kernel_timers(timer.pairs)
            timer.outer[0].record(cur)
        fn()
        if timer is not None:
            timer.outer[1].record(cur)
            timer.names = self.mage.last_launches()

    def select(self, timer=None):
        w = self.w
        kw = dict(o=self.o, lse=self.lse, idx=self.idx, scores=self.scores, workspace=self.ws,
                  select_stream=self.side, idx_ready=self.ready)

        def fn():
            if w.paged:
                self.mage.select_exact_paged(self.q1, self.kp, self.vp, self.table, self.lens, w.k,
                                             w.scale, **kw)
            else:
                self.mage.select_exact(self.q1, self.k, self.v, w.k, w.scale, **kw)
            self.torch.cuda.current_stream().wait_event(self.ready)
        self._call(timer, fn)

    def exact_only(self, timer=None):
        w = self.w

        def fn():
            if w.paged:
                self.mage.exact_attn_paged(self.q1, self.kp, self.vp, self.table, self.lens, w.scale,
                                           o=self.o, lse=self.lse, workspace=self.ws)
            else:
                self.mage.exact_attn(self.q1, self.k, self.v, w.scale, o=self.o, lse=self.lse,
                                     workspace=self.ws)
        self._call(timer, fn)

    def sparse(self, t, timer=None, stream=None):
        w = self.w
        q = self.qs[t % len(self.qs)]

        def fn():
            if w.paged:
                self.mage.sparse_attn_paged(q, self.kp, self.vp, self.table, self.lens, self.idx,
                                            w.scale, o=self.o2, lse=self.lse2, workspace=self.ws,
                                            stream=stream)
            else:
                self.mage.sparse_attn(q, self.k, self.v, self.idx, w.scale, o=self.o2,
                                      lse=self.lse2, workspace=self.ws, stream=stream)
        self._call(timer, fn)

    def block(self, t, timer=None):
        """The block's own rows merged into the prefix result of the last sparse step."""
        q = self.qs[t % len(self.qs)]
        self._call(timer, lambda: self.mage.block_attn(q, self.kb, self.vb, self.o2, self.lse2, self.w.scale,
                                                       o=self.o3, lse=self.lse3))

    def sparse_block(self, t, timer=None):
        """A later step with the block's own rows fused in as one more split."""
        w = self.w
        q = self.qs[t % len(self.qs)]

        def fn():
            if w.paged:
                self.mage.sparse_block_attn_paged(q, self.kp, self.vp, self.table, self.lens, self.idx,
                                                  self.kb, self.vb, w.scale, o=self.o3, lse=self.lse3,
                                                  workspace=self.ws)
            else:
                self.mage.sparse_block_attn(q, self.k, self.v, self.idx, self.kb, self.vb, w.scale,
                                            o=self.o3, lse=self.lse3, workspace=self.ws)
        self._call(timer, fn)

    def pages(self, P, kp, timer=None):
        """Step 1 with page-granular selection into self.pidx / self.pidx_pages."""
        w = self.w
        if not hasattr(self, "pidx") or self.pidx.shape[-1] != P * kp:
            S, Hkv = w.num_seqs, w.num_kv_heads
            self.pidx = self.torch.empty(S, Hkv, P * kp, dtype=self.torch.int32, device=self.dev)
            self.pidx_pages = self.torch.empty(S, Hkv, kp, dtype=self.torch.int32, device=self.dev)

        def fn():
            kw = dict(o=self.o, lse=self.lse, idx=self.pidx, page_idx=self.pidx_pages, workspace=self.ws)
            if w.paged:
                self.mage.select_pages_paged(self.q1, self.kp, self.vp, self.table, self.lens, P, kp, w.scale, **kw)
            else:
                self.mage.select_pages(self.q1, self.k, self.v, P, kp, w.scale, **kw)
        self._call(timer, fn)

    def adaptive(self, timer=None):
        """Step 1 with head-adaptive budgets into self.aidx / self.acounts."""
        w = self.w
        if not hasattr(self, "aidx"):
            S, Hkv = w.num_seqs, w.num_kv_heads
            self.aidx = self.torch.empty(S, Hkv, w.k * Hkv, dtype=self.torch.int32, device=self.dev)
            self.acounts = self.torch.empty(S, Hkv, dtype=self.torch.int32, device=self.dev)

        def fn():
            kw = dict(o=self.o, lse=self.lse, idx=self.aidx, counts=self.acounts, workspace=self.ws)
            if w.paged:
                self.mage.select_adaptive_paged(self.q1, self.kp, self.vp, self.table, self.lens, w.k, w.scale, **kw)
            else:
                self.mage.select_adaptive(self.q1, self.k, self.v, w.k, w.scale, **kw)
        self._call(timer, fn)

    def sparse_counts(self, t, timer=None):
        """A later step over the adaptive rows and counts."""
        w = self.w
        q = self.qs[t % len(self.qs)]
        k_seq = w.k * w.num_kv_heads

        def fn():
            if w.paged:
                self.mage.sparse_attn_counts_paged(q, self.kp, self.vp, self.table, self.lens, self.aidx, self.acounts,
                                                   k_seq, w.scale, o=self.o2, lse=self.lse2, workspace=self.ws)
            else:
                self.mage.sparse_attn_counts(q, self.k, self.v, self.aidx, self.acounts, k_seq, w.scale, o=self.o2,
                                             lse=self.lse2, workspace=self.ws)
        self._call(timer, fn)

    def sparse_idx(self, t, idx, timer=None):
        """A later step over the given index rows."""
        w = self.w
        q = self.qs[t % len(self.qs)]

        def fn():
            if w.paged:
                self.mage.sparse_attn_paged(q, self.kp, self.vp, self.table, self.lens, idx, w.scale, o=self.o2,
                                            lse=self.lse2, workspace=self.ws)
            else:
                self.mage.sparse_attn(q, self.k, self.v, idx, w.scale, o=self.o2, lse=self.lse2, workspace=self.ws)
        self._call(timer, fn)

    def topk_only(self, timer=None):
        w = self.w
        S, Hkv = w.num_seqs, w.num_kv_heads
        lens = None if not w.paged else [n for n in w.seq_lens for _ in range(Hkv)]
        self._call(timer, lambda: self.mage.topk(self.scores.view(S * Hkv, -1), w.k, lens=lens,
                                                 idx=self.idx.view(S * Hkv, -1), workspace=self.ws))


def anchor_diag(torch, mage, r, w, qs, sel_us, sparse_us):
    """Recall of the set in use against every step's own top-k set under a
    query drift (qs = Q_1..Q_T on the GPU), for anchor periods A (the set is
    chosen again at steps 1, 1 + A, ...; A = T is selection at step 1 only),
    and of the set chosen by the mean query at step 1. Every set and count
    comes from the GPU (the own sets are the main selection run on each step's
    queries)."""
    T = w.steps

    def select(q):
        if w.paged:
            return mage.select_exact_paged(q, r.kp, r.vp, r.table, r.lens, w.k, w.scale, want_scores=False,
                                           workspace=r.ws)[2]
        return mage.select_exact(q, r.k, r.v, w.k, w.scale, want_scores=False, workspace=r.ws)[2]

    own = [select(q).clone() for q in qs]
    if w.paged:
        mq = mage.select_mean_query_paged(qs[0], r.kp, r.vp, r.table, r.lens, w.k, w.scale, workspace=r.ws)[0]
    else:
        mq = mage.select_mean_query(qs[0], r.k, r.v, w.k, w.scale, workspace=r.ws)[0]

    def recall(a, b):
        c, _, cb = mage.idx_overlap(a, b)
        return (c.double() / cb.double().clamp(min=1)).cpu().numpy().ravel()

    out = {"first_sparse_step_recall": round(float(recall(own[0], own[1]).mean()), 4), "anchor_periods": {}}
    for A in sorted({T, 16, 8, 4, 2}, reverse=True):
        if A > T:
            continue
        rec = np.concatenate([recall(own[((t) // A) * A], own[t]) for t in range(1, T)])
        n_anchor = -(-T // A)
        block_us = n_anchor * sel_us + (T - n_anchor) * sparse_us
        out["anchor_periods"][str(A)] = {"mean_recall": round(float(rec.mean()), 4),
                                         "min_recall": round(float(rec.min()), 4),
                                         "anchors_per_block": n_anchor, "block_us": round(block_us, 1)}
    mq_rec = np.concatenate([recall(mq, own[t]) for t in range(T)])
    out["mean_query_step1_set"] = {"recall_vs_step1_own": round(float(recall(mq, own[0]).mean()), 4),
                                   "mean_recall_over_steps": round(float(mq_rec.mean()), 4)}
    return out


def page_diag(torch, mage, r, w, fl, P=16):
    """Page-granular selection at the same position budget (k / P pages of P
    positions): cold step-1 and later-step times, the recall of the page set
    against the position set, and the block-averaged score mass each keeps."""
    kp = max(1, w.k // P)
    T = w.steps
    r.select()                       # the position set and scores of Q1
    torch.cuda.synchronize()
    sel_t, sp_t = [], []
    for i in range(5):
        fl()
        tm = KernelTimer(torch, mage.MAX_TIMED_LAUNCHES)
        r.pages(P, kp, tm)
        sel_t.append(tm)
    for i in range(2 * (T - 1) if T > 1 else 2):
        fl()
        tm = KernelTimer(torch, mage.MAX_TIMED_LAUNCHES)
        r.sparse_idx(i, r.pidx, tm)
        sp_t.append(tm)
    torch.cuda.synchronize()
    c, _, cb = mage.idx_overlap(r.pidx, r.idx)
    recall = (c.double() / cb.double().clamp(min=1)).mean().item()
    sc = r.scores.double()

    def mass(idx):
        m = idx >= 0
        return (sc.gather(2, idx.clamp(min=0).long()) * m).sum(-1).mean().item()

    sel_k = by_kernel(sel_t)
    return {"page_tokens": P, "k_pages": kp,
            "select_gpu_us_median": round(statistics.median([t.busy_ms() * 1e3 for t in sel_t]), 1),
            "select_kernels_us_median": {n: round(statistics.median(v), 2) for n, v in sel_k.items()},
            "sparse_step_gpu_us_median": round(statistics.median([t.busy_ms() * 1e3 for t in sp_t]), 2),
            "recall_vs_position_set": round(recall, 4),
            "score_mass_pages": round(mass(r.pidx), 4), "score_mass_positions": round(mass(r.idx), 4)}


def budget_diag(torch, mage, r, w, fl):
    """Head-adaptive budgets at the same total (k * Hkv positions per sequence):
    cold step-1 and later-step times, the spread of the per-head counts, and
    the block-averaged score mass kept per head against the uniform k."""
    T = w.steps
    r.select()
    torch.cuda.synchronize()
    sel_t, sp_t = [], []
    for i in range(5):
        fl()
        tm = KernelTimer(torch, mage.MAX_TIMED_LAUNCHES)
        r.adaptive(tm)
        sel_t.append(tm)
    for i in range(2 * (T - 1) if T > 1 else 2):
        fl()
        tm = KernelTimer(torch, mage.MAX_TIMED_LAUNCHES)
        r.sparse_counts(i, tm)
        sp_t.append(tm)
    torch.cuda.synchronize()
    sc = r.scores.double()

    def mass(idx):
        m = idx >= 0
        return (sc.gather(2, idx.clamp(min=0).long()) * m).sum(-1)

    c = r.acounts.cpu().numpy().ravel()
    m_u, m_a = mass(r.idx), mass(r.aidx)
    return {"k_per_sequence": w.k * w.num_kv_heads,
            "select_gpu_us_median": round(statistics.median([t.busy_ms() * 1e3 for t in sel_t]), 1),
            "select_kernels_us_median": {n: round(statistics.median(v), 2) for n, v in by_kernel(sel_t).items()},
            "sparse_step_gpu_us_median": round(statistics.median([t.busy_ms() * 1e3 for t in sp_t]), 2),
            "counts_min_median_max": [int(c.min()), int(np.median(c)), int(c.max())],
            "score_mass_per_head_uniform": round(m_u.mean().item(), 4),
            "score_mass_per_head_adaptive": round(m_a.mean().item(), 4),
            "worst_head_mass_uniform": round(m_u.min().item(), 4),
            "worst_head_mass_adaptive": round(m_a.min().item(), 4)}


def batch_diag(torch, mage, w, dev, fl, batches=(1, 2, 4, 8, 16), reps=10):
    """The sparse step of this workload's per-sequence shape at several batch
    sizes, cold: inputs drawn on the GPU (K, V ~ N(0, 1), Q ~ N(0, 1/d), each
    (seq, KV head) a uniform random set of k positions), timed like the main
    sparse step. Shows how far the gather kernel gets once the step is large
    enough to leave its latency floor."""
    N, Hkv, Hq, d, B = w.seq_lens[0], w.num_kv_heads, w.num_q_heads, w.head_dim, w.block
    ws = mage.Workspace(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 99)
    out = []
    # the largest batch twice: random positions, then each unit's k positions as one
    # contiguous run (a control: the same work with streaming row addresses)
    plan = [(S, "random") for S in batches] + [(batches[-1], "contiguous run")]
    for S, pattern in plan:
        wb = workloads.Workload(f"{w.name}-x{S}", (N,) * S, Hq, Hkv, d, B, w.k, w.steps)
        k = torch.randn(S, Hkv, N, d, generator=g, device=dev).to(torch.bfloat16)
        v = torch.randn(S, Hkv, N, d, generator=g, device=dev).to(torch.bfloat16)
        q = (torch.randn(S, B, Hq, d, generator=g, device=dev) * d ** -0.5).to(torch.bfloat16)
        ke = w.k_eff(0)
        if pattern == "random":
            idx = torch.rand(S, Hkv, N, generator=g, device=dev).topk(ke, dim=-1).indices
            idx = idx.sort(dim=-1).values.to(torch.int32).contiguous()
        else:
            start = torch.randint(0, N - ke + 1, (S, Hkv, 1), generator=g, device=dev)
            idx = (start + torch.arange(ke, device=dev)).to(torch.int32).contiguous()
        o = torch.empty(S, B, Hq, d, dtype=torch.float32, device=dev)
        lse = torch.empty(S, B, Hq, dtype=torch.float32, device=dev)
        mage.sparse_attn(q, k, v, idx, 1.0, o=o, lse=lse, workspace=ws)   # sizes the workspace
        timers = []
        for _ in range(reps):
            fl()
            tm = KernelTimer(torch, mage.MAX_TIMED_LAUNCHES)
            cur = torch.cuda.current_stream()
            mage.arm_kernel_timers(tm.pairs)
            tm.outer[0].record(cur)
            mage.sparse_attn(q, k, v, idx, 1.0, o=o, lse=lse, workspace=ws)
            tm.outer[1].record(cur)
            tm.names = mage.last_launches()
            timers.append(tm)
        torch.cuda.synchronize()
        med = statistics.median([t.busy_ms() * 1e3 for t in timers])
        gather = statistics.median(by_kernel(timers)["sparse_attn_kernel"])
        nb = sparse_bytes(wb)
        cb = sparse_chunk_bytes(wb) if len(timers[0].names) > 1 else nb
        out.append({"seqs": S, "positions": pattern, "bytes": nb, "gpu_us_median": round(med, 2), "GBps": round(nb / (med * 1e-6) / 1e9, 1),
                    "frac_of_peak": round(nb / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "gather_kernel_us_median": round(gather, 2),
                    "gather_kernel_frac_of_peak": round(cb / (gather * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "kernels": timers[0].names})
        del k, v, q, idx, o, lse
        torch.cuda.empty_cache()
    return out


MAIN_STREAM = ("exact_chunk_kernel", "exact_merge_kernel[exact]")


def select_chain_us(tm):
    """Step 1's GPU time from its kernels' durations: the exact pass, then the
    longer of the split merge (main stream) and the selection kernels (score
    sweep and top-k, select stream), which run side by side."""
    d = {}
    for name, ms in zip(tm.names, tm.kernels_ms()):
        d[name] = d.get(name, 0.0) + ms * 1e3
    side = sum(v for n, v in d.items() if n not in MAIN_STREAM)
    return d.get("exact_chunk_kernel", 0.0) + max(d.get("exact_merge_kernel[exact]", 0.0), side)


def event_pair_us(torch, fn, fl, reps):
    """Median GPU time between an event recorded before fn() and one recorded after
    it on the current stream (uninstrumented kernels), a flush before each."""
    pairs = []
    for _ in range(reps):
        fl()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    return statistics.median([a.elapsed_time(b) * 1e3 for a, b in pairs])


def overlap_diag(torch, mage, r, w, fl, empty_us, reps=7):
    """The selection overlapped with other work (the MAGE page's summary and
    "Key results": selection runs on a second stream during the rest of step 1).
    Stand-in for the rest of the step: the next layer's exact pass over a second
    KV cache of the same shape, issued on the main stream while the score sweep
    and top-k of this layer run on the select stream. Uninstrumented event pairs
    (minus the empty pair), cold."""
    dev = r.dev
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 123)
    if w.paged:
        kp2 = torch.randn(r.kp.shape, generator=g, device=dev).to(torch.bfloat16)
        vp2 = torch.randn(r.vp.shape, generator=g, device=dev).to(torch.bfloat16)
    else:
        k2 = torch.randn(r.k.shape, generator=g, device=dev).to(torch.bfloat16)
        v2 = torch.randn(r.v.shape, generator=g, device=dev).to(torch.bfloat16)
    ws2 = mage.Workspace(dev)
    o2 = torch.empty_like(r.o)
    l2 = torch.empty_like(r.lse)

    def exact_next():
        if w.paged:
            mage.exact_attn_paged(r.q1, kp2, vp2, r.table, r.lens, w.scale, o=o2, lse=l2, workspace=ws2)
        else:
            mage.exact_attn(r.q1, k2, v2, w.scale, o=o2, lse=l2, workspace=ws2)

    def select(side):
        kw = dict(o=r.o, lse=r.lse, idx=r.idx, scores=r.scores, workspace=r.ws,
                  select_stream=side, idx_ready=r.ready if side is not None else None)
        if w.paged:
            mage.select_exact_paged(r.q1, r.kp, r.vp, r.table, r.lens, w.k, w.scale, **kw)
        else:
            mage.select_exact(r.q1, r.k, r.v, w.k, w.scale, **kw)

    def overlapped():
        select(r.side)
        exact_next()
        torch.cuda.current_stream().wait_event(r.ready)

    def serial():
        select(None)
        exact_next()

    def exact_both():
        r.exact_only()
        exact_next()

    for fn in (overlapped, serial, exact_both):   # sizes the workspaces
        fn()
    torch.cuda.synchronize()
    t_ov = event_pair_us(torch, overlapped, fl, reps) - empty_us
    t_se = event_pair_us(torch, serial, fl, reps) - empty_us
    t_ex = event_pair_us(torch, exact_both, fl, reps) - empty_us
    t_one = event_pair_us(torch, lambda: select(r.side) or torch.cuda.current_stream().wait_event(r.ready),
                          fl, reps) - empty_us
    t_ex1 = event_pair_us(torch, r.exact_only, fl, reps) - empty_us
    sel_cost = max(t_se - t_ex, 1e-9)
    return {"two_layers_overlapped_us": round(t_ov, 1), "two_layers_one_stream_us": round(t_se, 1),
            "two_exact_passes_us": round(t_ex, 1),
            "first_step_overhead_overlapped": round(t_ov / t_ex - 1, 4),
            "first_step_overhead_one_stream": round(t_se / t_ex - 1, 4),
            "selection_hidden_frac": round((t_se - t_ov) / sel_cost, 4),
            "one_layer_select_us": round(t_one, 1), "one_layer_exact_us": round(t_ex1, 1),
            "one_layer_first_step_overhead": round(t_one / t_ex1 - 1, 4),
            "note": "uninstrumented event pairs minus the empty pair, cold (flush before each); layer 1 = "
                    "exact+select, layer 2 = exact pass over a second cache of the same shape (the rest of "
                    "step 1); overlapped: layer 1's score sweep and top-k on the select stream while the main "
                    "stream runs layer 2; one stream: the same kernels in order; overhead = time / (two exact "
                    "passes) - 1; hidden = share of the selection's one-stream cost that the overlap removes"}


def graph_diag(torch, mage, r, w, reps=5):
    """The T-1 later steps of a block launched back to back, warm (no flush between
    steps): replayed from one captured HIP graph (no host work per step) and
    launched eagerly; per-step GPU time from one event pair around all of them."""
    T = w.steps
    n = T - 1
    s = torch.cuda.Stream(device=r.dev)
    for t in range(n):   # eager warm-up: the workspace has its size before capture
        r.sparse(t)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for t in range(n):
                r.sparse(t, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()

    def replay():
        g.replay()

    def eager():
        for t in range(n):
            r.sparse(t)
    out = {}
    for name, fn in (("graph", replay), ("eager", eager)):
        per = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            per.append(a.elapsed_time(b) * 1e3 / n)
        out[f"{name}_us_per_step_median"] = round(statistics.median(per), 2)
    out["steps_per_replay"] = n
    out["note"] = ("warm (rows stay in the caches across steps, no flush); graph = one captured graph of the "
                   "T-1 later-step launches replayed, eager = the same launches from Python")
    return out


def by_kernel(timers):
    """{kernel name: [durations in us]} over a list of finished timers."""
    out = {}
    for t in timers:
        for name, ms in zip(t.names, t.kernels_ms()):
            out.setdefault(name, []).append(ms * 1e3)
    return out


def pct(a, p):
    return float(np.percentile(a, p))


def ragged_side(torch, mage, dev, fl, sparse_calls=40, select_calls=6):
    """The ragged paged batch (8 sequences of 8K-128K, 16-token pages, shuffled page
    table) measured beside the headline workload with the same protocol: cold calls,
    kernel durations from the launches' own events."""
    w = workloads.CONFIG_BY_NAME["ragged"]
    t0 = time.perf_counter()
    inp = workloads.make_inputs(w, steps=4)
    r = Runner(torch, mage, w, inp, dev)
    del inp
    log(f"[bench] ragged inputs in {time.perf_counter() - t0:.1f} s")
    for t in range(3):
        r.select()
        r.sparse(t)
    torch.cuda.synchronize()
    sp, sel = [], []
    for i in range(sparse_calls):
        fl()
        tm = KernelTimer(torch, mage.MAX_TIMED_LAUNCHES)
        r.sparse(i, tm)
        sp.append(tm)
    for _ in range(select_calls):
        fl()
        tm = KernelTimer(torch, mage.MAX_TIMED_LAUNCHES)
        r.select(tm)
        sel.append(tm)
    torch.cuda.synchronize()
    sp_us = [t.busy_ms() * 1e3 for t in sp]
    k_us = by_kernel(sp)["sparse_attn_kernel"]
    sel_us = [select_chain_us(t) for t in sel]
    nb = sparse_bytes(w)
    kmean = statistics.mean(k_us)
    bytes_sel = select_bytes(w)
    ideal_sel = max(bytes_sel / (HBM_PEAK_GBS * 1e9), exact_flops(w) / (BF16_PEAK_TFLOPS * 1e12)) * 1e6
    traffic = traffic_record(w.name)
    out = {"workload": f"ragged: {w.num_seqs} seqs, N={list(w.seq_lens)}, {w.num_q_heads} q / {w.num_kv_heads} KV "
                       f"heads, d={w.head_dim}, B={w.block}, k={w.k}, 16-token pages, shuffled page table",
           "sparse_step_us_mean": round(statistics.mean(sp_us), 2),
           "sparse_step_us_median": round(statistics.median(sp_us), 2),
           "steps_per_s": round(1e6 / statistics.mean(sp_us), 1),
           "bytes_per_step": nb,
           "GBps": round(nb / (kmean * 1e-6) / 1e9, 1),
           "frac": round(nb / (kmean * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "traffic_bytes_per_launch": None if traffic is None else traffic["bytes_per_launch"],
           "traffic_ratio": None if traffic is None else round(traffic["bytes_per_launch"] / nb, 3),
           "exact_select_us_median": round(statistics.median(sel_us), 1),
           "exact_select_roofline_us": round(ideal_sel, 1),
           "exact_select_roofline_frac": round(ideal_sel / statistics.median(sel_us), 4),
           "exact_select_kernels_us_median": {n: round(statistics.median(v), 2) for n, v in by_kernel(sel).items()}}
    del r
    torch.cuda.empty_cache()
    return out


# ---- the oracle on the host cores ------------------------------------------------
def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(w, inp, budget_s=20.0):
    """The fp64 oracle as it stands, timed on the host cores over the same workload:
    step 1 (exact + scores + top-k) over every (seq, KV head) unit, whole, repeated
    while it fits about 45% of the budget; then whole-batch sparse steps with the
    oracle's own index sets for about 45%. Returns sparse steps/s of the whole batch."""
    import oracle
    S, Hkv, G = w.num_seqs, w.num_kv_heads, w.group
    units = [(s, h) for s in range(S) for h in range(Hkv)]

    def unit_kv(s, h):
        n = w.seq_lens[s]
        if w.paged:
            kk = oracle.depage(inp.k_pool, inp.page_table[s:s + 1], [n])[0][h:h + 1][None]
            vv = oracle.depage(inp.v_pool, inp.page_table[s:s + 1], [n])[0][h:h + 1][None]
            return np.ascontiguousarray(kk), np.ascontiguousarray(vv)
        return inp.k[s:s + 1, h:h + 1].contiguous(), inp.v[s:s + 1, h:h + 1].contiguous()

    # paged caches are de-paged before any clock starts
    kv = {u: unit_kv(*u) for u in units}
    sel_runs, idx_of = [], {}
    while not sel_runs or (sum(sel_runs) + sel_runs[0] < 0.45 * budget_s and len(sel_runs) < 3):
        t0 = time.perf_counter()
        for (s, h) in units:
            kc, vc = kv[(s, h)]
            q1 = inp.q1[s:s + 1, :, h * G:(h + 1) * G].contiguous()
            _, _, _, idx = oracle.select_exact(q1, kc, vc, w.scale, w.k)
            idx_of[(s, h)] = idx
        sel_runs.append(time.perf_counter() - t0)
    work = []
    for (s, h) in units:
        kc, vc = kv[(s, h)]
        work.append((inp.q_steps[0][s:s + 1, :, h * G:(h + 1) * G].contiguous(), kc, vc, idx_of[(s, h)]))
    step_t = []
    while len(step_t) < 3 or (sum(step_t) < 0.45 * budget_s and len(step_t) < 5000):
        t0 = time.perf_counter()
        for q2, kc, vc, idx in work:
            oracle.sparse(q2, kc, vc, idx, w.scale)
        step_t.append(time.perf_counter() - t0)
    med = statistics.median(step_t)
    sel_med = statistics.median(sel_runs)
    sample = (f"oracle (C++ fp64, OpenMP) on the host: step 1 over all {len(units)} (seq, KV head) units "
              f"{len(sel_runs)}x (median {sel_med:.2f} s), then {len(step_t)} whole-batch sparse steps "
              f"(median {med * 1e3:.1f} ms per step)")
    return {"value": 1.0 / med, "select_step_s": sel_med, "select_runs": len(sel_runs), "sample": sample,
            "cores": oracle.num_threads(), "cpu_seconds": sum(sel_runs) + sum(step_t)}


# ---- traffic from committed counter summaries ------------------------------------
def traffic_record(config: str):
    """The per-launch HBM bytes of the sparse gather kernel from the committed counter
    summary, or None when it is absent or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"sparse_traffic_{config}.md")
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic: "):
                rec = json.loads(line[len("traffic: "):])
    if rec is None or rec.get("source_digest") != source_digest():
        return None
    return rec


# ---- the benchmark ---------------------------------------------------------------
def run_bench(args):
    import torch
    import block_sparse_kv_amd as mage
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    w = workloads.CONFIG_BY_NAME[args.config]
    t0 = time.perf_counter()
    inp = workloads.make_inputs(w)
    log(f"[bench] inputs for {w.name} drawn in {time.perf_counter() - t0:.1f} s")
    r = Runner(torch, mage, w, inp, dev)
    scratch = torch.empty(256 * 1024 * 1024, dtype=torch.int32, device=dev)   # 1 GiB
    fill = [0]

    def flush():
        fill[0] += 1
        scratch.fill_(fill[0])
        if args.flush == "clean":
            scratch.view(torch.float32).sum()   # reads the 1 GiB back (no widening copy): clean lines

    if args.no_flush:
        args.flush = "none"
    fl = (lambda: None) if args.flush == "none" else flush
    T = w.steps
    for _ in range(args.warmup):
        r.select()
        for t in range(T - 1):
            r.sparse(t)
    torch.cuda.synchronize()
    log("[bench] warm-up done")

    sel_timers = [KernelTimer(torch, mage.MAX_TIMED_LAUNCHES) for _ in range(args.steps)]
    sp_timers = [KernelTimer(torch, mage.MAX_TIMED_LAUNCHES) for _ in range(args.steps * (T - 1))]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        fl()
        r.select(sel_timers[i])
        for t in range(T - 1):
            fl()
            r.sparse(t, sp_timers[i * (T - 1) + t])
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    log(f"[bench] timed {args.steps} blocks in {wall:.2f} s wall (flush '{args.flush}' before every call)")

    # secondary measurements
    ex_timers = []
    for _ in range(5):
        fl()
        tm = KernelTimer(torch, mage.MAX_TIMED_LAUNCHES)
        r.exact_only(tm)
        ex_timers.append(tm)
    warm_timers = []
    for t in range(2 * (T - 1)):
        tm = KernelTimer(torch, mage.MAX_TIMED_LAUNCHES)
        r.sparse(t, tm)
        warm_timers.append(tm)
    r.select()
    torch.cuda.synchronize()
    blk_timers, fused_timers = [], []
    for t in range(0 if args.no_diag else 5):
        r.sparse(t)
        fl()
        tm = KernelTimer(torch, mage.MAX_TIMED_LAUNCHES)
        r.block(t, tm)
        blk_timers.append(tm)
    for t in range(0 if args.no_diag else 5):
        fl()
        tm = KernelTimer(torch, mage.MAX_TIMED_LAUNCHES)
        r.sparse_block(t, tm)
        fused_timers.append(tm)
    tk_timers = []
    for _ in range(5):
        fl()
        tm = KernelTimer(torch, mage.MAX_TIMED_LAUNCHES)
        r.topk_only(tm)
        tk_timers.append(tm)
    empty = []
    for _ in range(20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        b.record()
        empty.append((a, b))
    torch.cuda.synchronize()
    empty_pre = statistics.median([a.elapsed_time(b) * 1e3 for a, b in empty])
    sel_outer = event_pair_us(torch, r.select, fl, 7) - empty_pre
    ex_outer = event_pair_us(torch, r.exact_only, fl, 7) - empty_pre
    overlap = overlap_diag(torch, mage, r, w, fl, empty_pre)
    log("[bench] selection overlap measured")
    graphs = graph_diag(torch, mage, r, w)
    log("[bench] graph replay measured")
    # plain copy of known size: the calibration kernel for FETCH_SIZE / WRITE_SIZE counter runs
    # (timed: the measured copy bandwidth, a second roofline beside the 8 TB/s spec)
    src = torch.ones(COPY_MIB * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    copy_ms = []
    for _ in range(2):
        fl()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.neg(src, out=dst)
        b.record()
        copy_ms.append((a, b))
    torch.cuda.synchronize()
    copy_gbps = 2 * COPY_MIB * 1024 * 1024 / (min(a.elapsed_time(b) for a, b in copy_ms) * 1e-3) / 1e9

    sp_busy = [t.busy_ms() * 1e3 for t in sp_timers]
    sp_span = [t.span_ms() * 1e3 for t in sp_timers]
    sp_outer = [t.outer_ms() * 1e3 for t in sp_timers]
    sp_k = by_kernel(sp_timers)
    chunk_name = "sparse_attn_kernel"
    chunk_us = sp_k[chunk_name]
    sel_busy = [select_chain_us(t) for t in sel_timers]
    sel_serial = [t.busy_ms() * 1e3 for t in sel_timers]
    sel_span = [t.span_ms() * 1e3 for t in sel_timers]
    sel_k = by_kernel(sel_timers)
    ex_busy = [t.busy_ms() * 1e3 for t in ex_timers]
    warm_busy = [t.busy_ms() * 1e3 for t in warm_timers]
    tk_busy = [t.busy_ms() * 1e3 for t in tk_timers]
    empty_us = statistics.median([a.elapsed_time(b) * 1e3 for a, b in empty])

    sp_mean = statistics.mean(sp_busy)
    sbytes = sparse_bytes(w)
    cbytes = sparse_chunk_bytes(w) if len(sp_timers[0].names) > 1 else sbytes
    chunk_mean = statistics.mean(chunk_us)
    achieved = cbytes / (chunk_mean * 1e-6) / 1e9
    bytes_sel = select_bytes(w)
    ideal_sel_us = max(bytes_sel / (HBM_PEAK_GBS * 1e9), exact_flops(w) / (BF16_PEAK_TFLOPS * 1e12)) * 1e6
    sel_med = statistics.median(sel_busy)
    ex_med = statistics.median(ex_busy)
    exact_k = statistics.median(sel_k["exact_chunk_kernel"])
    score_k = statistics.median(sel_k["score_kernel"])
    topk_names = [n for n in sel_k if n.startswith("topk")]
    topk_k = sum(statistics.median(sel_k[n]) for n in topk_names)
    ntot = sum(w.seq_lens)
    block_us = statistics.mean(sel_busy) + (T - 1) * sp_mean
    traffic = traffic_record(w.name)
    us = lambda v: round(v, 2)  # noqa: E731
    t0 = time.perf_counter()
    diag = {}
    if not args.no_diag:
        blk_med = statistics.median([t.busy_ms() * 1e3 for t in blk_timers])
        fused_med = statistics.median([t.busy_ms() * 1e3 for t in fused_timers])
        diag["block_attn"] = {
            "gpu_us_median": us(blk_med), "bytes": block_bytes(w),
            "GBps": round(block_bytes(w) / (blk_med * 1e-6) / 1e9, 1),
            "sparse_plus_block_us": us(statistics.median(sp_busy) + blk_med),
            "fused_step_gpu_us_median": us(fused_med),
            "fused_step_kernels_us_median": {n: us(statistics.median(v)) for n, v in by_kernel(fused_timers).items()},
            "note": "cold, not part of value: gpu_us_median = the block's queries over its own B rows merged "
                    "into a sparse step's output through log-sum-exp (separate launch); fused_step = the "
                    "sparse step with the block rows as one more tile per wave of the last split (one call)"}
        diag["page_selection"] = page_diag(torch, mage, r, w, fl)
        diag["head_adaptive_budgets"] = budget_diag(torch, mage, r, w, fl)
        if not w.paged:
            diag["sparse_batch_scaling"] = batch_diag(torch, mage, w, dev, fl)
            log("[bench] sparse batch scaling measured")
    log(f"[bench] page-granular selection measured")
    sp_med = statistics.median(sp_busy)
    if not args.no_diag:
        diag["anchor_recall"] = {
            "iid": anchor_diag(torch, mage, r, w, [r.q1] + r.qs[:T - 1], sel_med, sp_med),
            "walk": anchor_diag(torch, mage, r, w, [r.q1] + [q.to(dev) for q in workloads.walk_queries(w)],
                                sel_med, sp_med),
            "note": "recall = |set in use ∩ step's own top-k| / |own|, mean over (seq, KV head) and "
                    "steps 2..T; iid: the workload's fresh per-step noise around Q1; walk: Q_t = "
                    "Q_(t-1) + N(0, (sigma*sqrt(2/T))^2), a random walk from Q1; block_us = anchors x "
                    "cold exact+select + the rest x cold sparse step"}
    torch.cuda.synchronize()
    log(f"[bench] anchor/recall diagnostic in {time.perf_counter() - t0:.1f} s")
    out = {
        "metric": METRIC,
        "value": round(1e6 / sp_mean, 1),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(block_us * 1e-3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.num_seqs} seq, {w.num_q_heads} q / {w.num_kv_heads} KV heads, "
                               f"d={w.head_dim}, N={'ragged ' + str(list(w.seq_lens)) if w.paged else ntot}, "
                               f"B={w.block}, k={w.k}, {T} steps/block"
                               f"{', 16-token pages, shuffled page table' if w.paged else ''}",
                   "global_batch": w.num_seqs, "seq_len": w.max_seq_len, "parallelism": "single GPU",
                   "step": f"1 bench step = 1 block = step-1 exact+select + {T - 1} sparse steps "
                           f"(ms_per_step); value = sparse denoising steps/s, cold (before each call "
                           f"{FLUSH_DESC[args.flush]}); a call's time is the sum of its kernels' GPU "
                           f"durations"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else traffic["bytes_per_launch"],
                     "kernel": f"{chunk_name} (sparse gather + attention, one launch per step)",
                     "bytes_per_launch": cbytes, "kernel_us_mean": us(chunk_mean),
                     "kernel_us_median": us(statistics.median(chunk_us)), "launches": len(chunk_us),
                     "copy_GBps_measured": round(copy_gbps, 1),
                     "frac_of_measured_copy": round(achieved / copy_gbps, 4)},
        "sparse_step": {"bytes": sbytes, "gpu_us_mean": us(sp_mean),
                        "gpu_us_median": us(statistics.median(sp_busy)),
                        "gpu_us_p10": us(pct(sp_busy, 10)), "gpu_us_p90": us(pct(sp_busy, 90)),
                        "GBps": round(sbytes / (sp_mean * 1e-6) / 1e9, 1),
                        "frac_of_peak": round(sbytes / (sp_mean * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "kernels_us_mean": {n: us(statistics.mean(v)) for n, v in sp_k.items()},
                        "instrumented_span_us_mean": us(statistics.mean(sp_span)),
                        "event_pair_us_mean": us(statistics.mean(sp_outer)),
                        "empty_event_pair_us": us(empty_us),
                        "warm_gpu_us_median": us(statistics.median(warm_busy)),
                        "warm_GBps": round(sbytes / (statistics.median(warm_busy) * 1e-6) / 1e9, 1)},
        "exact_select": {"gpu_us_median": round(sel_med, 1), "roofline_us": round(ideal_sel_us, 1),
                         "roofline_frac": round(ideal_sel_us / sel_med, 4), "bytes": bytes_sel,
                         "timing": "exact pass + the longer of (split merge on the main stream, score sweep + "
                                   "top-k on the select stream), from the kernels' own start/end events",
                         "serial_kernel_sum_us_median": round(statistics.median(sel_serial), 1),
                         "uninstrumented_event_pair_us_median": round(sel_outer, 1),
                         "uninstrumented_roofline_frac": round(ideal_sel_us / sel_outer, 4),
                         "exact_only_uninstrumented_us_median": round(ex_outer, 1),
                         "kernels_us_median": {n: us(statistics.median(v)) for n, v in sel_k.items()},
                         "exact_pass_GBps": round(exact_pass_bytes(w) / (exact_k * 1e-6) / 1e9, 1),
                         "exact_pass_TFLOPs": round(exact_flops(w) / (exact_k * 1e-6) / 1e12, 1),
                         "exact_pass_mfma_frac": round(exact_flops(w) / (exact_k * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "score_GBps": round(score_bytes(w) / (score_k * 1e-6) / 1e9, 1),
                         "topk_us": us(topk_k),
                         "topk_GBps": round(ntot * w.num_kv_heads * 4 / (topk_k * 1e-6) / 1e9, 1),
                         "topk_alone_gpu_us_median": us(statistics.median(tk_busy)),
                         "exact_only_gpu_us_median": round(ex_med, 1),
                         "first_step_overhead": round(sel_med / ex_med - 1, 4),
                         "instrumented_span_us_median": round(statistics.median(sel_span), 1),
                         "event_pair_us_median": round(statistics.median([t.outer_ms() * 1e3 for t in sel_timers]), 1)},
        "selection_overlap": overlap,
        "sparse_graph_replay": graphs,
        "speedup_vs_exact_per_step": round(ex_med / statistics.median(sp_busy), 2),
        "wall_s_timed_region": round(wall, 3),
        "flushes_in_timed_region": args.steps * T if args.flush != "none" else 0,
        "flush": FLUSH_DESC[args.flush],
        "gpu": torch.cuda.get_device_name(0),
        "kernel_source_digest": source_digest(),
    }
    out.update(diag)
    if not args.no_ragged and not w.paged:
        out["ragged_paged"] = ragged_side(torch, mage, dev, fl)
        log("[bench] ragged paged batch measured")
    if traffic is not None:
        out["roofline"]["traffic_source"] = f"profiles/sparse_traffic_{w.name}.md"
    if not args.no_cpu:
        t0 = time.perf_counter()
        cb = cpu_baseline(w, inp)
        out["cpu_baseline"] = {"value": round(cb["value"], 3), "unit": "steps/s", "cores": cb["cores"],
                               "kind": "oracle", "sample": cb["sample"],
                               "select_step_s": round(cb["select_step_s"], 3),
                               "select_step_runs": cb["select_runs"],
                               "cpu_seconds": round(cb["cpu_seconds"], 1),
                               "cpu_model": cpu_model(), "host": platform.machine()}
        log(f"[bench] cpu baseline in {time.perf_counter() - t0:.1f} s")
    print(json.dumps(out), flush=True)


# ---- profile summaries -----------------------------------------------------------
def _short(name: str) -> str:
    for key in ("exact_chunk_kernel", "sparse_attn_kernel", "exact_merge_kernel", "score_kernel",
                "topk_select_kernel", "topk_hist_kernel", "topk_prep_kernel",
                "block_attn_kernel", "mean_query_kernel", "idx_overlap_kernel", "page_sum_kernel",
                "page_expand_kernel", "gap_zero_kernel", "budget_split_kernel", "FillFunctor",
                "neg_kernel", "reduce_kernel"):
        if key in name:
            return {"FillFunctor": "flush (fill)", "neg_kernel": "copy (neg)",
                    "reduce_kernel": "flush (read)"}.get(key, key)
    return name[:60]


def _dispatches(path, value_col=None):
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r.get("Dispatch_Id") or r.get("Correlation_Id") or 0))
    return rows


def _cold_flags(names):
    """A dispatch is cold when the dispatch before it is the 1 GiB flush (its
    read-back, or the fill itself with --flush dirty)."""
    return [i > 0 and names[i - 1] in ("flush (fill)", "flush (read)") and not names[i].startswith("flush")
            for i in range(len(names))]


def summarize_trace(d):
    path = glob.glob(os.path.join(d, "*kernel_trace.csv"))[0]
    rows = _dispatches(path)
    names = [_short(r["Kernel_Name"]) for r in rows]
    cold = _cold_flags(names)
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    agg = {}
    for n, c, t in zip(names, cold, dur):
        a = agg.setdefault(n, {"all": [], "cold": []})
        a["all"].append(t)
        if c:
            a["cold"].append(t)
    print("| kernel | dispatches | mean us (all) | cold dispatches | mean us (cold) | median us (cold) |")
    print("|---|---|---|---|---|---|")
    for n, a in sorted(agg.items(), key=lambda kv: -sum(kv[1]["all"])):
        c = a["cold"]
        print(f"| {n} | {len(a['all'])} | {statistics.mean(a['all']):.2f} | {len(c)} | "
              f"{statistics.mean(c) if c else float('nan'):.2f} | {statistics.median(c) if c else float('nan'):.2f} |")
    # step-1 timelines: every cold exact pass and the dispatches after it up to the next flush,
    # in start order, relative to the exact pass's start (both streams)
    order = sorted(range(len(rows)), key=lambda i: int(rows[i]["Start_Timestamp"]))
    lines = []
    for j, i in enumerate(order):
        if names[i] != "exact_chunk_kernel" or not cold[i]:
            continue
        t0 = int(rows[i]["Start_Timestamp"])
        seq = []
        for i2 in order[j:]:
            if names[i2].startswith("flush"):
                break
            seq.append(f"{names[i2]} {(int(rows[i2]['Start_Timestamp']) - t0) / 1e3:.1f}-"
                       f"{(int(rows[i2]['End_Timestamp']) - t0) / 1e3:.1f}")
        lines.append("; ".join(seq))
    if lines:
        print()
        print("Step-1 timelines (cold exact pass and what follows it until the next flush; us from its start):")
        print()
        for ln in lines[:6]:
            print(f"- {ln}")


def summarize_pmc(fetch_dir, write_dir, config):
    w = workloads.CONFIG_BY_NAME[config]

    def load(d, counter):
        path = glob.glob(os.path.join(d, "*counter_collection.csv"))[0]
        rows = [r for r in _dispatches(path) if r["Counter_Name"] == counter]
        names = [_short(r["Kernel_Name"]) for r in rows]
        cold = _cold_flags(names)
        vals = {}
        for n, c, r in zip(names, cold, rows):
            vals.setdefault(n, {"all": [], "cold": []})["all"].append(float(r["Counter_Value"]))
            if c:
                vals[n]["cold"].append(float(r["Counter_Value"]))
        return vals

    f, wr = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    copy_bytes = COPY_MIB * 1024 * 1024
    cf = copy_bytes / (statistics.mean(f["copy (neg)"]["all"]) * 1024)
    cw = copy_bytes / (statistics.mean(wr["copy (neg)"]["all"]) * 1024)
    # the later step is one launch (its split merge runs in its last work-groups): K/V rows, Q and O
    algo = {"sparse_attn_kernel": sparse_bytes(w), "exact_chunk_kernel": exact_pass_bytes(w),
            "score_kernel": score_bytes(w), "copy (neg)": 2 * copy_bytes}
    print(f"Copy calibration: a {COPY_MIB} MiB fp32 copy (torch.neg) reads {COPY_MIB} MiB and writes "
          f"{COPY_MIB} MiB; FETCH_SIZE reads {copy_bytes / cf / 1024:.0f} KiB and WRITE_SIZE "
          f"{copy_bytes / cw / 1024:.0f} KiB per dispatch, so bytes = FETCH_SIZE KiB x 1024 x {cf:.4f} "
          f"and WRITE_SIZE KiB x 1024 x {cw:.4f}.\n")
    print("| kernel | cold dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | calibrated MB | algorithmic MB | ratio |")
    print("|---|---|---|---|---|---|---|")
    rec = None
    for n in sorted(f):
        fc = f[n]["cold"] or f[n]["all"]
        wc = (wr.get(n, {}).get("cold") or wr.get(n, {}).get("all") or [0.0])
        fb, wb = statistics.mean(fc) * 1024 * cf, statistics.mean(wc) * 1024 * cw
        a = algo.get(n)
        print(f"| {n} | {len(f[n]['cold'])} | {statistics.mean(fc):.0f} | {statistics.mean(wc):.0f} | "
              f"{(fb + wb) / 1e6:.2f} | {'' if a is None else f'{a / 1e6:.2f}'} | "
              f"{'' if a is None else f'{(fb + wb) / a:.3f}'} |")
        if n == "sparse_attn_kernel":
            rec = {"config": config, "kernel": n, "bytes_per_launch": int(round(fb + wb)),
                   "fetch_bytes": int(round(fb)), "write_bytes": int(round(wb)),
                   "fetch_factor": round(cf, 5), "write_factor": round(cw, 5),
                   "source_digest": source_digest()}
    print()
    if rec is not None:
        print("traffic: " + json.dumps(rec))


def summarize_counters(d, config):
    """Per kernel class, from one rocprofv3 --pmc run of MfmaUtil (rocprofv3's
    derived metric: SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE times the
    SIMD count), TCC_HIT_sum and TCC_MISS_sum: the MFMA busy share of the SIMD
    cycles and the L2 hit rate."""
    path = glob.glob(os.path.join(d, "*counter_collection.csv"))[0]
    per = {}
    for r in _dispatches(path):
        key = int(r["Dispatch_Id"])
        e = per.setdefault(key, {"name": _short(r["Kernel_Name"]),
                                 "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        e[r["Counter_Name"]] = float(r["Counter_Value"])
    keys = sorted(per)
    cold = dict(zip(keys, _cold_flags([per[k]["name"] for k in keys])))
    print(f"Config {config}. MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs), as rocprofv3 "
          "derives it; L2 hit = TCC_HIT / (TCC_HIT + TCC_MISS). Cold dispatches (right after the flush) "
          "are averaged where there are any.\n")
    print("| kernel | dispatches (cold) | MFMA busy | L2 hit |")
    print("|---|---|---|---|")
    by = {}
    for k in keys:
        by.setdefault(per[k]["name"], []).append(k)
    for n in sorted(by):
        e = [per[k] for k in ([k for k in by[n] if cold[k]] or by[n])]
        util = statistics.mean(x.get("MfmaUtil", 0.0) for x in e)
        hit = statistics.mean(x.get("TCC_HIT_sum", 0.0) for x in e)
        miss = statistics.mean(x.get("TCC_MISS_sum", 0.0) for x in e)
        print(f"| {n} | {len(by[n])} ({sum(cold[k] for k in by[n])}) | {util:.1f}% | "
              f"{'' if hit + miss == 0 else f'{100 * hit / (hit + miss):.1f}%'} |")
    print()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10, help="timed blocks (each: step 1 + T-1 sparse steps)")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="head128k", choices=sorted(workloads.CONFIG_BY_NAME))
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-ragged", action="store_true",
                    help="skip the ragged paged batch measured beside a contiguous workload")
    ap.add_argument("--no-diag", action="store_true",
                    help="skip the next-row measurements (block attention, anchors and recall, page "
                         "selection, head-adaptive budgets): profiler runs of the main path")
    ap.add_argument("--flush", choices=sorted(FLUSH_DESC), default="clean",
                    help="cache state before each timed call")
    ap.add_argument("--no-flush", action="store_true", help="same as --flush none")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="MFMA busy, L2 hit rate and clock per kernel from a counter run")
    args = ap.parse_args()
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace)
    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc, args.config)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters, args.config)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    run_bench(args)


if __name__ == "__main__":
    main()
