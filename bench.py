"""Benchmark of the MAGE hot path on one MI355X.

One bench step = one block of block-diffusion decoding for one layer: step 1
(exact attention + block-averaged scores + top-k on a second stream), then
T-1 sparse steps over the reused index set with fresh queries. Default
workload: 1 sequence, 32 query / 8 KV heads, d=128, N=131072 prefix, B=32,
k=1024, T=32 (the MAGE page's headline shape under "Key results").

Protocol: inputs are resident in HBM before timing. Before every timed step a
1 GiB scratch buffer is overwritten on the same stream (outside the timed
window) so that K/V rows come from HBM, not from L2 or the 256 MB MALL; each
step is bracketed by HIP events on the stream its kernels run on. `value` is
sparse steps per second (cold); the warm (no flush) figure is reported
separately as cache bandwidth.

    python bench.py [--steps K] [--warmup W] [--config head128k] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_sparse_kv_amd as mage  # noqa: E402
import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "sparse-step denoising steps/sec and HBM GB/s (% peak) at 128K ctx, k=1024, B=32"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sparse_bytes(w: workloads.Workload) -> int:
    """Algorithmic bytes of one sparse step: k_eff rows of K and V per (seq, KV head),
    plus Q (bf16) read and O (fp32) written."""
    d = w.head_dim
    rows = sum(w.k_eff(s) for s in range(w.num_seqs)) * w.num_kv_heads
    q = w.num_seqs * w.block * w.num_q_heads * d * 2
    o = w.num_seqs * w.block * w.num_q_heads * d * 4
    return rows * d * 2 * 2 + q + o


def select_bytes(w: workloads.Workload) -> int:
    """Algorithmic bytes of step 1: Q + K + V read once, O + lse written, the
    scores written and read back once, idx written."""
    d, S, Hkv = w.head_dim, w.num_seqs, w.num_kv_heads
    ntot = sum(w.seq_lens)
    q = S * w.block * w.num_q_heads * d * 2
    kv = ntot * Hkv * d * 2 * 2
    o = S * w.block * w.num_q_heads * (d + 1) * 4
    sc = ntot * Hkv * 4 * 2
    idx = S * Hkv * w.k * 4
    return q + kv + o + sc + idx


def exact_flops(w: workloads.Workload) -> float:
    return 4.0 * w.block * w.num_q_heads * w.head_dim * sum(w.seq_lens)


class Runner:
    def __init__(self, w, inp, dev):
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

    def select(self):
        w = self.w
        kw = dict(o=self.o, lse=self.lse, idx=self.idx, scores=self.scores, workspace=self.ws,
                  select_stream=self.side, idx_ready=self.ready)
        if w.paged:
            mage.select_exact_paged(self.q1, self.kp, self.vp, self.table, self.lens, w.k, w.scale, **kw)
        else:
            mage.select_exact(self.q1, self.k, self.v, w.k, w.scale, **kw)
        torch.cuda.current_stream().wait_event(self.ready)

    def exact_only(self):
        w = self.w
        if w.paged:
            mage.exact_attn_paged(self.q1, self.kp, self.vp, self.table, self.lens, w.scale,
                                  o=self.o, lse=self.lse, workspace=self.ws)
        else:
            mage.exact_attn(self.q1, self.k, self.v, w.scale, o=self.o, lse=self.lse, workspace=self.ws)

    def sparse(self, t):
        w = self.w
        q = self.qs[t % len(self.qs)]
        if w.paged:
            mage.sparse_attn_paged(q, self.kp, self.vp, self.table, self.lens, self.idx, w.scale,
                                   o=self.o2, lse=self.lse2, workspace=self.ws)
        else:
            mage.sparse_attn(q, self.k, self.v, self.idx, w.scale, o=self.o2, lse=self.lse2,
                             workspace=self.ws)

    def topk_only(self):
        w = self.w
        S, Hkv = w.num_seqs, w.num_kv_heads
        lens = None if not w.paged else [n for n in w.seq_lens for _ in range(Hkv)]
        mage.topk(self.scores.view(S * Hkv, -1), w.k, lens=lens, idx=self.idx.view(S * Hkv, -1),
                  workspace=self.ws)


def timed(fn, flush, n):
    """Per-call HIP-event durations (ms) of fn, each preceded by a cache flush."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        if flush is not None:
            flush()
        evs[i][0].record()
        fn(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def cpu_baseline(w, inp, max_seconds=30.0):
    """The fp64 oracle on the host cores over a bounded sample of the same workload."""
    import oracle
    res = {}
    # one full sparse step (every KV head) with the GPU-independent oracle index set of head 0 reused
    S, Hkv = w.num_seqs, w.num_kv_heads
    G = w.group
    n0 = w.seq_lens[0]
    # step-1 exact + select for KV head 0 of sequence 0
    q1 = inp.q1[:1, :, 0:G].contiguous()
    if w.paged:
        kc = torch.from_numpy(oracle.depage(inp.k_pool, inp.page_table[:1], [n0])[0][None, :1].copy()).view(torch.bfloat16)
        vc = torch.from_numpy(oracle.depage(inp.v_pool, inp.page_table[:1], [n0])[0][None, :1].copy()).view(torch.bfloat16)
        kfull = vfull = None
    else:
        kc, vc = inp.k[:1, :1].contiguous(), inp.v[:1, :1].contiguous()
        kfull, vfull = inp.k, inp.v
    t0 = time.perf_counter()
    _, _, _, idx0 = oracle.select_exact(q1, kc, vc, w.scale, w.k)
    t_sel_head = time.perf_counter() - t0
    res["select_one_head_s"] = t_sel_head
    # sparse steps over all heads (contiguous workloads) or head 0 (paged)
    if kfull is not None:
        idx = np.repeat(idx0, Hkv, axis=1)
        runs = []
        while len(runs) < 5 and sum(runs) < max_seconds / 3:
            t0 = time.perf_counter()
            oracle.sparse(inp.q_steps[0], kfull, vfull, idx, w.scale)
            runs.append(time.perf_counter() - t0)
        t_sparse = statistics.median(runs)
        sample = (f"oracle: step-1 exact+select of 1 of {S * Hkv} (seq, KV head) units "
                  f"({t_sel_head:.2f} s), then {len(runs)} full sparse steps over all {Hkv} KV heads "
                  f"(median {t_sparse * 1e3:.1f} ms)")
    else:
        runs = []
        while len(runs) < 5 and sum(runs) < max_seconds / 3:
            t0 = time.perf_counter()
            oracle.sparse(inp.q_steps[0][:1, :, 0:G].contiguous(), kc, vc, idx0, w.scale)
            runs.append(time.perf_counter() - t0)
        t_sparse = statistics.median(runs) * S * Hkv
        sample = (f"oracle: step-1 exact+select and {len(runs)} sparse steps of (seq 0, KV head 0), "
                  f"scaled x{S * Hkv} to the whole batch")
    res["value"] = 1.0 / t_sparse
    res["select_step_s_est"] = t_sel_head * S * Hkv * (sum(w.seq_lens) / (n0 * S))
    res["sample"] = sample
    res["cores"] = oracle.num_threads()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10, help="timed blocks (each: step 1 + T-1 sparse steps)")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="head128k", choices=sorted(workloads.CONFIG_BY_NAME))
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-flush", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    w = workloads.CONFIG_BY_NAME[args.config]
    t0 = time.perf_counter()
    inp = workloads.make_inputs(w)
    log(f"[bench] inputs for {w.name} drawn in {time.perf_counter() - t0:.1f} s")
    r = Runner(w, inp, dev)
    scratch = torch.empty(256 * 1024 * 1024, dtype=torch.int32, device=dev)   # 1 GiB
    fill = [0]

    def flush():
        fill[0] += 1
        scratch.fill_(fill[0])

    fl = None if args.no_flush else flush
    T = w.steps
    # warm-up
    for _ in range(args.warmup):
        r.select()
        for t in range(T - 1):
            r.sparse(t)
    torch.cuda.synchronize()
    log("[bench] warm-up done")

    # timed region: K blocks
    sel_ms, sp_ms = [], []
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for _ in range(args.steps):
        sel_ms += timed(lambda i: r.select(), fl, 1)
        sp_ms += timed(lambda i: r.sparse(i), fl, T - 1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    log(f"[bench] timed {args.steps} blocks in {wall:.2f} s wall")

    # secondary measurements
    exact_ms = timed(lambda i: r.exact_only(), fl, 5)
    warm = timed(lambda i: r.sparse(i), None, 3 * (T - 1))
    r.select()
    torch.cuda.synchronize()
    topk_ms = timed(lambda i: r.topk_only(), fl, 5)
    empty = timed(lambda i: None, None, 20)

    sp_med = statistics.median(sp_ms)
    sp_mean = statistics.mean(sp_ms)
    sel_med = statistics.median(sel_ms)
    block_ms = statistics.mean(sel_ms) + (T - 1) * sp_mean
    sbytes = sparse_bytes(w)
    gbs = sbytes / (sp_mean * 1e-3) / 1e9
    bytes_sel = select_bytes(w)
    ideal_sel_us = max(bytes_sel / (HBM_PEAK_GBS * 1e9), exact_flops(w) / (BF16_PEAK_TFLOPS * 1e12)) * 1e6
    ntot = sum(w.seq_lens)
    out = {
        "metric": METRIC,
        "value": round(1e3 / sp_mean, 1),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(block_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.num_seqs} seq, {w.num_q_heads} q / {w.num_kv_heads} KV heads, "
                               f"d={w.head_dim}, N={'ragged ' if w.paged else ''}{ntot if not w.paged else list(w.seq_lens)}, "
                               f"B={w.block}, k={w.k}, {T} steps/block"
                               f"{', 16-token pages' if w.paged else ''}",
                   "global_batch": w.num_seqs, "seq_len": w.max_seq_len, "parallelism": "single GPU",
                   "step": f"1 block = step-1 exact+select + {T - 1} sparse steps; value = sparse steps/s (cold)"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "attn_chunk_kernel<128, sparse> (one launch per sparse step)",
                     "bytes_per_launch": sbytes},
        "sparse_step_us": {"mean": round(sp_mean * 1e3, 2), "median": round(sp_med * 1e3, 2),
                           "p10": round(float(np.percentile(sp_ms, 10)) * 1e3, 2),
                           "p90": round(float(np.percentile(sp_ms, 90)) * 1e3, 2),
                           "warm_median": round(statistics.median(warm) * 1e3, 2),
                           "warm_GBps": round(sbytes / (statistics.median(warm) * 1e-3) / 1e9, 1),
                           "empty_event_pair_us": round(statistics.median(empty) * 1e3, 2)},
        "exact_select_us": {"median": round(sel_med * 1e3, 1),
                            "roofline_us": round(ideal_sel_us, 1),
                            "roofline_frac": round(ideal_sel_us / (sel_med * 1e3), 4),
                            "bytes": bytes_sel,
                            "exact_only_median_us": round(statistics.median(exact_ms) * 1e3, 1),
                            "first_step_overhead": round(sel_med / statistics.median(exact_ms) - 1, 4),
                            "exact_GBps": round(bytes_sel / (statistics.median(exact_ms) * 1e-3) / 1e9, 1),
                            "exact_TFLOPs": round(exact_flops(w) / (statistics.median(exact_ms) * 1e-3) / 1e12, 1),
                            "topk_median_us": round(statistics.median(topk_ms) * 1e3, 2),
                            "topk_GBps": round(ntot * w.num_kv_heads * 4 / (statistics.median(topk_ms) * 1e-3) / 1e9, 1)},
        "speedup_vs_exact_per_step": round(statistics.median(exact_ms) / sp_med, 2),
        "wall_s_timed_region": round(wall, 3),
        "gpu": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu:
        t0 = time.perf_counter()
        cb = cpu_baseline(w, inp)
        out["cpu_baseline"] = {"value": round(cb["value"], 4), "unit": "steps/s", "cores": cb["cores"],
                               "kind": "oracle", "sample": cb["sample"],
                               "select_step_s_est": round(cb["select_step_s_est"], 2),
                               "host": platform.processor() or platform.machine()}
        log(f"[bench] cpu baseline in {time.perf_counter() - t0:.1f} s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
