"""Seeded synthetic inputs for block-shared top-k sparse KV attention.

This module only draws inputs. It holds none of the method's arithmetic (no
attention, no scoring, no selection), so the CPU oracle under ``oracle/`` and
the HIP path under ``block_sparse_kv_amd/`` can both be fed from it without
sharing anything else.

Workloads (shapes from the MAGE page on atlas.scime.ai, "Key results": 128K
context, k=1024, 32 denoising steps per block; the other shapes are synthetic
stand-ins for the LongBench / Needle-in-a-Haystack runs named under
"Experimental setup", which need datasets and trained weights):

* ``tiny``     1 seq, 1/1 heads, d=64,  N=1024,  B=16, k=64,   4 steps
* ``gqa32k``   1 seq, 32/8 heads, d=128, N=32768, B=32, k=512,  32 steps
* ``head128k`` 1 seq, 32/8 heads, d=128, N=131072, B=32, k=1024, 32 steps
* ``mha64k``   1 seq, 16/16 heads, d=128, N=65536, B=64, k=256, 16 steps
* ``ragged``   8 seqs, N in {8K,16K,24K,32K,48K,64K,96K,128K}, 32/8 heads,
               d=128, B=32, k=1024, 32 steps, 16-token pages, shuffled table

Recipe (values drawn in fp32, rounded to bf16 once, round-to-nearest-even):

* Q1 ~ N(0,1); for d=128 workloads it is pre-scaled by 1/sqrt(128) and the
  softmax scale is 1.0; the tiny workload keeps Q1 ~ N(0,1) and uses scale
  1/sqrt(64) = 0.125.
* K, V ~ N(0,1).
* Planted keys (all but ``mha64k``): ``tiny`` plants 16 keys with
  K[p] += 3 * mean_b(Q1[b]); the others plant 2% of positions per
  (seq, KV head) with K[p] += 3 * sqrt(d) * m_hat, m_hat the unit vector of
  the mean of Q1 over the block's B tokens and the head group's G query heads.
* ``mha64k``: 10% of positions per (seq, head) are replaced by
  c_j + N(0, 0.01^2), centroids c_j ~ N(0, I_d), j uniform over 64 centroids.
* Later steps: Q_t = Q1 + N(0, sigma^2) with fresh noise per step (sigma 0.1
  for ``tiny``, 0.05 otherwise).
* Random-walk drift (``walk_queries``, for the anchor re-selection
  diagnostic only): Q_t = Q_{t-1} + N(0, tau^2) with tau = sigma * sqrt(2/T),
  so the drift from Q1 has standard deviation sigma half-way through the
  block and keeps growing after that.
* Paged: the pool is [P][Hkv][page][d]; physical page ids are a seeded
  permutation of 0..P-1 handed out in order to each sequence's logical pages.

Every stream comes from ``numpy.random.SeedSequence(seed, spawn_key=...)``
with a spawn key naming its purpose and (seq, head), so draws are independent
of thread scheduling and of which parts a caller asks for.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
import os

import numpy as np
import torch

# spawn-key purposes
_Q1, _K, _V, _PLANT, _CLUSTER, _NOISE, _PERM, _WALK = range(8)


@dataclass(frozen=True)
class Workload:
    name: str
    seq_lens: tuple            # N_s per sequence
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block: int                 # B, query tokens per block
    k: int                     # top-k budget per (seq, KV head)
    steps: int                 # T, denoising steps per block (1 exact + T-1 sparse)
    paged: bool = False
    page_size: int = 16
    keys: str = "plant_unit"   # "plant_mean" | "plant_unit" | "clusters" | "plain"
    num_plants: int | None = None   # absolute count (tiny); else plant_frac of N_s
    plant_frac: float = 0.02
    q_noise: float = 0.05
    q_prescale: bool = True    # Q1 multiplied by 1/sqrt(d)
    seed: int = 0

    @property
    def num_seqs(self) -> int:
        return len(self.seq_lens)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def rows(self) -> int:
        """Query rows per KV head: B tokens x G query heads."""
        return self.block * self.group

    @property
    def scale(self) -> float:
        return 1.0 if self.q_prescale else 1.0 / math.sqrt(self.head_dim)

    @property
    def max_seq_len(self) -> int:
        return max(self.seq_lens)

    def k_eff(self, s: int) -> int:
        return min(self.k, self.seq_lens[s])


def _tiny(seed):
    return Workload("tiny", (1024,), 1, 1, 64, 16, 64, 4, keys="plant_mean",
                    num_plants=16, q_noise=0.1, q_prescale=False, seed=seed)


CONFIGS = [
    _tiny(1000),
    Workload("gqa32k", (32768,), 32, 8, 128, 32, 512, 32, seed=1001),
    Workload("head128k", (131072,), 32, 8, 128, 32, 1024, 32, seed=1002),
    Workload("mha64k", (65536,), 16, 16, 128, 64, 256, 16, keys="clusters",
             seed=1003),
    Workload("ragged", tuple(n * 1024 for n in (8, 16, 24, 32, 48, 64, 96, 128)),
             32, 8, 128, 32, 1024, 32, paged=True, seed=1004),
]
CONFIG_BY_NAME = {c.name: c for c in CONFIGS}


def custom(seq_lens, num_q_heads, num_kv_heads, head_dim, block, k, steps=2, *,
           paged=False, page_size=16, keys="plant_unit", seed=7, q_noise=0.05,
           q_prescale=True, num_plants=None, plant_frac=0.02, name="custom"):
    """A small workload with the same recipe, for tests."""
    return Workload(name, tuple(int(n) for n in seq_lens), num_q_heads, num_kv_heads,
                    head_dim, block, k, steps, paged=paged, page_size=page_size,
                    keys=keys, num_plants=num_plants, plant_frac=plant_frac,
                    q_noise=q_noise, q_prescale=q_prescale, seed=seed)


def _rng(seed, *key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs), numpy only.

    Used inside the generator's worker threads, which must not call torch (its
    CPU kernels start an OpenMP team per calling thread)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _u16_view(t: torch.Tensor) -> np.ndarray:
    """numpy uint16 view sharing the storage of a bf16 CPU tensor."""
    return t.view(torch.int16).numpy().view(np.uint16)


def _q1_f32(w: Workload) -> np.ndarray:
    q = _rng(w.seed, _Q1).standard_normal(
        (w.num_seqs, w.block, w.num_q_heads, w.head_dim), dtype=np.float32)
    if w.q_prescale:
        q *= np.float32(1.0 / math.sqrt(w.head_dim))
    return q


def _kv_head(w: Workload, q1: np.ndarray, s: int, h: int):
    """K, V of one (seq, KV head) as fp32 [N_s][d], plus the planted positions."""
    n, d = w.seq_lens[s], w.head_dim
    kk = _rng(w.seed, _K, s, h).standard_normal((n, d), dtype=np.float32)
    vv = _rng(w.seed, _V, s, h).standard_normal((n, d), dtype=np.float32)
    plants = np.zeros(0, dtype=np.int64)
    if w.keys in ("plant_mean", "plant_unit"):
        r = _rng(w.seed, _PLANT, s, h)
        cnt = w.num_plants if w.num_plants is not None else int(round(w.plant_frac * n))
        cnt = min(cnt, n)
        plants = np.sort(r.choice(n, size=cnt, replace=False))
        g = w.group
        m = q1[s, :, h * g:(h + 1) * g, :].astype(np.float64).mean(axis=(0, 1))
        if w.keys == "plant_mean":
            add = 3.0 * m
        else:
            nrm = np.linalg.norm(m)
            add = 3.0 * math.sqrt(d) * (m / nrm if nrm > 0 else m)
        kk[plants] += add.astype(np.float32)
    elif w.keys == "clusters":
        r = _rng(w.seed, _CLUSTER, s, h)
        cent = r.standard_normal((64, d), dtype=np.float32)
        cnt = int(round(0.1 * n))
        pos = r.choice(n, size=cnt, replace=False)
        which = r.integers(0, 64, size=cnt)
        kk[pos] = cent[which] + np.float32(0.01) * r.standard_normal((cnt, d), dtype=np.float32)
    return kk, vv, plants


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def step_queries(w: Workload, q1f: np.ndarray | None = None, steps=None):
    """Q_t for t = 2..T as bf16 tensors (fresh noise per step)."""
    if q1f is None:
        q1f = _q1_f32(w)
    out = []
    for t in range(2, (steps or w.steps) + 1):
        noise = _rng(w.seed, _NOISE, t).standard_normal(q1f.shape, dtype=np.float32)
        out.append(_bf16(q1f + np.float32(w.q_noise) * noise))
    return out


def walk_queries(w: Workload, q1f: np.ndarray | None = None, steps=None):
    """Q_t for t = 2..T as bf16 tensors under a random-walk drift from Q1."""
    if q1f is None:
        q1f = _q1_f32(w)
    T = steps or w.steps
    tau = np.float32(w.q_noise * math.sqrt(2.0 / T))
    out, cur = [], q1f.copy()
    for t in range(2, T + 1):
        cur = cur + tau * _rng(w.seed, _WALK, t).standard_normal(q1f.shape, dtype=np.float32)
        out.append(_bf16(cur))
    return out


@dataclass
class Inputs:
    w: Workload
    q1: torch.Tensor                 # bf16 [S][B][Hq][d]
    q_steps: list                    # bf16 [S][B][Hq][d] for t = 2..T
    k: torch.Tensor | None = None    # bf16 [S][Hkv][N][d] (contiguous workloads)
    v: torch.Tensor | None = None
    k_pool: torch.Tensor | None = None   # bf16 [P][Hkv][page][d] (paged workloads)
    v_pool: torch.Tensor | None = None
    page_table: torch.Tensor | None = None  # int32 [S][max_pages], -1 past the end
    seq_lens: torch.Tensor | None = None    # int32 [S]
    plants: dict = field(default_factory=dict)  # (s, h) -> planted positions


def make_inputs(w: Workload | int | str, *, steps: int | None = None,
                with_steps: bool = True) -> Inputs:
    """Draw every input of a workload (a Workload, a CONFIGS index or a name)."""
    if isinstance(w, int):
        w = CONFIGS[w]
    elif isinstance(w, str):
        w = CONFIG_BY_NAME[w]
    S, Hkv, d = w.num_seqs, w.num_kv_heads, w.head_dim
    q1f = _q1_f32(w)
    q1 = _bf16(q1f)
    jobs = [(s, h) for s in range(S) for h in range(Hkv)]
    plants = {}
    lens = torch.tensor(w.seq_lens, dtype=torch.int32)
    if not w.paged:
        if len(set(w.seq_lens)) != 1:
            raise ValueError("contiguous workloads need one prefix length for all sequences")
        n = w.seq_lens[0]
        k = torch.empty((S, Hkv, n, d), dtype=torch.bfloat16)
        v = torch.empty_like(k)
        kn, vn = _u16_view(k), _u16_view(v)

        def fill(job):
            s, h = job
            kk, vv, pl = _kv_head(w, q1f, s, h)
            kn[s, h] = _bf16_bits(kk)
            vn[s, h] = _bf16_bits(vv)
            plants[job] = pl
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, jobs))
        inp = Inputs(w, q1, [], k=k, v=v, seq_lens=lens, plants=plants)
    else:
        ps = w.page_size
        npages = [(n + ps - 1) // ps for n in w.seq_lens]
        P = sum(npages)
        perm = _rng(w.seed, _PERM).permutation(P).astype(np.int64)
        table = np.full((S, max(npages)), -1, dtype=np.int32)
        off = 0
        for s, np_ in enumerate(npages):
            table[s, :np_] = perm[off:off + np_]
            off += np_
        k_pool = torch.zeros((P, Hkv, ps, d), dtype=torch.bfloat16)
        v_pool = torch.zeros_like(k_pool)
        kpn, vpn = _u16_view(k_pool), _u16_view(v_pool)

        def fill(job):
            s, h = job
            kk, vv, pl = _kv_head(w, q1f, s, h)
            n = w.seq_lens[s]
            pad = npages[s] * ps - n
            kb = _bf16_bits(np.pad(kk, ((0, pad), (0, 0)))).reshape(npages[s], ps, d)
            vb = _bf16_bits(np.pad(vv, ((0, pad), (0, 0)))).reshape(npages[s], ps, d)
            ids = table[s, :npages[s]].astype(np.int64)
            kpn[ids, h] = kb
            vpn[ids, h] = vb
            plants[job] = pl
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, jobs))
        inp = Inputs(w, q1, [], k_pool=k_pool, v_pool=v_pool,
                     page_table=torch.from_numpy(table), seq_lens=lens, plants=plants)
    if with_steps:
        inp.q_steps = step_queries(w, q1f, steps)
    return inp


def to_paged(k: torch.Tensor, v: torch.Tensor, page_size: int, seed: int):
    """Scatter a contiguous [S][Hkv][N][d] cache into a shuffled page pool.

    Returns (k_pool, v_pool, page_table, seq_lens) with the same layout as the
    paged workloads, so a test can run one cache through both addressings.
    """
    S, Hkv, n, d = k.shape
    npg = (n + page_size - 1) // page_size
    P = S * npg
    perm = _rng(seed, _PERM).permutation(P).astype(np.int64)
    table = perm.reshape(S, npg).astype(np.int32)
    pad = npg * page_size - n
    k_pool = torch.zeros((P, Hkv, page_size, d), dtype=k.dtype)
    v_pool = torch.zeros_like(k_pool)
    for s in range(S):
        ids = torch.from_numpy(table[s].astype(np.int64))
        kp = torch.nn.functional.pad(k[s], (0, 0, 0, pad)).view(Hkv, npg, page_size, d)
        vp = torch.nn.functional.pad(v[s], (0, 0, 0, pad)).view(Hkv, npg, page_size, d)
        k_pool[ids] = kp.permute(1, 0, 2, 3)
        v_pool[ids] = vp.permute(1, 0, 2, 3)
    return k_pool, v_pool, torch.from_numpy(table), torch.full((S,), n, dtype=torch.int32)


def random_scores(num_heads: int, n: int, *, seed: int, ties: str = "none") -> torch.Tensor:
    """fp32 score-like arrays (non-negative) for exercising top-k on its own.

    ties: "none" (continuous values), "many" (values drawn from a small set so
    that the threshold falls inside a run of equal values), "all" (every value
    equal), "zeros" (mostly +0.0 with a few positive values).
    """
    r = _rng(seed, 99)
    if ties == "none":
        a = r.exponential(1.0, size=(num_heads, n)).astype(np.float32) / np.float32(n)
    elif ties == "many":
        a = (r.integers(0, 37, size=(num_heads, n)).astype(np.float32) / np.float32(64.0))
    elif ties == "all":
        a = np.full((num_heads, n), np.float32(1.0 / max(n, 1)), dtype=np.float32)
    elif ties == "zeros":
        a = np.zeros((num_heads, n), dtype=np.float32)
        m = r.random((num_heads, n)) < 0.05
        a[m] = r.random(int(m.sum())).astype(np.float32)
    else:
        raise ValueError(ties)
    return torch.from_numpy(a)
