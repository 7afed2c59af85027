"""Seeded synthetic inputs for the fused chunked top-K KL loss.

This module is shared by the tests, the benchmark and the smoke check. It only draws
inputs: student hidden states H[N,d], the LM-head weight W[V,d] and the offline top-K
teacher cache (token ids idx[N,K] and logits t[N,K]). It holds none of the loss
arithmetic, so neither the oracle nor the GPU path depends on it for anything but data.

Workloads follow the pages' head shape (gpt-oss-120b: V = 201,088, S = 32K, B = 4, and a
top-100 teacher cache per position; "Making knowledge distillation cheap enough to run in
production", paragraphs on the dense teacher tensor and the offline cache), plus smaller
heads of the same structure. Teacher rows come in two kinds, following that page's remark
that top-K caching is harmless for confident (peaked) positions and lossy for ambiguous
(flat) ones:

* peaked row: r_2..r_K ~ N(0,1) sorted descending and t_1 = T*log(1.5*sum_k exp(r_k/T)),
  which gives the top entry probability 0.6 under softmax(t/T) before storage rounding;
* flat row: t ~ N(0, var) sorted descending (var = 0.5 unless the config says otherwise).

Token ids are distinct within a row. Either uniform over the vocabulary, or Zipf(1.1)
over ranks 1..V (weight r^-1.1, token id = rank - 1) drawn one at a time with repeats
rejected, which is sampling without replacement with successive renormalisation.

N(mu, var) is written with the variance, as W ~ N(0, 1/d) keeps the logits O(1).

Every array is drawn in fixed blocks of rows; block j of stream s uses
``PCG64([seed, s, j])``. Row n of every array is therefore the same whatever the total
number of rows, and blocks can be drawn on several threads. bf16 storage is represented
by its 16-bit patterns (numpy has no bf16 type), rounded to nearest even.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "CONFIGS",
    "Problem",
    "make",
    "bf16_bits",
    "bf16_to_f32",
    "normal_rows",
    "uniform_distinct",
    "zipf_distinct",
    "peaked_logits",
    "flat_logits",
]

# Stream offsets within one config seed.
_S_H, _S_W, _S_IDX, _S_T, _S_KIND = 0, 1, 2, 3, 4
_BLOCK = 2048  # rows per generator block

# name -> recipe.  "mix" draws each row's kind with Bernoulli(1/2): peaked rows take Zipf ids,
# flat rows take uniform ids.
CONFIGS = {
    "tiny": dict(B=1, S=256, d=128, V=2048, K=16, T=1.0, chunk=64, dtype="fp32",
                 teacher="normal", teacher_var=2.0, ids="uniform", seed=1000),
    "small": dict(B=2, S=2048, d=1024, V=32000, K=100, T=1.0, chunk=1024, dtype="bf16",
                  teacher="peaked", ids="zipf", seed=1001),
    "qwen": dict(B=1, S=8192, d=2048, V=151936, K=100, T=2.0, chunk=2048, dtype="bf16",
                 teacher="flat", teacher_var=0.5, ids="uniform", seed=1002,
                 chunk_sweep=(512, 1024, 2048, 4096)),
    "gptoss": dict(B=1, S=32768, d=2880, V=201088, K=100, T=1.0, chunk=2048, dtype="bf16",
                   teacher="mix", teacher_var=0.5, ids="mix", seed=1003),
    "full": dict(B=4, S=32768, d=2880, V=201088, K=100, T=1.0, chunk=4096, dtype="bf16",
                 teacher="mix", teacher_var=0.5, ids="mix", seed=1004),
}


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _rng(seed: int, stream: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), int(stream), int(block)]))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    return ((u + (((u >> 16) & 1) + np.uint32(0x7FFF))) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_rows(rows: int, cols: int, std: float, seed: int, stream: int,
                dtype: str = "bf16") -> np.ndarray:
    """rows x cols array of N(0, std^2) draws; uint16 bf16 bits or float32."""
    out = np.empty((rows, cols), np.uint16 if dtype == "bf16" else np.float32)
    nblk = (rows + _BLOCK - 1) // _BLOCK

    def work(j: int) -> None:
        r0, r1 = j * _BLOCK, min(rows, (j + 1) * _BLOCK)
        buf = _rng(seed, stream, j).standard_normal((r1 - r0, cols), dtype=np.float32)
        if std != 1.0:
            buf *= np.float32(std)
        out[r0:r1] = bf16_bits(buf) if dtype == "bf16" else buf

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(work, range(nblk)))
    return out


def _first_k_distinct(cand: np.ndarray, K: int):
    """For each row of cand, the first K distinct values in draw order.

    Returns (ok_mask, picked) where picked has K columns for rows with ok_mask True."""
    order = np.argsort(cand, axis=1, kind="stable")
    srt = np.take_along_axis(cand, order, axis=1)
    dup_sorted = np.zeros(srt.shape, bool)
    dup_sorted[:, 1:] = srt[:, 1:] == srt[:, :-1]
    dup = np.empty_like(dup_sorted)
    np.put_along_axis(dup, order, dup_sorted, axis=1)
    keep = ~dup
    cnt = np.cumsum(keep, axis=1)
    ok = cnt[:, -1] >= K
    sel = keep & (cnt <= K) & ok[:, None]
    picked = cand[sel].reshape(-1, K)
    return ok, picked


def _distinct_rows(n: int, K: int, V: int, rng: np.random.Generator, draw) -> np.ndarray:
    """n rows of K distinct ids; each row is the first K distinct values of an iid sequence
    from draw(rng, shape). Sequences of rows that fall short are extended, not redrawn."""
    if K > V:
        raise ValueError("K > V")
    m = max(2 * K, 32)
    seqs = draw(rng, (n, m))
    out = np.empty((n, K), np.int32)
    todo = np.arange(n)
    while True:
        ok, picked = _first_k_distinct(seqs, K)
        out[todo[ok]] = picked
        if ok.all():
            return out
        todo = todo[~ok]
        seqs = seqs[~ok]
        seqs = np.concatenate([seqs, draw(rng, (len(todo), seqs.shape[1]))], axis=1)


def uniform_distinct(n: int, K: int, V: int, rng: np.random.Generator) -> np.ndarray:
    return _distinct_rows(n, K, V, rng, lambda g, s: g.integers(0, V, size=s, dtype=np.int64))


_ZIPF_CDF: dict = {}


def _zipf_cdf(V: int, a: float) -> np.ndarray:
    key = (V, a)
    if key not in _ZIPF_CDF:
        w = np.arange(1, V + 1, dtype=np.float64) ** (-a)
        c = np.cumsum(w)
        _ZIPF_CDF[key] = c / c[-1]
    return _ZIPF_CDF[key]


def zipf_distinct(n: int, K: int, V: int, rng: np.random.Generator, a: float = 1.1) -> np.ndarray:
    cdf = _zipf_cdf(V, a)

    def draw(g, s):
        r = np.searchsorted(cdf, g.random(s), side="right")  # rank - 1
        return np.minimum(r, V - 1).astype(np.int64)

    return _distinct_rows(n, K, V, rng, draw)


def peaked_logits(n: int, K: int, T: float, rng: np.random.Generator) -> np.ndarray:
    """Sorted descending; top entry set so that it carries probability 0.6 at temperature T."""
    r = -np.sort(-rng.standard_normal((n, K - 1)), axis=1) if K > 1 else np.zeros((n, 0))
    t1 = T * np.log(1.5 * np.exp(r / T).sum(axis=1)) if K > 1 else np.zeros(n)
    return np.concatenate([t1[:, None], r], axis=1)


def flat_logits(n: int, K: int, var: float, rng: np.random.Generator) -> np.ndarray:
    return -np.sort(-(np.sqrt(var) * rng.standard_normal((n, K))), axis=1)


def full_teacher_logits(kind: str, n: int, V: int, seed: int) -> np.ndarray:
    """Full-vocabulary teacher logits (float32) for the top-K truncation study.
    peaked: 6*N(0,1) logits with the largest raised so that it carries probability 0.6 (T = 1);
            the next hundred tokens then hold almost all of the remaining mass;
    flat:   0.5*N(0,1) logits, spread almost evenly over the vocabulary."""
    g = np.random.default_rng([seed, 11, 0 if kind == "peaked" else 1])
    x = g.standard_normal((n, V))
    if kind == "peaked":
        x *= 6.0
        top = np.argmax(x, axis=1)
        rows = np.arange(n)
        rest = x.copy()
        rest[rows, top] = -np.inf
        mx = rest.max(axis=1)
        x[rows, top] = mx + np.log(1.5 * np.exp(rest - mx[:, None]).sum(axis=1))
    elif kind == "flat":
        x *= 0.5
    else:
        raise ValueError(kind)
    return x.astype(np.float32)


@dataclass
class Problem:
    """One synthetic workload. Arrays are in their storage dtype:
    fp32 configs hold float32, bf16 configs hold uint16 bf16 bit patterns."""

    name: str
    N: int
    d: int
    V: int
    K: int
    T: float
    chunk: int
    dtype: str
    H: np.ndarray
    W: np.ndarray
    idx: np.ndarray
    tlog: np.ndarray
    peaked: np.ndarray
    extra: dict = field(default_factory=dict)

    def f32(self, which: str) -> np.ndarray:
        a = getattr(self, which)
        return bf16_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, np.float32)

    def f64(self, which: str) -> np.ndarray:
        return self.f32(which).astype(np.float64)


def _cache_rows(cfg: dict, N: int, K: int, V: int, T: float, seed: int):
    """idx int32 [N,K], teacher logits float64 [N,K], peaked bool [N], drawn per row block."""
    idx = np.empty((N, K), np.int32)
    t = np.empty((N, K), np.float64)
    kind = np.empty(N, bool)
    nblk = (N + _BLOCK - 1) // _BLOCK
    teacher, ids = cfg["teacher"], cfg["ids"]
    var = cfg.get("teacher_var", 0.5)

    def work(j: int) -> None:
        # A block is always drawn whole and then cut, so row n does not depend on N.
        r0, r1 = j * _BLOCK, min(N, (j + 1) * _BLOCK)
        n = _BLOCK
        if teacher == "mix":
            pk = _rng(seed, _S_KIND, j).random(n) < 0.5
        else:
            pk = np.full(n, teacher == "peaked")
        kind[r0:r1] = pk[: r1 - r0]
        gi, gt = _rng(seed, _S_IDX, j), _rng(seed, _S_T, j)
        if ids == "mix":
            blk = np.empty((n, K), np.int32)
            if pk.any():
                blk[pk] = zipf_distinct(int(pk.sum()), K, V, gi)
            if (~pk).any():
                blk[~pk] = uniform_distinct(int((~pk).sum()), K, V, gi)
        elif ids == "zipf":
            blk = zipf_distinct(n, K, V, gi)
        else:
            blk = uniform_distinct(n, K, V, gi)
        idx[r0:r1] = blk[: r1 - r0]
        if teacher in ("normal", "flat"):
            tb = flat_logits(n, K, var, gt)
        elif teacher == "peaked":
            tb = peaked_logits(n, K, T, gt)
        else:
            tb = np.empty((n, K))
            if pk.any():
                tb[pk] = peaked_logits(int(pk.sum()), K, T, gt)
            if (~pk).any():
                tb[~pk] = flat_logits(int((~pk).sum()), K, var, gt)
        t[r0:r1] = tb[: r1 - r0]

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(work, range(nblk)))
    return idx, t, kind


def make(name: str, N: int | None = None, seed: int | None = None, **over) -> Problem:
    """Build a config by name. N overrides the row count (rows are a prefix of the full
    config's rows); other keys (d, V, K, T, chunk, dtype, ...) override the recipe."""
    if name not in CONFIGS:
        raise KeyError(f"unknown config {name!r}; known: {sorted(CONFIGS)}")
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    if seed is None:
        seed = cfg["seed"]
    N = cfg["B"] * cfg["S"] if N is None else int(N)
    d, V, K, T = cfg["d"], cfg["V"], cfg["K"], float(cfg["T"])
    dt = cfg["dtype"]
    H = normal_rows(N, d, 1.0, seed, _S_H, dt)
    W = normal_rows(V, d, 1.0 / np.sqrt(d), seed, _S_W, dt)
    idx, t64, kind = _cache_rows(cfg, N, K, V, T, seed)
    t32 = t64.astype(np.float32)
    tlog = bf16_bits(t32) if dt == "bf16" else t32
    return Problem(name=name, N=N, d=d, V=V, K=K, T=T, chunk=int(cfg["chunk"]), dtype=dt,
                   H=H, W=W, idx=idx, tlog=tlog, peaked=kind,
                   extra={k: v for k, v in cfg.items() if k not in ("B", "S", "d", "V", "K", "T", "chunk", "dtype")})


def sample_rows(N: int, n: int, seed: int) -> np.ndarray:
    """n distinct row ids in [0, N), sorted, from a seeded stream (used to pick checked rows)."""
    g = np.random.Generator(np.random.PCG64([int(seed), 7]))
    return np.sort(g.choice(N, size=min(n, N), replace=False)).astype(np.int64)


def sample_vocab(V: int, n: int, seed: int) -> np.ndarray:
    """n distinct vocab ids: the hot ids 0..3 and V-1 (masked tail) plus seeded others."""
    forced = np.array(sorted({0, 1, 2, 3, V - 1} & set(range(V))), np.int64)
    g = np.random.Generator(np.random.PCG64([int(seed), 8]))
    rest = np.setdiff1d(np.arange(V), forced)
    extra = g.choice(rest, size=max(0, min(n, V) - len(forced)), replace=False)
    return np.sort(np.concatenate([forced, extra])).astype(np.int64)
