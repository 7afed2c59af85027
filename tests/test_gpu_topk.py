"""The offline top-K cache producer (kd_topk_cache) against the oracle's sort, bit for bit:
ids and values, on random rows, rows full of ties, signed zeros and infinities, K at its limits,
padded rows, and rows at the gpt-oss vocabulary size."""

import os

import numpy as np
import pytest
import torch

import datagen
import oracle
import lm_head_kl_amd as kd
from gpu_helpers import say, to_torch

pytestmark = pytest.mark.gpu


def check(x: np.ndarray, K: int, dtype: str, label: str, ld: int = 0):
    """x: fp32 values (exactly representable in dtype). Compares ids and values bitwise."""
    say("topk", label, f"N={x.shape[0]} V={x.shape[1]} K={K} {dtype}")
    N, V = x.shape
    if dtype == "bf16":
        store = datagen.bf16_bits(x)
        assert np.array_equal(datagen.bf16_to_f32(store), x)
    else:
        store = x.astype(np.float32)
    if ld > V:
        pad = np.zeros((N, ld), store.dtype)
        pad[:, :V] = store
        dev = to_torch(pad)[:, :V]
    else:
        dev = to_torch(store)
    idx, vals = kd.topk_cache(dev, K)
    torch.cuda.synchronize()
    want_idx, want_val = oracle.topk_cache(x, K)
    got_idx = idx.cpu().numpy()
    assert np.array_equal(got_idx, want_idx), label
    got_val = vals.float().cpu().numpy()
    # values are copies of the selected entries
    assert np.array_equal(got_val.view(np.uint32), np.take_along_axis(x, want_idx.astype(np.int64), 1).view(np.uint32))


def bf16_values(a):
    return datagen.bf16_to_f32(datagen.bf16_bits(a.astype(np.float32)))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_random_rows(dtype):
    g = np.random.default_rng(11)
    x = g.standard_normal((64, 2048)).astype(np.float32) * 3
    if dtype == "bf16":
        x = bf16_values(x)
    check(x, 16, dtype, "random")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_ties_and_special_values(dtype):
    g = np.random.default_rng(12)
    rows = [
        g.integers(-2, 3, 1000).astype(np.float32),                      # five distinct values
        np.full(1000, 0.75, np.float32),                                  # every entry equal
        np.where(g.random(1000) < 0.5, np.float32(-0.0), np.float32(0.0)),  # signed zeros only
        np.concatenate([[np.inf, -np.inf, np.inf], g.standard_normal(997).astype(np.float32)]),
    ]
    x = np.stack(rows).astype(np.float32)
    x[2, 500] = 1.0
    if dtype == "bf16":
        x = bf16_values(x)
    for K in (1, 7, 100, 1000):
        check(x, K, dtype, f"ties/special K={K}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("V", [1000, 201088])
def test_nan_rows(dtype, V):
    """Rows with NaN: scattered, all NaN, NaN next to +-inf, fewer than K numbers, NaN of either
    sign. NaN ranks below every number (-inf included), NaN among NaN by the lower id; the
    oracle's order is pinned to that. Ids bit for bit, values as copies of the chosen entries."""
    g = np.random.default_rng(16)
    nan, nneg = np.float32(np.nan), -np.float32(np.nan)
    rows = []
    r = (g.standard_normal(V) * 3).astype(np.float32)
    r[g.choice(V, V // 10, replace=False)] = nan                    # scattered NaN
    rows.append(r)
    rows.append(np.full(V, nan, np.float32))                         # every entry NaN
    r = g.standard_normal(V).astype(np.float32)
    r[:6] = [nan, np.inf, -np.inf, nneg, np.inf, -np.inf]              # NaN next to +-inf
    r[g.choice(np.arange(6, V), 30, replace=False)] = nan
    rows.append(r)
    r = np.full(V, nneg, np.float32)
    r[g.choice(V, 40, replace=False)] = g.integers(-2, 3, 40)         # 40 numbers with ties, rest NaN
    rows.append(r)
    r = g.standard_normal(V).astype(np.float32)
    r[V // 2:] = nan                                                   # NaN tail
    rows.append(r)
    x = np.stack(rows)
    store = datagen.bf16_bits(x) if dtype == "bf16" else x
    dev = to_torch(store)
    for K in (1, 7, 100, 1000):
        say("topk NaN rows", dtype, f"V={V} K={K}")
        idx, vals = kd.topk_cache(dev, K)
        torch.cuda.synchronize()
        xv = datagen.bf16_to_f32(store) if dtype == "bf16" else x
        want_idx, _ = oracle.topk_cache(xv, K)
        assert np.array_equal(idx.cpu().numpy(), want_idx), K
        want_bits = np.take_along_axis(store, want_idx.astype(np.int64), 1)
        got = vals.cpu()
        got_bits = got.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else got.numpy()
        assert np.array_equal(got_bits.view(want_bits.dtype).view(np.uint8), want_bits.view(np.uint8)), K


def test_k_limits_and_padded_rows():
    g = np.random.default_rng(13)
    x = bf16_values(g.standard_normal((8, 3000)))
    check(x, 1024, "bf16", "K=1024")
    check(x[:, :777], 777, "bf16", "K=V")
    check(x, 100, "bf16", "padded rows", ld=3072 + 8)


@pytest.mark.parametrize("K", [100, 500])
def test_gptoss_vocabulary(K):
    """Rows at V = 201,088: Gaussian teacher logits in bf16 (many exact ties near the K-th) and
    peaked rows whose top token is far above the rest."""
    g = np.random.default_rng(14)
    x = g.standard_normal((32, 201088)).astype(np.float32) * 2.0
    x[::2, g.integers(0, 201088, 16)] += 12.0
    check(bf16_values(x), K, "bf16", "gpt-oss vocabulary")


def test_cache_feeds_the_loss():
    """The produced cache used as the teacher of the fused loss gives the oracle's loss."""
    p = datagen.make("tiny")
    g = np.random.default_rng(15)
    teacher = g.standard_normal((p.N, p.V)).astype(np.float32) * 2
    idx, vals = kd.topk_cache(to_torch(teacher), p.K)
    H, W = to_torch(p.H), to_torch(p.W)
    f = kd.fused_kl_fwd(H, W, idx, vals, T=p.T, chunk=p.chunk)
    torch.cuda.synchronize()
    ci, cv = oracle.topk_cache(teacher, p.K)
    ref = oracle.kl_dense(p.f64("H"), p.f64("W"), ci, cv, p.T)
    assert abs(f.loss.item() - ref["loss"]) <= 1e-6 * abs(ref["loss"])


def draw_rows(g: np.random.Generator, N: int, V: int, K: int) -> np.ndarray:
    """Rows of mixed kinds: scaled normals, small integers (many ties), normals with signed zeros
    and infinities planted, and rows where many entries equal the value at the cutoff."""
    x = np.empty((N, V), np.float32)
    for n in range(N):
        kind = int(g.integers(0, 4))
        if kind == 0:
            x[n] = g.standard_normal(V) * float(g.choice([1e-3, 1.0, 100.0]))
        elif kind == 1:
            r = int(g.integers(0, 11))
            x[n] = g.integers(-r, r + 1, V)
        elif kind == 2:
            x[n] = g.standard_normal(V)
            m = int(g.integers(0, min(V, 40) + 1))
            pos = g.choice(V, size=m, replace=False)
            x[n, pos] = g.choice(np.array([0.0, -0.0, np.inf, -np.inf], np.float32), size=m)
        else:
            x[n] = g.standard_normal(V)
            cut = np.sort(x[n])[::-1][min(K, V) - 1]
            m = int(g.integers(1, V + 1))
            x[n, g.choice(V, size=m, replace=False)] = cut
    return x


N_RANDOM = int(os.environ.get("KD_TOPK_CASES", "24"))  # more with KD_TOPK_CASES=<n>


@pytest.mark.parametrize("i", range(N_RANDOM))
def test_random_shapes(i):
    """Seeded random (N, V, K, row stride, dtype, row kinds); ids and values bit for bit."""
    g = np.random.Generator(np.random.PCG64([4244, i]))
    V = int(g.choice([int(g.integers(1, 300)), int(g.integers(300, 5000)), int(g.integers(5000, 70000))]))
    N = int(g.integers(1, max(2, min(300, 4_000_000 // V))))
    K = int(g.choice([1, int(g.integers(1, min(V, 1024) + 1)), min(V, 1024)]))
    ld = V + int(g.choice([0, int(g.integers(1, 64))]))
    dtype = "bf16" if i % 2 else "fp32"
    x = draw_rows(g, N, V, K)
    if dtype == "bf16":
        x = bf16_values(x)
    check(x, K, dtype, f"random shape {i}", ld=ld)


def single_read_rows(g: np.random.Generator, N: int, V: int, K: int) -> np.ndarray:
    """Rows for the single-read pass (one workgroup per CU holds a whole row on chip): the kinds
    of ``draw_rows``, peaked rows, rows of negative values only, signed zeros among the largest
    entries, and rows that pass it back to the exact kernel (every entry -inf, all equal, a few
    numbers among NaN)."""
    x = draw_rows(g, N, V, K)
    for n in range(N):
        kind = n % 9
        if kind == 4:
            x[n] = g.standard_normal(V) * 2.0
            x[n, g.integers(0, V, 8)] += 12.0
        elif kind == 5:
            x[n] = -np.abs(g.standard_normal(V)) - 1.0
        elif kind == 6:
            x[n] = -np.abs(g.standard_normal(V)) - 0.5
            pos = g.choice(V, size=2 * K + 3, replace=False)
            x[n, pos] = np.where(g.random(pos.size) < 0.5, np.float32(-0.0), np.float32(0.0))
        elif kind == 7:
            x[n] = -np.inf if n % 2 else np.float32(0.25)
        elif kind == 8 and n % 4 == 0:
            x[n] = np.nan
            x[n, g.choice(V, size=max(1, K // 2), replace=False)] = g.standard_normal(max(1, K // 2))
    return x


@pytest.mark.parametrize(
    "dtype,V,K,N,pad",
    [
        ("bf16", 201088, 100, 300, 0),   # the gpt-oss vocabulary; more rows than CUs
        ("bf16", 201088, 128, 40, 8),    # the largest K of the pass; padded rows
        ("bf16", 204800, 1, 40, 0),      # the longest row it holds
        ("bf16", 201087, 13, 40, 1),     # ragged tail
        ("bf16", 201087, 13, 40, 0),     # a row stride off 16-byte alignment: the exact kernel only
        ("bf16", 68272, 64, 520, 0),     # the shortest row it takes; two rows per CU and more
        ("fp32", 102400, 100, 40, 0),
        ("fp32", 50001, 7, 300, 3),      # ragged tail, padded rows
        ("fp32", 34136, 128, 40, 0),
    ],
)
def test_single_read_pass(dtype, V, K, N, pad):
    """kd_topk_cache at the row lengths where a whole row is held on chip and read once, with the
    rows it cannot settle redone by the exact kernel; ids and values bit for bit."""
    run_single_read(np.random.Generator(np.random.PCG64([4245, V, K])), dtype, V, K, N, pad)


# Seeded draws over the row lengths and widths the single-read pass takes (more with
# KD_TOPK_SINGLE_CASES=<n>).
N_SINGLE = int(os.environ.get("KD_TOPK_SINGLE_CASES", "6"))


@pytest.mark.parametrize("i", range(N_SINGLE))
def test_single_read_random(i):
    g = np.random.Generator(np.random.PCG64([4246, i]))
    dtype = "bf16" if i % 2 == 0 else "fp32"
    V = int(g.integers(68272, 204801)) if dtype == "bf16" else int(g.integers(34136, 102401))
    K = int(g.choice([1, int(g.integers(1, 129)), 128]))
    N = int(g.integers(1, 300))
    pad = int(g.choice([0, 0, int(g.integers(1, 16))]))
    run_single_read(g, dtype, V, K, N, pad)


def run_single_read(g: np.random.Generator, dtype: str, V: int, K: int, N: int, pad: int) -> None:
    x = single_read_rows(g, N, V, K)
    xs = datagen.bf16_bits(x) if dtype == "bf16" else x  # what the device holds
    xv = datagen.bf16_to_f32(xs) if dtype == "bf16" else x
    say("topk single read", dtype, f"N={N} V={V} K={K} ld={V + pad}")
    buf = np.zeros((N, V + pad), xs.dtype)
    buf[:, :V] = xs
    idx, vals = kd.topk_cache(to_torch(buf)[:, :V], K)
    torch.cuda.synchronize()
    want_idx, _ = oracle.topk_cache(xv, K)
    assert np.array_equal(idx.cpu().numpy(), want_idx)
    want_bits = np.take_along_axis(xs, want_idx.astype(np.int64), 1)
    got = vals.cpu()
    got_bits = got.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else got.numpy()
    assert np.array_equal(got_bits.view(np.uint8), want_bits.view(np.uint8))
