"""Pins for the fp64 oracle (CPU only).

None of these re-derives the oracle's own formula. Each checks the oracle against
something independent of it:

* a literal brute force (pure-Python loops, no log-sum-exp shift, full-vocabulary
  teacher distribution, math.fsum);
* central finite differences of the loss;
* torch autograd;
* torch's cross_entropy and kl_div special cases;
* closed forms;
* invariants that hold for any correct implementation.

Together they catch a dropped term, a wrong sign or index, a transposed operand and a
missing temperature factor.
"""

import math

import numpy as np
import pytest
import torch

import oracle


def rand_problem(N, d, V, K, seed, scale=1.0, tscale=1.5):
    g = np.random.default_rng(seed)
    H = g.standard_normal((N, d)) * scale
    W = g.standard_normal((V, d)) / math.sqrt(d)
    idx = np.stack([g.choice(V, K, replace=False) for _ in range(N)]).astype(np.int32)
    t = g.standard_normal((N, K)) * tscale
    return H, W, idx, t


# ---------------------------------------------------------------- brute force

def brute(H, W, idx, t, T, n_norm, g):
    """Literal definition with Python floats: full-vocabulary teacher distribution p,
    student q_v = exp(u_v) / sum_w exp(u_w) without any shift, KL = sum_v p_v log(p_v/q_v)."""
    N, d = len(H), len(H[0])
    V = len(W)
    K = len(idx[0])
    loss_terms, row_kl, lse_out, zk_out = [], [], [], []
    G = [[0.0] * V for _ in range(N)]
    for n in range(N):
        z = [math.fsum(H[n][j] * W[v][j] for j in range(d)) for v in range(V)]
        e = [math.exp(z[v] / T) for v in range(V)]
        Z = math.fsum(e)
        q = [ev / Z for ev in e]
        et = [math.exp(t[n][k] / T) for k in range(K)]
        Zt = math.fsum(et)
        p = [0.0] * V
        for k in range(K):
            p[idx[n][k]] = et[k] / Zt
        kl = math.fsum(p[v] * math.log(p[v] / q[v]) for v in range(V) if p[v] > 0)
        row_kl.append(kl)
        lse_out.append(math.log(Z))
        zk_out.append([z[idx[n][k]] for k in range(K)])
        for v in range(V):
            G[n][v] = g * T / n_norm * (q[v] - p[v])
    loss = g * T * T / n_norm * math.fsum(row_kl)
    dH = [[math.fsum(G[n][v] * W[v][j] for v in range(V)) for j in range(d)] for n in range(N)]
    dW = [[math.fsum(G[n][v] * H[n][j] for n in range(N)) for j in range(d)] for v in range(V)]
    return dict(loss=loss, row_kl=np.array(row_kl), lse=np.array(lse_out), zk=np.array(zk_out),
                dH=np.array(dH), dW=np.array(dW))


@pytest.mark.parametrize("N,d,V,K,T,g,seed", [
    (3, 4, 7, 3, 1.0, 1.0, 0),
    (4, 5, 9, 4, 2.0, 0.7, 1),
    (2, 3, 5, 1, 0.5, -1.3, 2),
    (4, 5, 9, 2, 1.7, 1.0, 3),
])
def test_brute_force(N, d, V, K, T, g, seed):
    H, W, idx, t = rand_problem(N, d, V, K, seed)
    ref = brute(H.tolist(), W.tolist(), idx.tolist(), t.tolist(), T, N, g)
    for fn in (lambda: oracle.kl_dense(H, W, idx, t, T, g=g),
               lambda: oracle.kl_chunked(H, W, idx, t, T, chunk=2, g=g),
               lambda: oracle.kl_fused(H, W, idx, t, T, chunk=3, vtile=4, g=g)):
        out = fn()
        assert abs(out["loss"] - ref["loss"]) <= 1e-13 * max(1.0, abs(ref["loss"]))
        for key in ("row_kl", "lse", "zk", "dH", "dW"):
            np.testing.assert_allclose(out[key], ref[key], rtol=1e-12, atol=1e-13, err_msg=key)
    rk = oracle.kl_rows(H, W, idx, t, T, rows=[N - 1, 0], n_norm=N, g=g)
    np.testing.assert_allclose(rk["dH"], ref["dH"][[N - 1, 0]], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(rk["row_kl"], ref["row_kl"][[N - 1, 0]], rtol=1e-12, atol=1e-14)
    # the per-row lse of a whole batch (any row block) and the vocab rows of dW from it
    for block in (1, 3, N):
        np.testing.assert_allclose(oracle.lse_all_rows(H, W, T, block=block), ref["lse"], rtol=1e-12, atol=1e-13)
        every = oracle.kl_rows_all(H, W, idx, t, T, block=block)
        np.testing.assert_allclose(every["lse"], ref["lse"], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(every["row_kl"], ref["row_kl"], rtol=1e-12, atol=1e-14)
    vocab = [V - 1, 0, 2] + sorted({int(i) for i in idx[0]})[:2]
    vocab = sorted(set(vocab))
    dw = oracle.dw_rows(H, W, idx, t, T, vocab, ref["lse"], n_norm=N, g=g)
    np.testing.assert_allclose(dw, ref["dW"][vocab], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("T", [1.0, 1.9])
def test_brute_force_masked_teacher_entries(T):
    """Cached teacher logits of -inf (masked entries, one or all but one per row): such an
    entry has p_t = 0 and adds nothing to the KL (the brute force's full-vocabulary sum skips
    p = 0), and the gradient does not subtract at it. Every formulation must stay finite and
    match the brute force."""
    N, d, V, K = 4, 5, 9, 4
    H, W, idx, t = rand_problem(N, d, V, K, 7)
    t[0, 1] = -np.inf
    t[1, [0, 2, 3]] = -np.inf        # one finite entry left
    t[3, 3] = -np.inf
    ref = brute(H.tolist(), W.tolist(), idx.tolist(), t.tolist(), T, N, 1.3)
    assert np.all(np.isfinite(ref["row_kl"]))
    outs = [oracle.kl_dense(H, W, idx, t, T, g=1.3),
            oracle.kl_chunked(H, W, idx, t, T, chunk=3, g=1.3),
            oracle.kl_fused(H, W, idx, t, T, chunk=2, vtile=4, g=1.3)]
    for out in outs:
        assert abs(out["loss"] - ref["loss"]) <= 1e-13 * max(1.0, abs(ref["loss"]))
        for key in ("row_kl", "lse", "dH", "dW"):
            np.testing.assert_allclose(out[key], ref[key], rtol=1e-12, atol=1e-13, err_msg=key)
    rk = oracle.kl_rows(H, W, idx, t, T, rows=[1, 0, 3], n_norm=N, g=1.3)
    np.testing.assert_allclose(rk["row_kl"], ref["row_kl"][[1, 0, 3]], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(rk["dH"], ref["dH"][[1, 0, 3]], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(oracle.kl_rows_all(H, W, idx, t, T, block=3)["row_kl"], ref["row_kl"],
                               rtol=1e-12, atol=1e-14)
    row_kl, lse, zk = oracle.kl_from_logits(H @ W.T, idx, t, T)
    np.testing.assert_allclose(row_kl, ref["row_kl"], rtol=1e-12, atol=1e-14)
    # a row whose only finite entry is id k: KL_n = -log p_s(k) = lse - z_k/T
    np.testing.assert_allclose(ref["row_kl"][1], ref["lse"][1] - ref["zk"][1][1] / T, rtol=1e-12)


@pytest.mark.parametrize("T", [1.0, 0.6, 2.5])
def test_kl_from_logits_matches_dense(T):
    """kl_from_logits on the logits z = H W^T gives the dense formulation's per-row KL, lse and
    gathered logits: a dropped teacher weight, a missing temperature or a wrong sign in it
    would break the equality on these non-degenerate rows."""
    N, d, V, K = 9, 6, 37, 5
    H, W, idx, t = rand_problem(N, d, V, K, 130, scale=1.5, tscale=2.0)
    ref = oracle.kl_dense(H, W, idx, t, T)
    row_kl, lse, zk = oracle.kl_from_logits(H @ W.T, idx, t, T)
    np.testing.assert_allclose(row_kl, ref["row_kl"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, ref["lse"], rtol=1e-13)
    np.testing.assert_allclose(zk, ref["zk"], rtol=1e-13, atol=1e-15)
    assert np.all(row_kl > 1e-3)  # far from the exact-zero case


# ---------------------------------------------------------- finite differences

@pytest.mark.parametrize("T", [1.0, 2.0])
def test_finite_differences(T):
    N, d, V, K = 6, 8, 23, 5
    H, W, idx, t = rand_problem(N, d, V, K, 10)
    g = 0.9
    out = oracle.kl_dense(H, W, idx, t, T, g=g)
    rng = np.random.default_rng(11)
    h = 1e-6

    def loss(Hx, Wx):
        return oracle.kl_dense(Hx, Wx, idx, t, T, g=g)["loss"]

    for _ in range(20):
        i, j = rng.integers(N), rng.integers(d)
        Hp, Hm = H.copy(), H.copy()
        Hp[i, j] += h
        Hm[i, j] -= h
        fd = (loss(Hp, W) - loss(Hm, W)) / (2 * h)
        assert abs(fd - out["dH"][i, j]) <= 1e-7 * max(1e-3, abs(out["dH"][i, j])) + 1e-9
        v, j = rng.integers(V), rng.integers(d)
        Wp, Wm = W.copy(), W.copy()
        Wp[v, j] += h
        Wm[v, j] -= h
        fd = (loss(H, Wp) - loss(H, Wm)) / (2 * h)
        assert abs(fd - out["dW"][v, j]) <= 1e-7 * max(1e-3, abs(out["dW"][v, j])) + 1e-9


# ------------------------------------------------------------- torch autograd

@pytest.mark.parametrize("T", [1.0, 2.5])
def test_autograd_general_k(T):
    """torch differentiates the KL term; its gradients must equal the closed form."""
    N, d, V, K = 7, 6, 31, 4
    H, W, idx, t = rand_problem(N, d, V, K, 20)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    logq = torch.log_softmax(Ht @ Wt.T / T, dim=1)
    logp = torch.log_softmax(torch.tensor(t) / T, dim=1)
    it = torch.tensor(idx, dtype=torch.long)
    kl = (logp.exp() * (logp - logq.gather(1, it))).sum(1)
    loss = T * T * kl.mean()
    loss.backward()
    out = oracle.kl_fused(H, W, idx, t, T, chunk=3, vtile=7)
    assert abs(out["loss"] - loss.item()) <= 1e-12
    np.testing.assert_allclose(out["dH"], Ht.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(out["dW"], Wt.grad.numpy(), rtol=1e-10, atol=1e-13)


# ------------------------------------------------------------ library special cases

@pytest.mark.parametrize("T", [1.0, 3.0])
def test_k1_is_cross_entropy(T):
    """With one cached entry the teacher is one-hot and the loss is T^2 * cross entropy."""
    N, d, V = 9, 5, 17
    H, W, idx, t = rand_problem(N, d, V, 1, 30)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    ce = torch.nn.functional.cross_entropy(Ht @ Wt.T / T, torch.tensor(idx[:, 0], dtype=torch.long))
    (T * T * ce).backward()
    out = oracle.kl_dense(H, W, idx, t, T)
    assert abs(out["loss"] - T * T * ce.item()) <= 1e-12
    np.testing.assert_allclose(out["dH"], Ht.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(out["dW"], Wt.grad.numpy(), rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("T", [1.0, 2.0])
def test_k_equals_v_is_kl_div(T):
    """With every token cached the teacher is a full softmax and torch's kl_div applies."""
    N, d, V = 5, 4, 11
    g = np.random.default_rng(40)
    H = g.standard_normal((N, d))
    W = g.standard_normal((V, d))
    idx = np.stack([g.permutation(V) for _ in range(N)]).astype(np.int32)
    t = g.standard_normal((N, V)) * 2
    full_t = np.empty((N, V))
    np.put_along_axis(full_t, idx.astype(np.int64), t, axis=1)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    kd = torch.nn.functional.kl_div(torch.log_softmax(Ht @ Wt.T / T, 1),
                                    torch.softmax(torch.tensor(full_t) / T, 1), reduction="batchmean")
    (T * T * kd).backward()
    out = oracle.kl_fused(H, W, idx, t, T, chunk=2, vtile=3)
    assert abs(out["loss"] - T * T * kd.item()) <= 1e-12
    np.testing.assert_allclose(out["dH"], Ht.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(out["dW"], Wt.grad.numpy(), rtol=1e-10, atol=1e-13)


# ---------------------------------------------------------------- closed forms

def test_uniform_student_closed_form():
    """W = 0 makes the student uniform: KL_n = log V + sum_k p_t log p_t; a flat teacher
    then gives log(V/K)."""
    N, d, V, K = 6, 4, 50, 7
    H, W, idx, t = rand_problem(N, d, V, K, 50)
    W0 = np.zeros_like(W)
    out = oracle.kl_dense(H, W0, idx, t, 1.3)
    a = t / 1.3
    p = np.exp(a) / np.exp(a).sum(1, keepdims=True)
    np.testing.assert_allclose(out["row_kl"], math.log(V) + (p * np.log(p)).sum(1), rtol=1e-13)
    flat = oracle.kl_fused(H, W0, idx, np.full_like(t, 0.25), 1.0, chunk=4, vtile=9)
    np.testing.assert_allclose(flat["row_kl"], math.log(V / K), rtol=1e-13)


def test_zero_when_student_equals_teacher():
    """Student logits equal to the cached logits at idx and -inf elsewhere give KL = 0."""
    N, V, K = 8, 40, 6
    g = np.random.default_rng(60)
    idx = np.stack([g.choice(V, K, replace=False) for _ in range(N)]).astype(np.int32)
    for T in (1.0, 0.7, 2.0):
        t = g.standard_normal((N, K)) * 3
        z = np.full((N, V), -np.inf)
        np.put_along_axis(z, idx.astype(np.int64), t, axis=1)
        row_kl, lse, zk = oracle.kl_from_logits(z, idx, t, T)
        assert np.all(np.abs(row_kl) <= 1e-15)
        np.testing.assert_array_equal(zk, t)


def test_gibbs_inequality():
    for seed in range(5):
        H, W, idx, t = rand_problem(16, 8, 60, 9, 70 + seed, scale=2.0, tscale=3.0)
        out = oracle.kl_dense(H, W, idx, t, 1.0)
        assert np.all(out["row_kl"] >= 0)


# --------------------------------------------------------- formulation equality

@pytest.mark.parametrize("chunk", [1, 7, 19])
@pytest.mark.parametrize("vtile", [1, 13, 41])
def test_formulations_agree(chunk, vtile):
    """Dense, forward-chunked and fused chunked give the same numbers."""
    N, d, V, K = 19, 6, 41, 5
    H, W, idx, t = rand_problem(N, d, V, K, 80)
    T, gg = 1.6, 0.8
    a = oracle.kl_dense(H, W, idx, t, T, g=gg)
    b = oracle.kl_chunked(H, W, idx, t, T, chunk=chunk, g=gg)
    c = oracle.kl_fused(H, W, idx, t, T, chunk=chunk, vtile=vtile, g=gg)
    for o in (b, c):
        assert abs(o["loss"] - a["loss"]) <= 1e-12 * abs(a["loss"])
        for key in ("lse", "row_kl", "zk", "dH", "dW"):
            np.testing.assert_allclose(o[key], a[key], rtol=1e-12, atol=1e-14, err_msg=key)


# ------------------------------------------------------------------ invariants

def test_shift_invariance():
    """Every row of G sums to zero: sum_v dW[v,:] = 0, and adding the same vector to every
    row of W leaves the loss and dH unchanged."""
    N, d, V, K = 12, 7, 33, 6
    H, W, idx, t = rand_problem(N, d, V, K, 90)
    a = oracle.kl_dense(H, W, idx, t, 1.4)
    np.testing.assert_allclose(a["dW"].sum(axis=0), 0.0, atol=1e-14)
    c = np.random.default_rng(91).standard_normal(d)
    b = oracle.kl_fused(H, W + c[None, :], idx, t, 1.4, chunk=5, vtile=8)
    assert abs(a["loss"] - b["loss"]) <= 1e-12 * a["loss"]
    np.testing.assert_allclose(a["dH"], b["dH"], rtol=1e-10, atol=1e-14)


def test_linear_in_upstream_gradient():
    N, d, V, K = 5, 4, 21, 3
    H, W, idx, t = rand_problem(N, d, V, K, 100)
    a = oracle.kl_dense(H, W, idx, t, 1.0, g=1.0)
    b = oracle.kl_dense(H, W, idx, t, 1.0, g=-2.5)
    np.testing.assert_allclose(b["dH"], -2.5 * a["dH"], rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(b["dW"], -2.5 * a["dW"], rtol=1e-14, atol=1e-16)
    c = oracle.kl_dense(H, W, idx, t, 1.0, n_norm=2 * N)
    np.testing.assert_allclose(c["dW"], 0.5 * a["dW"], rtol=1e-14, atol=1e-16)
    assert abs(c["loss"] - 0.5 * a["loss"]) <= 1e-15


def test_dw_rows_equals_dense_dw():
    """dW restricted to chosen vocabulary rows, from the batch's lse, equals those rows of the
    dense formulation's dW: all rows, cached and uncached ids, n_norm != N and g != 1."""
    N, d, V, K = 40, 9, 57, 6
    H, W, idx, t = rand_problem(N, d, V, K, 120)
    a = oracle.kl_dense(H, W, idx, t, 1.7, n_norm=100.0, g=-0.6)
    lse = oracle.lse_all_rows(H, W, 1.7, block=7)
    np.testing.assert_allclose(lse, a["lse"], rtol=1e-13, atol=1e-14)
    full = oracle.dw_rows(H, W, idx, t, 1.7, np.arange(V), lse, n_norm=100.0, g=-0.6)
    np.testing.assert_allclose(full, a["dW"], rtol=1e-11, atol=1e-15)
    some = np.array([0, 5, int(idx[3, 2]), V - 1])
    np.testing.assert_allclose(oracle.dw_rows(H, W, idx, t, 1.7, some, lse, n_norm=100.0, g=-0.6), a["dW"][some],
                               rtol=1e-11, atol=1e-15)


def test_rejects_bad_ids():
    H, W, idx, t = rand_problem(3, 4, 10, 3, 110)
    bad = idx.copy()
    bad[1, 2] = bad[1, 0]
    with pytest.raises(ValueError):
        oracle.kl_dense(H, W, bad, t, 1.0)
    bad = idx.copy()
    bad[0, 0] = 10
    with pytest.raises(ValueError):
        oracle.kl_fused(H, W, bad, t, 1.0, chunk=2, vtile=3)


def _rank_key(x, v):
    """Explicit order of the cache: larger values first, NaN below every number (even -inf),
    equal values (NaN among NaN, -0 with +0) by the lower id."""
    return (1, 0.0, v) if math.isnan(x) else (0, -x, v)


def test_topk_cache_matches_sort():
    """The cache producer's oracle against a plain per-row sort, ties by lower id."""
    g = np.random.default_rng(120)
    x = np.round(g.standard_normal((6, 50)) * 2) / 2  # many ties
    idx, vals = oracle.topk_cache(x, 7)
    for n in range(6):
        pairs = sorted(range(50), key=lambda v: (-x[n, v], v))[:7]
        assert list(idx[n]) == pairs
        np.testing.assert_array_equal(vals[n], x[n, pairs])


@pytest.mark.parametrize("K", [1, 5, 12, 30])
def test_topk_cache_nan_and_signed_values(K):
    """Rows with NaN: scattered, all NaN, next to +-inf, fewer than K numbers; and -0 beside +0.
    The oracle must rank NaN last with ties by id, and treat -0 as equal to +0."""
    g = np.random.default_rng(121)
    V = 30
    rows = []
    r = np.round(g.standard_normal(V) * 2) / 2
    r[[3, 11, 17]] = np.nan                                    # scattered NaN
    rows.append(r)
    rows.append(np.full(V, np.nan))                            # every entry NaN
    r = g.standard_normal(V)
    r[[0, 1, 2, 5]] = [np.nan, np.inf, -np.inf, np.nan]        # NaN next to +-inf
    r[[6, 7]] = [np.inf, -np.inf]
    rows.append(r)
    r = np.full(V, np.nan)
    r[[4, 9, 21]] = [1.5, -np.inf, 1.5]                        # three numbers, the rest NaN
    rows.append(r)
    r = np.zeros(V)
    r[::2] = -0.0                                              # signed zeros only
    r[[8, 13]] = [np.nan, -1.0]
    rows.append(r)
    x = np.stack(rows)
    idx, vals = oracle.topk_cache(x, K)
    for n in range(len(rows)):
        want = sorted(range(V), key=lambda v: _rank_key(x[n, v], v))[:K]
        assert list(idx[n]) == want, (n, list(idx[n]), want)
        np.testing.assert_array_equal(vals[n], x[n, want])  # NaN == NaN in this comparison



# --------------------------------------------------------------- top-K truncation study

def _brute_truncation(H, W, teacher, K, T):
    """Loops and math.fsum over one tiny row at a time, from the definitions."""
    out = []
    N, V = teacher.shape
    for n in range(N):
        z = [math.fsum(H[n, j] * W[v, j] for j in range(H.shape[1])) / T for v in range(V)]
        a = [teacher[n, v] / T for v in range(V)]
        zs, za = math.fsum(math.exp(x) for x in z), math.fsum(math.exp(x) for x in a)
        ps = [math.exp(x) / zs for x in z]
        pt = [math.exp(x) / za for x in a]
        top = sorted(range(V), key=lambda v: (-teacher[n, v], v))[:K]
        m = math.fsum(pt[v] for v in top)
        pk = [pt[v] / m if v in top else 0.0 for v in range(V)]
        kl_full = math.fsum(pt[v] * math.log(pt[v] / ps[v]) for v in range(V))
        kl_topk = math.fsum(pk[v] * math.log(pk[v] / ps[v]) for v in top)
        num = math.sqrt(math.fsum((pk[v] - pt[v]) ** 2 for v in range(V)))
        den = math.sqrt(math.fsum((ps[v] - pt[v]) ** 2 for v in range(V)))
        out.append((m, kl_full, kl_topk, num / den))
    return np.array(out)


def test_truncation_terms_brute_force():
    g = np.random.default_rng(21)
    H, W = g.standard_normal((3, 4)), g.standard_normal((9, 4))
    t = g.standard_normal((3, 9)) * 2
    t[1, :4] = 0.5  # ties across the K boundary: lower ids first
    for K, T in ((1, 1.0), (3, 0.7), (5, 2.0)):
        r = oracle.truncation_terms(H, W, t, K, T)
        b = _brute_truncation(H, W, t, K, T)
        for col, name in enumerate(("mass", "kl_full", "kl_topk", "grad_rel")):
            np.testing.assert_allclose(r[name], b[:, col], rtol=1e-12, atol=1e-14, err_msg=name)


def test_truncation_terms_identities():
    g = np.random.default_rng(22)
    H, W = g.standard_normal((6, 8)), g.standard_normal((50, 8)) / 3
    t = g.standard_normal((6, 50)) * 1.5
    # K = V keeps the whole teacher: nothing changes
    r = oracle.truncation_terms(H, W, t, 50)
    np.testing.assert_allclose(r["mass"], 1.0, rtol=1e-14)
    np.testing.assert_allclose(r["kl_topk"], r["kl_full"], rtol=1e-12)
    np.testing.assert_allclose(r["grad_rel"], 0.0, atol=1e-14)
    # the cached part of KL_full: m*(KL_topk + log m) = sum over the top K of p_t log(p_t/p_s)
    K = 7
    r = oracle.truncation_terms(H, W, t, K)
    u = H @ W.T
    log_ps = u - np.log(np.exp(u).sum(1, keepdims=True))
    log_pt = t - np.log(np.exp(t).sum(1, keepdims=True))
    top = np.argsort(-t, axis=1, kind="stable")[:, :K]
    rows = np.arange(6)[:, None]
    head = (np.exp(log_pt[rows, top]) * (log_pt[rows, top] - log_ps[rows, top])).sum(1)
    np.testing.assert_allclose(r["mass"] * (r["kl_topk"] + np.log(r["mass"])), head, rtol=1e-11)
    # KL_topk is the method's loss with the top-K cache as the teacher
    idx, vals = oracle.topk_cache(t, K)
    np.testing.assert_allclose(r["kl_topk"], oracle.kl_dense(H, W, idx, vals, 1.0)["row_kl"], rtol=1e-11)
    # more cached entries never lose mass
    m = [oracle.truncation_terms(H, W, t, k)["mass"] for k in (1, 5, 20, 50)]
    assert all(np.all(a <= b + 1e-15) for a, b in zip(m, m[1:]))


@pytest.mark.parametrize("T", [0.5, 2.0])
def test_one_token_head_is_exactly_zero(T):
    """V = 1 (so K = 1): student and teacher both put all mass on the one token, so every KL_n,
    the loss and every gradient are exactly 0, in each formulation (closed form)."""
    g = np.random.default_rng(31)
    N, d = 40, 24
    H, W = g.standard_normal((N, d)), g.standard_normal((1, d))
    idx = np.zeros((N, 1), np.int64)
    t = g.standard_normal((N, 1))
    for ref in (oracle.kl_dense(H, W, idx, t, T), oracle.kl_chunked(H, W, idx, t, T, chunk=16),
                oracle.kl_fused(H, W, idx, t, T, chunk=16, vtile=1)):
        assert ref["loss"] == 0.0 and not np.any(ref["row_kl"])
        assert not np.any(ref["dH"]) and not np.any(ref["dW"])
        np.testing.assert_allclose(ref["lse"], (H @ W.T)[:, 0] / T, rtol=1e-14)


def test_fp32_dot_product_bound_holds():
    """The GPU tests' fallback bound for gathered logits, gamma_(d+1) * sum |h_i w_i| with
    u = 2^-24, bounds fp32 dot products computed from fp32 inputs in several summation orders
    (numpy's fp32 matmul, a sequential fp32 loop, pairwise sums) against the exact fp64 value."""
    from gpu_helpers import zk_dot_bound
    g = np.random.default_rng(32)
    N, d, V, K = 64, 700, 300, 8
    H = g.standard_normal((N, d)).astype(np.float32)
    W = (g.standard_normal((V, d)) / np.sqrt(d)).astype(np.float32)
    idx = np.stack([g.choice(V, K, replace=False) for _ in range(N)])
    Hd, Wd = H.astype(np.float64), W.astype(np.float64)
    exact = np.take_along_axis(Hd @ Wd.T, idx, axis=1)
    bound = zk_dot_bound(Hd, Wd, idx)
    z_mm = np.take_along_axis((H @ W.T).astype(np.float64), idx, axis=1)
    prod = H[:, None, :] * W[idx]                       # fp32 products, [N, K, d]
    z_seq = np.zeros((N, K), np.float32)
    for i in range(d):                                  # left-to-right fp32 accumulation
        z_seq = (z_seq + prod[:, :, i]).astype(np.float32)
    z_pair = prod.astype(np.float32)
    while z_pair.shape[2] > 1:                          # pairwise fp32 accumulation
        if z_pair.shape[2] % 2:
            z_pair = np.concatenate([z_pair, np.zeros_like(z_pair[:, :, :1])], axis=2)
        z_pair = (z_pair[:, :, 0::2] + z_pair[:, :, 1::2]).astype(np.float32)
    for z in (z_mm, z_seq.astype(np.float64), z_pair[:, :, 0].astype(np.float64)):
        err = np.abs(z - exact)
        assert np.all(err <= bound), float((err / bound).max())
        assert (err / bound).max() > 0.0
