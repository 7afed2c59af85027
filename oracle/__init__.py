"""fp64 CPU oracle for the top-K distillation KL loss over the LM head.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU
baseline import this package. The GPU library and its Python binding never import,
call or link it, and it shares no code with them.

It is plain numpy in float64 on already-rounded inputs (bf16 or fp32 values upcast
exactly), written to be read against the definition rather than to be fast.

What is computed, and where the pages state it. Pages are cited by title and paragraph,
because they have no numbered sections or equations:

* The teacher side comes from an offline cache of the top-100 teacher logits per
  sequence position, stored once and reused. The tail beyond the top-K is thrown away.
  Sources: "Making knowledge distillation cheap enough to run in production", paragraphs
  "the first fix is offline distillation" and "the remaining restriction is the top-K
  approximation"; dailyai.com.br launch note, section "As duas inovações", item 1.
  So the teacher distribution is the softmax of the cached logits over the K cached
  entries, zero elsewhere.
* The loss is a Kullback-Leibler term between that teacher distribution and the
  student's full-vocabulary distribution. The student side is an equally dense
  log-probability grid over the whole vocabulary. Source: "Making knowledge distillation
  cheap enough...", paragraph on the three formulations (dense KL).
* Three formulations give the same value: dense, forward-chunked and fused chunked
  (same paragraph). The fused one projects one chunk of hidden states at a time, folds
  it into a running accumulator and recomputes the chunk in the backward pass.
  ``kl_dense``, ``kl_chunked`` and ``kl_fused`` below follow them.

The pages leave the following open. The readings taken:
(1) Direction: KL(p_t || p_s).
(2) Temperature T on both sides, with the loss scaled by T^2. Hence
    d loss / d z = g*(T/n_norm)*(P_s - P_t).
(3) Mean over all N rows, with denominator n_norm (default N).
(4) The student is normalised over all V, not over the K cached ids.
(5) Cached ids are distinct and in [0, V).
(6) A cached teacher logit may be -inf (a masked entry). Its probability is 0 and it adds
    nothing to the KL sum (0 log 0 = 0, as in the dense formulation's full-vocabulary sum).
    Every row needs at least one finite cached logit; +inf and NaN logits are outside the
    domain.

Notation: H [N,d] hidden states, W [V,d] LM-head weight, z = H W^T logits, u = z/T,
lse_n = logsumexp_v u_nv, t [N,K] cached teacher logits with ids idx [N,K],
p_t = softmax(t/T) over K, g the upstream gradient of the scalar loss.

Parity pins: every function here is checked in tests/test_oracle.py against:
* brute force (pure-Python loops with math.fsum);
* central finite differences of the loss;
* the Gibbs inequality;
* the exact-zero case;
* equality of the three formulations;
* torch's cross_entropy (K = 1) and kl_div (K = V);
* the uniform-student closed form;
* shift invariance;
* linearity in g.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "teacher_logp",
    "logsumexp_rows",
    "kl_from_logits",
    "kl_dense",
    "kl_chunked",
    "kl_fused",
    "kl_rows",
    "lse_all_rows",
    "kl_rows_all",
    "dw_rows",
    "topk_cache",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _check(idx: np.ndarray, V: int) -> None:
    idx = np.asarray(idx)
    if idx.size and (idx.min() < 0 or idx.max() >= V):
        raise ValueError("cached token id out of range")
    srt = np.sort(idx, axis=1)
    if idx.shape[1] > 1 and np.any(srt[:, 1:] == srt[:, :-1]):
        raise ValueError("cached token ids repeat within a row")


def teacher_logp(tlog, T: float) -> np.ndarray:
    """log p_t over the K cached entries: log softmax(t/T) along each row."""
    a = _f64(tlog) / T
    m = a.max(axis=1, keepdims=True)
    return a - (m + np.log(np.exp(a - m).sum(axis=1, keepdims=True)))


def _kl_terms(pt, lpt, zk, T: float, lse) -> np.ndarray:
    """Per-row sum over the cached entries of p_t (log p_t - (z_k/T - lse)), where entries
    with p_t = 0 (teacher logit -inf) add nothing: the 0 log 0 = 0 convention of the
    full-vocabulary KL sum."""
    with np.errstate(invalid="ignore"):
        t = pt * (lpt - (zk / T - np.asarray(lse)[:, None]))
    return np.where(pt > 0, t, 0.0).sum(axis=1)


def logsumexp_rows(u) -> np.ndarray:
    """lse_n = log sum_v exp(u_nv), shifted by the row max for range."""
    u = _f64(u)
    m = u.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return (m + np.log(np.exp(u - m).sum(axis=1, keepdims=True)))[:, 0]


def kl_from_logits(z, idx, tlog, T: float):
    """Per-row KL(p_t || softmax(z/T)) from given student logits z [N,V] (may hold -inf).

    Returns (row_kl [N], lse [N], zk [N,K])."""
    z = _f64(z)
    u = z / T
    lse = logsumexp_rows(u)
    zk = np.take_along_axis(z, np.asarray(idx, np.int64), axis=1)
    lpt = teacher_logp(tlog, T)
    pt = np.exp(lpt)
    row_kl = _kl_terms(pt, lpt, zk, T, lse)
    return row_kl, lse, zk


def _scale(N: int, n_norm, g: float, T: float):
    n = float(N if (n_norm is None or n_norm <= 0) else n_norm)
    return g * T * T / n, g * T / n  # loss scale, gradient scale


def kl_dense(H, W, idx, tlog, T: float, n_norm=None, g: float = 1.0) -> dict:
    """Dense formulation: expand the cached teacher into a full N x V probability grid and
    compare it with the full student log-probability grid (two N x V grids at once).

    Returns loss, lse, row_kl, zk, dH, dW (all float64)."""
    H, W = _f64(H), _f64(W)
    idx = np.asarray(idx, np.int64)
    N, V = H.shape[0], W.shape[0]
    _check(idx, V)
    z = H @ W.T
    u = z / T
    lse = logsumexp_rows(u)
    log_ps = u - lse[:, None]
    pt_grid = np.zeros((N, V))
    np.put_along_axis(pt_grid, idx, np.exp(teacher_logp(tlog, T)), axis=1)
    pos = pt_grid > 0
    terms = np.zeros((N, V))
    terms[pos] = pt_grid[pos] * (np.log(pt_grid[pos]) - log_ps[pos])  # 0 log 0 = 0
    row_kl = terms.sum(axis=1)
    ls, gs = _scale(N, n_norm, g, T)
    G = gs * (np.exp(log_ps) - pt_grid)
    return dict(loss=ls * row_kl.sum(), lse=lse, row_kl=row_kl,
                zk=np.take_along_axis(z, idx, axis=1), dH=G @ W, dW=G.T @ H)


def kl_chunked(H, W, idx, tlog, T: float, chunk: int, n_norm=None, g: float = 1.0) -> dict:
    """Forward-chunked formulation: the teacher stays sparse (K entries per row) and the loss
    is computed one slice of rows at a time; each slice's student logits are kept for its
    backward."""
    H, W = _f64(H), _f64(W)
    idx = np.asarray(idx, np.int64)
    N, V = H.shape[0], W.shape[0]
    _check(idx, V)
    lpt = teacher_logp(tlog, T)
    pt = np.exp(lpt)
    ls, gs = _scale(N, n_norm, g, T)
    lse = np.empty(N)
    row_kl = np.empty(N)
    zk = np.empty(idx.shape)
    dH = np.empty_like(H)
    dW = np.zeros_like(W)
    kept = []
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        z = H[r0:r1] @ W.T
        kept.append(z)
        lse[r0:r1] = logsumexp_rows(z / T)
        zk[r0:r1] = np.take_along_axis(z, idx[r0:r1], axis=1)
        row_kl[r0:r1] = _kl_terms(pt[r0:r1], lpt[r0:r1], zk[r0:r1], T, lse[r0:r1])
    for c, r0 in enumerate(range(0, N, chunk)):
        r1 = min(N, r0 + chunk)
        z = kept[c]
        G = np.exp(z / T - lse[r0:r1, None])
        rows = np.arange(r1 - r0)[:, None]
        G[rows, idx[r0:r1]] -= pt[r0:r1]
        G *= gs
        dH[r0:r1] = G @ W
        dW += G.T @ H[r0:r1]
    return dict(loss=ls * row_kl.sum(), lse=lse, row_kl=row_kl, zk=zk, dH=dH, dW=dW)


def kl_fused(H, W, idx, tlog, T: float, chunk: int, vtile: int, n_norm=None,
             g: float = 1.0) -> dict:
    """Fused chunked formulation: for each chunk of rows, project one vocab tile at a time,
    fold it into a running (max, sum) per row and pick out the logits at the cached ids;
    the tile is then discarded. The backward pass recomputes every tile of the chunk and
    accumulates dH for the chunk and dW for the tile."""
    H, W = _f64(H), _f64(W)
    idx = np.asarray(idx, np.int64)
    N, V = H.shape[0], W.shape[0]
    _check(idx, V)
    lpt = teacher_logp(tlog, T)
    pt = np.exp(lpt)
    ls, gs = _scale(N, n_norm, g, T)
    lse = np.empty(N)
    row_kl = np.empty(N)
    zk = np.full(idx.shape, np.nan)
    dH = np.zeros_like(H)
    dW = np.zeros_like(W)
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        Hc, ic = H[r0:r1], idx[r0:r1]
        m = np.full(r1 - r0, -np.inf)
        s = np.zeros(r1 - r0)
        for v0 in range(0, V, vtile):
            v1 = min(V, v0 + vtile)
            z = Hc @ W[v0:v1].T
            u = z / T
            m_new = np.maximum(m, u.max(axis=1))
            s = s * np.exp(m - m_new) + np.exp(u - m_new[:, None]).sum(axis=1)
            m = m_new
            hit = (ic >= v0) & (ic < v1)
            rr, kk = np.nonzero(hit)
            zk[r0 + rr, kk] = z[rr, ic[rr, kk] - v0]
        lse[r0:r1] = m + np.log(s)
        row_kl[r0:r1] = _kl_terms(pt[r0:r1], lpt[r0:r1], zk[r0:r1], T, lse[r0:r1])
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        Hc, ic = H[r0:r1], idx[r0:r1]
        for v0 in range(0, V, vtile):
            v1 = min(V, v0 + vtile)
            z = Hc @ W[v0:v1].T  # recomputed, never stored across the two passes
            G = np.exp(z / T - lse[r0:r1, None])
            hit = (ic >= v0) & (ic < v1)
            rr, kk = np.nonzero(hit)
            G[rr, ic[rr, kk] - v0] -= pt[r0 + rr, kk]
            G *= gs
            dH[r0:r1] += G @ W[v0:v1]
            dW[v0:v1] += G.T @ Hc
    return dict(loss=ls * row_kl.sum(), lse=lse, row_kl=row_kl, zk=zk, dH=dH, dW=dW)


def kl_rows(H, W, idx, tlog, T: float, rows, n_norm, g: float = 1.0, *, H_rows=None) -> dict:
    """The per-row outputs for a subset of rows of a larger batch: lse, zk, row_kl and the
    rows of dH. Each of these depends on its own row only, so this is the dense definition
    restricted to those rows. n_norm must be the batch's denominator (its N by default).
    H may be passed whole (rows are taken from it) or as H_rows, already sliced."""
    W = _f64(W)
    rows = np.asarray(rows, np.int64)
    Hr = _f64(H_rows) if H_rows is not None else _f64(H)[rows]
    ir = np.asarray(idx, np.int64)[rows]
    tr = np.asarray(tlog)[rows]
    V = W.shape[0]
    _check(ir, V)
    z = Hr @ W.T
    u = z / T
    lse = logsumexp_rows(u)
    lpt = teacher_logp(tr, T)
    pt = np.exp(lpt)
    zk = np.take_along_axis(z, ir, axis=1)
    row_kl = _kl_terms(pt, lpt, zk, T, lse)
    gs = g * T / float(n_norm)
    G = np.exp(u - lse[:, None])
    r = np.arange(len(rows))[:, None]
    G[r, ir] -= pt
    G *= gs
    return dict(lse=lse, row_kl=row_kl, zk=zk, dH=G @ W)


def lse_all_rows(H, W, T: float, block: int = 512) -> np.ndarray:
    """lse_n = logsumexp_v z_nv/T for every row of a large batch. Each row's value is the
    definition applied to that row alone (as in ``kl_rows``); rows are taken ``block`` at a time
    only to bound the size of the logit slab held in memory."""
    W = _f64(W)
    H = np.asarray(H)
    out = np.empty(H.shape[0])
    for r0 in range(0, H.shape[0], block):
        out[r0:r0 + block] = logsumexp_rows((_f64(H[r0:r0 + block]) @ W.T) / T)
    return out


def kl_rows_all(H, W, idx, tlog, T: float, block: int = 512) -> dict:
    """lse_n and KL_n for every row of a large batch. Each row's values are the definition
    applied to that row alone, as in ``kl_rows`` (the row's logits over all V, its teacher
    softmax over the K cached entries); rows are taken ``block`` at a time only to bound the
    logit slab held in memory. Returns dict(lse [N], row_kl [N])."""
    W = _f64(W)
    H = np.asarray(H)
    idx = np.asarray(idx, np.int64)
    tlog = np.asarray(tlog)
    N = H.shape[0]
    _check(idx, W.shape[0])
    lse = np.empty(N)
    row_kl = np.empty(N)
    for r0 in range(0, N, block):
        r1 = min(N, r0 + block)
        z = _f64(H[r0:r1]) @ W.T
        lse[r0:r1] = logsumexp_rows(z / T)
        lpt = teacher_logp(tlog[r0:r1], T)
        zk = np.take_along_axis(z, idx[r0:r1], axis=1)
        row_kl[r0:r1] = _kl_terms(np.exp(lpt), lpt, zk, T, lse[r0:r1])
    return dict(lse=lse, row_kl=row_kl)


def dw_rows(H, W, idx, tlog, T: float, vocab, lse, n_norm, g: float = 1.0) -> np.ndarray:
    """Rows ``vocab`` of dW = G^T H, where G = g*(T/n_norm)*(softmax(z/T) - P_t) and P_t is
    the teacher distribution scattered at the cached ids (zero elsewhere). Column v of G needs
    z[:, v] and every row's lse, which is passed in (``lse_all_rows``). This is the dense
    definition restricted to those columns."""
    H = _f64(H)
    V = np.asarray(W).shape[0]
    vocab = np.asarray(vocab, np.int64)
    Wv = _f64(np.asarray(W)[vocab])                       # only the rows asked for
    idx = np.asarray(idx, np.int64)
    _check(idx, V)
    zc = H @ Wv.T                                         # z[:, vocab]
    Pc = np.exp(zc / T - np.asarray(lse, np.float64)[:, None])
    pt = np.exp(teacher_logp(tlog, T))
    col = np.full(V, -1, np.int64)
    col[vocab] = np.arange(len(vocab))
    n, k = np.nonzero(col[idx] >= 0)                      # cached entries that fall in vocab
    Pc[n, col[idx[n, k]]] -= pt[n, k]
    return (g * T / float(n_norm)) * (Pc.T @ H)


def topk_cache(logits, K: int):
    """Offline cache for one teacher pass: the K largest logits per row and their token ids,
    largest first; equal logits are ordered by the lower token id."""
    x = _f64(logits)
    N, V = x.shape
    order = np.lexsort((np.broadcast_to(np.arange(V), x.shape), -x), axis=1)[:, :K]
    return order.astype(np.int32), np.take_along_axis(x, order, axis=1)


def truncation_terms(H, W, teacher, K: int, T: float = 1.0) -> dict:
    """What caching only the top K of a full-vocabulary teacher changes, per row.

    The pages name the top-K cache as the method's remaining restriction: it drops the tail
    of the teacher's distribution, which matters little for peaked positions and is lossy
    where the teacher spreads its mass over hundreds of candidates. Source: "Making knowledge
    distillation cheap enough to run in production", paragraph on the remaining restriction.

    With p_t = softmax(teacher/T) over all V, S its top-K ids (``topk_cache``), m = sum_S p_t,
    p_K = p_t/m on S and 0 elsewhere, p_s = softmax(H W^T / T):
      mass      m
      kl_full   KL(p_t || p_s), the loss against the whole teacher
      kl_topk   KL(p_K || p_s), the loss against the cached teacher (what the method computes)
      grad_rel  ||p_K - p_t|| / ||p_s - p_t|| (2-norms over V): the error of the cached
                teacher's logit gradient (p_s - p_K) relative to the full teacher's (p_s - p_t).
    """
    Hd, Wd, Td = _f64(H), _f64(W), _f64(teacher)
    N, V = Td.shape
    u = (Hd @ Wd.T) / T
    log_ps = u - logsumexp_rows(u)[:, None]
    a = Td / T
    log_pt = a - logsumexp_rows(a)[:, None]
    pt = np.exp(log_pt)
    ps = np.exp(log_ps)
    idx, _ = topk_cache(Td, K)
    rows = np.arange(N)[:, None]
    in_top = np.zeros((N, V), dtype=bool)
    in_top[rows, idx.astype(np.int64)] = True
    mass = np.where(in_top, pt, 0.0).sum(axis=1)
    kl_full = np.where(pt > 0, pt * (log_pt - log_ps), 0.0).sum(axis=1)
    log_pk = np.where(in_top, log_pt - np.log(mass)[:, None], -np.inf)
    pk = np.where(in_top, np.exp(log_pk), 0.0)
    kl_topk = np.where(in_top, pk * (np.where(in_top, log_pk, 0.0) - log_ps), 0.0).sum(axis=1)
    grad_rel = np.linalg.norm(pk - pt, axis=1) / np.linalg.norm(ps - pt, axis=1)
    return dict(mass=mass, kl_full=kl_full, kl_topk=kl_topk, grad_rel=grad_rel, idx=idx)
