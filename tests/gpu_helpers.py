"""Shared helpers for the GPU tests: move a datagen Problem to the device, run the library,
and compare with the oracle."""

import sys

import numpy as np
import torch

import datagen

TOL = {
    # the stated tolerances: loss and lse relative, dH and dW relative L2
    "fp32": dict(loss=1e-6, lse=1e-6, grad=1e-5),
    "bf16": dict(loss=2e-3, lse=2e-3, grad=1e-2),
}


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def to_torch(a: np.ndarray, dev="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def device_inputs(p: datagen.Problem, dev="cuda"):
    return (to_torch(p.H, dev), to_torch(p.W, dev), torch.from_numpy(p.idx).to(dev), to_torch(p.tlog, dev))


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def max_rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-30)))


def lse_err(a, b, T: float) -> float:
    """Largest lse error in units of max(|lse_n|, 1) + 4/T, to be held to the lse tolerance tol.
    lse_n is the log-sum-exp of the row's tempered logits, so its error is at most theirs; the
    logits (zk) are held to tol relative plus 4*tol absolute, which gives lse_n a bound of
    tol*(|lse_n| + 4/T). Where lse_n is far from 0 (at the configured heads it is near log V
    or above) this is the relative error with a small absolute slack; where it nears 0 (V = 1:
    lse_n is the one tempered logit) a purely relative bound would be undefined."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b) / (np.maximum(np.abs(b), 1.0) + 4.0 / T)))


def zk_dot_bound(H, W, idx) -> np.ndarray:
    """Forward error bound of each gathered logit z_nk = sum_i h_ni w_(idx_nk)i accumulated in
    fp32, with products exact (bf16 inputs) or rounded once (fp32 inputs), in any summation
    order: |fl(z) - z| <= gamma_(d+1) * sum_i |h_ni w_(idx_nk)i|, gamma_m = m u / (1 - m u),
    u = 2^-24 (the standard bound for a floating-point dot product; Higham, Accuracy and
    Stability of Numerical Algorithms, section 3.1). H and W as fp64 arrays, idx [N, K]."""
    d = H.shape[1]
    u = 2.0 ** -24
    g = (d + 1) * u / (1.0 - (d + 1) * u)
    aW = np.abs(W)
    out = np.empty(idx.shape)
    for r0 in range(0, H.shape[0], 256):
        s = np.abs(H[r0:r0 + 256]) @ aW.T
        out[r0:r0 + 256] = np.take_along_axis(s, np.asarray(idx[r0:r0 + 256], np.int64), axis=1)
    return g * out


def assert_zk(got, ref_zk, tol_lse: float, H, W, idx):
    """zk against the oracle: within tol relative plus 4*tol absolute, or else within the fp32
    dot-product bound (zk_dot_bound), which no correct gather and accumulation exceeds."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref_zk)
    ok = err <= tol_lse * np.abs(ref_zk) + 4.0 * tol_lse
    if not ok.all():
        bad = ~ok
        bound = zk_dot_bound(H, W, idx)
        assert np.all(err[bad] <= bound[bad]), (err[bad].max(), bound[bad].min())


def kl_input_bound(ref: dict, T: float, tol_lse: float) -> np.ndarray:
    """Per-row bound on the error of KL_n carried in from its inputs: the GPU forms
    KL_n = sum_k p_k (log p_k - zk_nk / T + lse_n) from lse and zk, each held to tol_lse
    relative, so KL_n may be off by tol_lse * (|lse_n| + max_k |zk_nk| / T) whatever its own
    size. It decides where KL_n is much smaller than the terms it cancels from (a flat
    teacher against a near-uniform student; V = 1, where every KL_n is exactly 0)."""
    return tol_lse * (np.abs(ref["lse"]) + np.abs(ref["zk"]).max(axis=1) / T)


def row_kl_err(got, ref: dict, T: float, tol: dict) -> float:
    """Largest per-row KL error over its bar, max(tol * max_m |KL_m|, the input bound); <= 1
    passes."""
    got = np.asarray(got, np.float64)
    bar = np.maximum(tol["loss"] * np.abs(ref["row_kl"]).max(), kl_input_bound(ref, T, tol["lse"]))
    return float(np.max(np.abs(got - ref["row_kl"]) / bar))


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
