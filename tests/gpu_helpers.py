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


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
