"""kd_fused_kl_fwd_noalloc: the fused forward with the library's static device scratch as its
workspace, for callers that cannot allocate. Its outputs must equal kd_fused_kl_fwd's bit for
bit (the same kernels run) and the oracle's within the stated tolerances, on two calls in a
row with the second problem smaller than the first; the second call must not change the
device's free memory; arguments the scratch cannot hold are rejected before anything runs."""

import ctypes
import os

import numpy as np
import pytest
import torch

import datagen
import oracle
import lm_head_kl_amd as kd
from lm_head_kl_amd import _lib
from lm_head_kl_amd._lib import KD_BF16, KdProblem

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
nogpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake pointers are only passed when no GPU is visible")
F = ctypes.c_void_p(0x10000)  # never dereferenced


def _prob(**kw):
    base = dict(N=4096, d=1024, V=32000, K=100, chunk=1024, T=1.0, n_norm=0.0, act=KD_BF16, tlogit=KD_BF16,
                flags=0, reserved=0)
    base.update(kw)
    return KdProblem(**base)


def _call(p, H=F, loss=F, lse=F):
    return _lib.lib().kd_fused_kl_fwd_noalloc(ctypes.byref(p), H, F, F, F, loss, lse, None, None, None)


@pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libkdkl.so not built")
@nogpu
def test_noalloc_argument_checks():
    """Host-side checks, nothing enqueued: a problem whose forward workspace exceeds the scratch,
    KD_VALIDATE_IDX (it would copy to the host and wait), NULL and misaligned pointers."""
    assert _lib.KD_NOALLOC_SCRATCH_BYTES == 64 << 20
    # the forward's workspace grows by about 8K + 16 Q bytes a row (Q = 1 vocabulary lane at
    # V = 256): 90,000 rows at K = 100 do not fit
    assert _call(_prob(N=90000, d=8, V=256)) == 5
    assert _call(_prob(flags=_lib.KD_VALIDATE_IDX)) == 4
    assert _call(_prob(), loss=None) == 1 and _call(_prob(), lse=None) == 1
    assert _call(_prob(), H=ctypes.c_void_p(0x10008)) == 4
    assert _call(_prob(K=0)) == 2
    assert _lib.lib().kd_fused_kl_fwd_noalloc(None, F, F, F, F, F, F, None, None, None) == 1


def _outputs(N, K, dev):
    return (torch.empty((), dtype=torch.float32, device=dev), torch.empty(N, dtype=torch.float32, device=dev),
            torch.empty(N, dtype=torch.float32, device=dev), torch.empty((N, K), dtype=torch.float32, device=dev))


@pytest.mark.gpu
def test_noalloc_forward_matches_the_workspace_forward():
    cases = [
        ("gptoss", dict(), 2e-3),                                         # N = 32768 at the gpt-oss head
        ("small", dict(), 2e-3),                                          # N = 4096, bf16, Zipf ids
        ("tiny", dict(N=300, d=200, V=1000, K=7, T=1.3, dtype="fp32"), 1e-6),  # smaller, ragged, fp32
    ]
    dev = torch.device("cuda:0")
    for i, (cfg, over, tol) in enumerate(cases):
        p = datagen.make(cfg, **over)
        print(f"[gpu-test] noalloc call {i + 1}: {cfg} N={p.N} d={p.d} V={p.V} K={p.K} {p.dtype}", flush=True)
        H = torch.from_numpy(np.ascontiguousarray(p.H).view(np.int16)).to(dev).view(torch.bfloat16) \
            if p.H.dtype == np.uint16 else torch.from_numpy(p.H).to(dev)
        W = torch.from_numpy(np.ascontiguousarray(p.W).view(np.int16)).to(dev).view(torch.bfloat16) \
            if p.W.dtype == np.uint16 else torch.from_numpy(p.W).to(dev)
        t = torch.from_numpy(np.ascontiguousarray(p.tlog).view(np.int16)).to(dev).view(torch.bfloat16) \
            if p.tlog.dtype == np.uint16 else torch.from_numpy(p.tlog).to(dev)
        idx = torch.from_numpy(p.idx).to(dev)
        ref = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=p.chunk, want_zk=True)
        loss, lse, row_kl, zk = _outputs(p.N, p.K, dev)
        torch.cuda.synchronize()
        free0, _ = torch.cuda.mem_get_info(dev)
        alloc0 = torch.cuda.memory_allocated(dev)
        kd.fused_kl_fwd_noalloc(H, W, idx, t, loss, lse, row_kl, zk, T=p.T, chunk=p.chunk)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated(dev) == alloc0
        if i > 0:  # the first call may be the library's first use of the device (code object load)
            assert torch.cuda.mem_get_info(dev)[0] == free0
        for a, b in ((loss, ref.loss), (lse, ref.lse), (row_kl, ref.row_kl), (zk, ref.zk)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        if cfg == "gptoss":  # every row's lse and KL_n from the stored oracle values
            lse_ref = np.load(os.path.join(GOLDEN, "gptoss_lse.npy"), allow_pickle=False)
            kl_ref = np.load(os.path.join(GOLDEN, "gptoss_rowkl.npy"), allow_pickle=False)
            want = dict(lse=lse_ref, row_kl=kl_ref, loss=float(np.sum(kl_ref)) * p.T * p.T / p.N)
        else:
            want = oracle.kl_chunked(p.f64("H"), p.f64("W"), p.idx, p.f64("tlog"), p.T, chunk=max(p.chunk, 256))
        assert abs(loss.item() - want["loss"]) <= tol * abs(want["loss"])
        lse_h = lse.double().cpu().numpy()
        assert np.max(np.abs(lse_h - want["lse"]) / np.abs(want["lse"])) <= tol
        rk = row_kl.double().cpu().numpy()
        assert np.max(np.abs(rk - want["row_kl"]) / np.abs(want["row_kl"])) <= tol


@pytest.mark.gpu
def test_noalloc_rejects_before_launch_on_gpu():
    """With real tensors: a problem the scratch cannot hold and KD_VALIDATE_IDX are rejected on
    the host, and the outputs are left as they were."""
    dev = torch.device("cuda:0")
    N, d, V, K = 90000, 8, 256, 100
    H = torch.zeros((N, d), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((V, d), dtype=torch.bfloat16, device=dev)
    idx = torch.zeros((N, K), dtype=torch.int32, device=dev)
    t = torch.zeros((N, K), dtype=torch.bfloat16, device=dev)
    loss, lse, row_kl, zk = _outputs(N, K, dev)
    lse.fill_(7.0)
    with pytest.raises(kd.KdError) as e:
        kd.fused_kl_fwd_noalloc(H, W, idx, t, loss, lse, T=1.0, chunk=2048)
    assert e.value.code == 5
    with pytest.raises(kd.KdError) as e:
        kd.fused_kl_fwd_noalloc(H[:100], W, idx[:100], t[:100], loss, lse[:100], T=1.0, chunk=64,
                                flags=kd.KD_VALIDATE_IDX)
    assert e.value.code == 4
    torch.cuda.synchronize()
    assert bool((lse == 7.0).all())
