"""Properties of the HIP path that hold at any size: determinism, accumulation, the id
validation flag, the K = 1 cross-entropy case, agreement of the fused and dense paths,
autograd wiring, and peak device memory that does not grow with the sequence beyond the
per-row buffers."""

import numpy as np
import pytest
import torch

import datagen
import lm_head_kl_amd as kd
from gpu_helpers import TOL, device_inputs, host, rel_l2, say

pytestmark = pytest.mark.gpu


def test_bitwise_deterministic():
    p = datagen.make("small", N=2048)
    say("determinism small N=2048")
    H, W, idx, t = device_inputs(p)
    outs = []
    for _ in range(2):
        f = kd.fused_kl_fwd(H, W, idx, t, T=1.0, chunk=512, want_zk=True)
        dH, dW = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=1.0, chunk=512)
        torch.cuda.synchronize()
        outs.append([x.clone() for x in (f.loss, f.lse, f.row_kl, f.zk, dH, dW)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int8) if a.dtype == torch.bfloat16 else a, b.view(torch.int8)
                           if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_backward_reproducible_across_plan_order(dtype):
    """The plan fills each (row block, vocab tile) bucket in atomic order, so an entry's place in
    its bucket changes between calls. With K = 1024 over 12 vocab tiles a bucket's 512th entry
    falls in rows 5-6, whose entries are therefore subtracted by the in-register path in one call
    and by the loop in the next: the fp32 gradients must still come out bit for bit the same."""
    p = datagen.make("tiny", N=505, d=584, V=3038, K=1024, T=1.0, chunk=256, dtype=dtype,
                     teacher="flat", ids="uniform", seed=5009)
    say("backward reproducible over plan order", dtype)
    H, W, idx, t = device_inputs(p)
    f = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=256)
    outs = []
    for _ in range(4):
        dH, dW = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=256)
        torch.cuda.synchronize()
        outs.append((dH.clone(), dW.clone()))
    for dH, dW in outs[1:]:
        assert torch.equal(dH.view(torch.int16) if dtype == "bf16" else dH,
                           outs[0][0].view(torch.int16) if dtype == "bf16" else outs[0][0])
        assert torch.equal(dW, outs[0][1])


def test_accumulate_dw_doubles():
    p = datagen.make("tiny")
    say("KD_ACCUMULATE_DW")
    H, W, idx, t = device_inputs(p)
    f = kd.fused_kl_fwd(H, W, idx, t, T=1.0, chunk=64)
    # One chunk: the second call adds exactly the same fp32 values, so the sum is exact.
    _, dW1 = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=1.0, chunk=p.N)
    acc = dW1.clone()
    kd.fused_kl_bwd(H, W, idx, t, f.lse, T=1.0, chunk=p.N, flags=kd.KD_ACCUMULATE_DW, dW=acc)
    torch.cuda.synchronize()
    assert torch.equal(acc, dW1 + dW1)
    # Several chunks: the running sum differs from 2*dW only by fp32 rounding.
    _, dW4 = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=1.0, chunk=64)
    acc4 = dW4.clone()
    kd.fused_kl_bwd(H, W, idx, t, f.lse, T=1.0, chunk=64, flags=kd.KD_ACCUMULATE_DW, dW=acc4)
    torch.cuda.synchronize()
    assert rel_l2(host(acc4), 2 * host(dW4)) <= 1e-6


def test_validate_flag():
    p = datagen.make("tiny")
    say("KD_VALIDATE_IDX")
    H, W, idx, t = device_inputs(p)
    f = kd.fused_kl_fwd(H, W, idx, t, T=1.0, chunk=64, flags=kd.KD_VALIDATE_IDX)
    torch.cuda.synchronize()
    dup = idx.clone()
    dup[5, 3] = dup[5, 0]
    with pytest.raises(kd.KdError) as e:
        kd.fused_kl_fwd(H, W, dup, t, T=1.0, chunk=64, flags=kd.KD_VALIDATE_IDX)
    assert e.value.code == 6
    oob = idx.clone()
    oob[7, 1] = p.V
    with pytest.raises(kd.KdError) as e:
        kd.fused_kl_bwd(H, W, oob, t, f.lse, T=1.0, chunk=64, flags=kd.KD_VALIDATE_IDX)
    assert e.value.code == 6
    # without the flag an out-of-range id is skipped, never dereferenced
    neg = idx.clone()
    neg[3, 2] = -5
    g = kd.fused_kl_fwd(H, W, neg, t, T=1.0, chunk=64)
    torch.cuda.synchronize()
    assert torch.isfinite(g.lse).all()


def test_workspace_too_small_is_rejected():
    p = datagen.make("tiny")
    H, W, idx, t = device_inputs(p)
    small = torch.empty(1024, dtype=torch.uint8, device="cuda")
    prob = kd.make_problem(H, W, idx, t, 1.0, 64)
    need = kd.fused_workspace_bytes(prob)
    assert need > 1024
    import ctypes
    from lm_head_kl_amd import _lib
    loss = torch.empty((), device="cuda")
    lse = torch.empty(p.N, device="cuda")
    code = _lib.lib().kd_fused_kl_fwd(ctypes.byref(prob), ctypes.c_void_p(H.data_ptr()),
                                      ctypes.c_void_p(W.data_ptr()), ctypes.c_void_p(idx.data_ptr()),
                                      ctypes.c_void_p(t.data_ptr()), ctypes.c_void_p(loss.data_ptr()),
                                      ctypes.c_void_p(lse.data_ptr()), None, None,
                                      ctypes.c_void_p(small.data_ptr()), 1024, None)
    assert code == 5


def test_binding_rejects_bad_buffers():
    """The binding checks what the C ABI cannot (device, layout, size of caller tensors) and
    raises before anything is enqueued."""
    p = datagen.make("tiny")
    H, W, idx, t = device_inputs(p)
    f = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=64)
    prob = kd.make_problem(H, W, idx, t, p.T, 64)
    need = kd.fused_workspace_bytes(prob)
    bad = {
        "dW on the host": dict(dW=torch.empty(W.shape, dtype=torch.float32)),
        "dW not contiguous": dict(dW=torch.empty((W.shape[1], W.shape[0]), dtype=torch.float32,
                                                  device="cuda").t()),
        "dW of another dtype": dict(dW=torch.empty(W.shape, dtype=torch.bfloat16, device="cuda")),
        "workspace on the host": dict(workspace=torch.empty(need, dtype=torch.uint8)),
        "workspace too small": dict(workspace=torch.empty(need - 256, dtype=torch.uint8, device="cuda")),
    }
    for label, kw in bad.items():
        with pytest.raises(kd.KdError):
            kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=64, **kw)
        say("  rejected:", label)
    with pytest.raises(kd.KdError):
        kd.fused_kl_bwd(H, W, idx, t, f.lse[:-1], T=p.T, chunk=64)
    with pytest.raises(kd.KdError):
        kd.fused_kl_bwd(H, W, idx, t, f.lse.double(), T=p.T, chunk=64)
    with pytest.raises(kd.KdError):
        kd.chunked_kl(H, W, idx, t, T=p.T, chunk=64, dW=torch.empty(W.shape, dtype=torch.float32))
    with pytest.raises(kd.KdError):
        kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=64, workspace=torch.empty(16, device="cuda"))
    with pytest.raises(kd.KdError):
        kd.fused_kl_fwd(H[None], W, idx, t, T=p.T, chunk=64)
    # a workspace of another element type counts in bytes
    ws = torch.empty((need + 3) // 4, dtype=torch.float32, device="cuda")
    dH, dW = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=64, workspace=ws)
    dH0, dW0 = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(dH, dH0) and torch.equal(dW, dW0)


@pytest.mark.parametrize("T", [1.0, 2.0])
def test_k1_matches_torch_cross_entropy(T):
    """One cached entry per row: the loss is T^2 times cross entropy of z/T at that id."""
    p = datagen.make("small", N=1024, K=1, T=T)
    say("K=1 vs cross_entropy", T)
    H, W, idx, t = device_inputs(p)
    f = kd.fused_kl_fwd(H, W, idx, t, T=T, chunk=512)
    torch.cuda.synchronize()
    z = H.float() @ W.float().t()
    ce = torch.nn.functional.cross_entropy(z / T, idx[:, 0].long())
    assert abs(f.loss.item() - T * T * ce.item()) <= 2e-3 * T * T * ce.item()


def test_fused_equals_dense_path():
    p = datagen.make("small", N=1024)
    say("fused vs dense, small N=1024")
    H, W, idx, t = device_inputs(p)
    f = kd.fused_kl_fwd(H, W, idx, t, T=1.0, chunk=256)
    dH, dW = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=1.0, chunk=256)
    loss, lse, row_kl, dH2, dW2 = kd.dense_kl(H, W, idx, t, T=1.0)
    torch.cuda.synchronize()
    assert abs(f.loss.item() - loss.item()) <= 1e-4 * loss.item()
    assert rel_l2(host(f.lse), host(lse)) <= 1e-6
    assert rel_l2(host(dH), host(dH2)) <= 5e-3 and rel_l2(host(dW), host(dW2)) <= 5e-3


def test_chunk_invariance():
    p = datagen.make("small", N=2048)
    say("chunk invariance")
    H, W, idx, t = device_inputs(p)
    f = kd.fused_kl_fwd(H, W, idx, t, T=1.0, chunk=512)
    res = [kd.fused_kl_bwd(H, W, idx, t, f.lse, T=1.0, chunk=c) for c in (300, 1024, 2048)]
    torch.cuda.synchronize()
    for dH, dW in res[1:]:
        assert rel_l2(host(dH), host(res[0][0])) <= 5e-3
        assert rel_l2(host(dW), host(res[0][1])) <= 5e-3


def test_autograd_function():
    p = datagen.make("tiny")
    say("autograd FusedKL")
    H, W, idx, t = device_inputs(p)
    Hp = H.clone().requires_grad_(True)
    Wp = W.clone().requires_grad_(True)
    loss = kd.fused_kl(Hp, Wp, idx, t, T=1.0, chunk=64)
    (3.0 * loss).backward()
    f = kd.fused_kl_fwd(H, W, idx, t, T=1.0, chunk=64)
    dH, dW = kd.fused_kl_bwd(H, W, idx, t, f.lse, grad_loss=torch.tensor(3.0, device="cuda"), T=1.0, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(Hp.grad, dH) and torch.equal(Wp.grad, dW)


def _peak(fn):
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    fn()
    torch.cuda.synchronize()
    return torch.cuda.max_memory_allocated() - base


def test_fused_peak_memory_flat_in_sequence():
    """At the gpt-oss head (V = 201,088, d = 2880, chunk 2048) the fused call's peak beyond its
    inputs is the per-row buffers (lse, zk, dH, cache plan) plus a constant: growing S leaves
    the constant unchanged. Below 8192 rows the calls keep no stage-tiled copy of W (1.16 GB),
    so the constant there is smaller, never larger."""
    V, d, K = 201088, 2880, 100
    W = torch.randn(V, d, device="cuda", dtype=torch.bfloat16)
    extra = []
    for S in (4096, 8192, 16384, 32768):
        H = torch.randn(S, d, device="cuda", dtype=torch.bfloat16)
        idx = torch.stack([torch.randperm(V, device="cuda")[:K] for _ in range(1)]).repeat(S, 1).int()
        t = torch.randn(S, K, device="cuda", dtype=torch.bfloat16)

        def step():
            f = kd.fused_kl_fwd(H, W, idx, t, T=1.0, chunk=2048, want_row_kl=False)
            kd.fused_kl_bwd(H, W, idx, t, f.lse, T=1.0, chunk=2048)

        pk = _peak(step)
        per_row = S * (d * 2 + 4 + K * 4 * 2 + K * 4 + 16)  # dH, lse, zk + plan, partials
        extra.append(pk - per_row)
        say(f"  S={S} fused peak {pk / 1e9:.3f} GB  minus per-row {extra[-1] / 1e9:.3f} GB")
        del H, idx, t
    # dW (fp32, 2.3 GB), the tiled copy of W (1.16 GB) and the gradient tile (C x V bf16,
    # 0.82 GB) dominate; no growth with S
    big = extra[1:]
    assert max(big) - min(big) <= 0.02 * max(big)
    assert extra[0] <= min(big)


def test_skip_dw_frozen_head():
    """KD_SKIP_DW computes the same dH bit for bit and leaves dW alone; the autograd term uses it
    when W does not require a gradient."""
    p = datagen.make("small", N=1536)
    say("KD_SKIP_DW")
    H, W, idx, t = device_inputs(p)
    f = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=512)
    dH_full, dW_full = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=512)
    dH_skip, dW_none = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=512, flags=kd.KD_SKIP_DW)
    torch.cuda.synchronize()
    assert dW_none is None
    assert torch.equal(dH_full.view(torch.int16), dH_skip.view(torch.int16))
    # autograd: frozen head
    Hg = H.clone().requires_grad_(True)
    loss = kd.fused_kl(Hg, W, idx, t, T=p.T, chunk=512)
    loss.backward()
    torch.cuda.synchronize()
    assert torch.equal(Hg.grad.view(torch.int16), dH_full.view(torch.int16))
    assert W.grad is None


def test_validate_ids_without_sync():
    """kd_validate_ids leaves its result in a device word: 0 for a sound cache, bit 1 for an id
    out of range, bit 2 for a repeated id. It enqueues only kernels, so it can sit in a captured
    graph in front of the loss; each replay clears the word and checks the ids as they are then."""
    p = datagen.make("tiny")
    say("kd_validate_ids")
    H, W, idx, t = device_inputs(p)
    assert int(kd.validate_ids(idx, p.V).item()) == 0
    dup = idx.clone()
    dup[5, 3] = dup[5, 0]
    oob = idx.clone()
    oob[7, 1] = p.V
    both = dup.clone()
    both[9, 2] = -1
    assert int(kd.validate_ids(dup, p.V).item()) == 2
    assert int(kd.validate_ids(oob, p.V).item()) == 1
    assert int(kd.validate_ids(both, p.V).item()) == 3
    # in a graph with the forward
    st = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(kd.fused_workspace_bytes(kd.make_problem(H, W, idx, t, p.T, 64)), dtype=torch.uint8,
                     device="cuda")
    work = idx.clone()
    eager = kd.fused_kl_fwd(H, W, work, t, T=p.T, chunk=64, workspace=ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kd.validate_ids(work, p.V, st)
        kd.fused_kl_fwd(H, W, work, t, T=p.T, chunk=64, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kd.validate_ids(work, p.V, st)
        f = kd.fused_kl_fwd(H, W, work, t, T=p.T, chunk=64, workspace=ws)
    for ids, want in ((idx, 0), (both, 3), (dup, 2), (idx, 0)):
        work.copy_(ids)
        g.replay()
        torch.cuda.synchronize()
        assert int(st.item()) == want
        if want == 0:
            assert torch.equal(f.lse, eager.lse) and torch.equal(f.loss, eager.loss)
