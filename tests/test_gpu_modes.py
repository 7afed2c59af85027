"""Masked teacher entries (cached logit -inf) on every formulation, the memory-lean fused
backward (KD_LOW_MEMORY) against the oracle and the default backward, and the autograd term
with an fp32 dW accumulator."""

import os

import numpy as np
import pytest
import torch

import datagen
import oracle
import lm_head_kl_amd as kd
from gpu_helpers import TOL, device_inputs, host, max_rel, rel_l2, say

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def masked_problem(dtype, N, d, V, K, T, seed=5):
    """A tiny-recipe problem whose cached teacher logits are -inf at about a third of the
    entries (never the first of a row, so every row keeps a finite entry)."""
    p = datagen.make("tiny", N=N, d=d, V=V, K=K, T=T, dtype=dtype, chunk=128)
    tl = p.f32("tlog").copy()
    g = np.random.default_rng(seed)
    m = g.random(tl.shape) < 0.35
    m[:, 0] = False
    tl[m] = -np.inf
    p.tlog = datagen.bf16_bits(tl) if dtype == "bf16" else tl.astype(np.float32)
    assert np.isneginf(p.f64("tlog")).sum() == m.sum()
    return p


def check_out(label, tol, ref, loss, lse, row_kl, dH, dW, grad):
    for a in (loss, lse, row_kl, dH, dW):
        assert bool(torch.isfinite(a.float()).all()), label
    got = float(loss.item()) * grad
    assert abs(got - ref["loss"]) <= tol["loss"] * abs(ref["loss"]), (label, got, ref["loss"])
    assert max_rel(host(lse), ref["lse"]) <= tol["lse"], label
    assert max_rel(host(row_kl), ref["row_kl"]) <= tol["loss"], label
    e_dh, e_dw = rel_l2(host(dH), ref["dH"]), rel_l2(host(dW), ref["dW"])
    say(f"  {label}: dH relL2 {e_dh:.2e}  dW relL2 {e_dw:.2e}")
    assert e_dh <= tol["grad"] and e_dw <= tol["grad"], label


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("N,d,V,K,T", [
    (300, 64, 1500, 24, 1.0),
    (200, 64, 40, 40, 1.3),      # K = V: every token cached, a third of them masked
])
def test_masked_teacher_entries_every_path(dtype, N, d, V, K, T):
    """A -inf teacher logit has p_t = 0: it adds nothing to KL_n and nothing is subtracted at
    its id. The fused pair (default and memory-lean), the single-pass, forward-chunked and
    dense calls must stay finite and match the dense oracle, which sums p log p over the full
    vocabulary with 0 log 0 = 0."""
    p = masked_problem(dtype, N, d, V, K, T)
    say("masked teacher entries", dtype, f"N={N} d={d} V={V} K={K}")
    H, W, idx, t = device_inputs(p)
    grad = 0.8
    g = torch.tensor(grad, dtype=torch.float32, device=H.device)
    ref = oracle.kl_dense(p.f64("H"), p.f64("W"), p.idx, p.f64("tlog"), p.T, g=grad)
    tol = TOL[dtype]
    for flags, label in ((0, "fused"), (kd.KD_LOW_MEMORY, "fused low-memory")):
        f = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=128, flags=flags)
        dH, dW = kd.fused_kl_bwd(H, W, idx, t, f.lse, grad_loss=g, T=p.T, chunk=128, flags=flags)
        torch.cuda.synchronize()
        check_out(label, tol, ref, f.loss, f.lse, f.row_kl, dH, dW, grad)
    for fn, label in ((kd.fused_kl_fwdbwd, "single pass"), (kd.chunked_kl, "forward-chunked")):
        loss, lse, row_kl, dH, dW = fn(H, W, idx, t, T=p.T, chunk=128, grad_loss=g)
        torch.cuda.synchronize()
        check_out(label, tol, ref, loss, lse, row_kl, dH, dW, grad)
    loss, lse, row_kl, dH, dW = kd.dense_kl(H, W, idx, t, T=p.T, grad_loss=g)
    torch.cuda.synchronize()
    check_out("dense", tol, ref, loss, lse, row_kl, dH, dW, grad)


# ------------------------------------------------------------------ memory-lean backward

def lean_vs_oracle(p, chunk, tol, grad=1.0, n_norm=None, label=""):
    say("low-memory parity", label or p.name, f"N={p.N} d={p.d} V={p.V} K={p.K} chunk={chunk} {p.dtype}")
    H, W, idx, t = device_inputs(p)
    nn = 0.0 if n_norm is None else n_norm
    g = torch.tensor(grad, dtype=torch.float32, device=H.device)
    f = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=chunk, n_norm=nn, flags=kd.KD_LOW_MEMORY)
    dH, dW = kd.fused_kl_bwd(H, W, idx, t, f.lse, grad_loss=g, T=p.T, chunk=chunk, n_norm=nn,
                             flags=kd.KD_LOW_MEMORY)
    torch.cuda.synchronize()
    ref = oracle.kl_chunked(p.f64("H"), p.f64("W"), p.idx, p.f64("tlog"), p.T, chunk=max(chunk, 256),
                            n_norm=n_norm, g=grad)
    check_out(label or p.name, tol, ref, f.loss, f.lse, f.row_kl, dH, dW, grad)
    return H, W, idx, t, f, dH, dW


def test_low_memory_tiny_fp32():
    p = datagen.make("tiny")
    lean_vs_oracle(p, p.chunk, TOL["fp32"])


def test_low_memory_small_bf16():
    p = datagen.make("small")
    lean_vs_oracle(p, p.chunk, TOL["bf16"], grad=-0.6, n_norm=5000.0)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("shape", [
    dict(N=300, d=200, V=1000, K=7, chunk=128, T=1.3),     # every size ragged
    dict(N=1, d=64, V=300, K=1, chunk=1, T=0.7),           # one row, K = 1
    dict(N=301, d=64, V=700, K=9, chunk=3, T=1.0),          # chunks not a multiple of 4 or of a block
    dict(N=600, d=648, V=5000, K=40, chunk=1000, T=1.1),    # one chunk holding more than two blocks
    dict(N=64, d=32, V=40, K=40, chunk=64, T=1.0),          # K = V
])
def test_low_memory_ragged_shapes(dtype, shape):
    p = datagen.make("tiny", N=shape["N"], d=shape["d"], V=shape["V"], K=shape["K"], T=shape["T"],
                     dtype=dtype, chunk=shape["chunk"])
    lean_vs_oracle(p, shape["chunk"], TOL[dtype], grad=0.75, label=f"lean {shape} {dtype}")


def test_low_memory_matches_default_and_flags():
    """Against the default backward on the same inputs (the two differ in summation order only),
    repeatable bit for bit, KD_ACCUMULATE_DW doubling dW, KD_SKIP_DW giving the same dH."""
    p = datagen.make("small", N=2000)
    say("low-memory vs default, flags")
    H, W, idx, t = device_inputs(p)
    f = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=768)
    dH0, dW0 = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=768)
    dH1, dW1 = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=768, flags=kd.KD_LOW_MEMORY)
    dH2, dW2 = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=768, flags=kd.KD_LOW_MEMORY)
    torch.cuda.synchronize()
    assert rel_l2(host(dH1), host(dH0)) <= 5e-3 and rel_l2(host(dW1), host(dW0)) <= 5e-3
    assert torch.equal(dH1.view(torch.int16), dH2.view(torch.int16)) and torch.equal(dW1, dW2)
    acc = dW1.clone()
    kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=768, flags=kd.KD_LOW_MEMORY | kd.KD_ACCUMULATE_DW, dW=acc)
    dH3, none = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=768, flags=kd.KD_LOW_MEMORY | kd.KD_SKIP_DW)
    torch.cuda.synchronize()
    # one dW pass per chunk adds the chunks into the old values one at a time, so the doubled
    # dW matches 2 dW to rounding, not bit for bit
    assert rel_l2(host(acc), 2 * host(dW1)) <= 1e-6 and none is None
    assert torch.equal(dH3.view(torch.int16), dH1.view(torch.int16))


def test_stage_tiled_copies_change_no_bit_and_keep_the_flags():
    """From 8192 rows the default calls read W and H through stage-tiled copies, the memory-lean
    ones as stored. The forward's arithmetic is the same either way, so lse, zk, KL_n and the loss
    agree bit for bit; on the tiled backward KD_SKIP_DW gives the same dH bit for bit and
    KD_ACCUMULATE_DW adds into dW."""
    p = datagen.make("tiny", N=8448, d=264, V=3000, dtype="bf16", chunk=768)
    say("stage-tiled vs as stored, flags", f"N={p.N} d={p.d} V={p.V} K={p.K}")
    H, W, idx, t = device_inputs(p)
    f = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=768, want_zk=True)
    g = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=768, want_zk=True, flags=kd.KD_LOW_MEMORY)
    torch.cuda.synchronize()
    for a, b in ((f.loss, g.loss), (f.lse, g.lse), (f.zk, g.zk), (f.row_kl, g.row_kl)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    dH0, dW0 = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=768)
    dH1, none = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=768, flags=kd.KD_SKIP_DW)
    acc = dW0.clone()
    kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=768, flags=kd.KD_ACCUMULATE_DW, dW=acc)
    torch.cuda.synchronize()
    assert none is None and torch.equal(dH1.view(torch.int16), dH0.view(torch.int16))
    assert rel_l2(host(acc), 2 * host(dW0)) <= 1e-6


def test_low_memory_gptoss_sampled():
    """The memory-lean backward at the gpt-oss head (N = 32768, chunk 2048): dH on 256 seeded
    rows against the oracle, 256 rows of the full-batch dW against oracle.dw_rows (from the
    stored every-row lse), and dW's columns summing to zero."""
    p = datagen.make("gptoss")
    say("low-memory gpt-oss sampled")
    H, W, idx, t = device_inputs(p)
    f = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=2048, flags=kd.KD_LOW_MEMORY)
    dH, dW = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=2048, flags=kd.KD_LOW_MEMORY)
    torch.cuda.synchronize()
    rows = datagen.sample_rows(p.N, 256, p.extra["seed"])
    ref = oracle.kl_rows(None, p.f64("W"), p.idx, p.f64("tlog"), p.T, rows, n_norm=p.N,
                         H_rows=datagen.bf16_to_f32(p.H[rows]))
    e = rel_l2(host(dH[torch.from_numpy(rows).to(dH.device)]), ref["dH"])
    say(f"  sampled dH relL2 {e:.2e}")
    assert e <= TOL["bf16"]["grad"]
    colsum = dW.double().sum(0)
    scale = dW.double().abs().sum(0)
    assert float((colsum.abs() / scale.clamp_min(1e-30)).max()) < 1e-3
    vocab = datagen.sample_vocab(p.V, 256, p.extra["seed"])
    got = host(dW[torch.from_numpy(vocab).to(dW.device)])
    del dH, dW, f
    lse_ref = np.load(os.path.join(GOLDEN, "gptoss_lse.npy"), allow_pickle=False)
    want = oracle.dw_rows(p.f32("H"), p.f32("W"), p.idx, p.f64("tlog"), p.T, vocab, lse_ref, n_norm=p.N)
    e_dw = rel_l2(got, want)
    say(f"  dW rows relL2 {e_dw:.2e}")
    assert e_dw <= TOL["bf16"]["grad"]


# ------------------------------------------------------------------ autograd with fp32 dW

def test_fused_kl_autograd_bf16_with_fp32_accumulator():
    """A bf16 head through the autograd term: with an fp32 accumulator, dW stays in fp32 and two
    micro-batches (halves of the small config, n_norm = the whole batch) add up in it; H's
    gradients come back in bf16. Both against the oracle on the whole batch; without the
    accumulator W.grad is the same dW rounded to bf16."""
    p = datagen.make("small")
    say("FusedKL bf16 with fp32 dW accumulator")
    H, W, idx, t = device_inputs(p)
    ref = oracle.kl_chunked(p.f64("H"), p.f64("W"), p.idx, p.f64("tlog"), p.T, chunk=1024)
    acc = torch.zeros(W.shape, dtype=torch.float32, device=H.device)
    Wp = W.clone().requires_grad_(True)
    half = p.N // 2
    dHs, total = [], 0.0
    for r0 in (0, half):
        Hp = H[r0:r0 + half].clone().requires_grad_(True)
        loss = kd.fused_kl(Hp, Wp, idx[r0:r0 + half], t[r0:r0 + half], T=p.T, chunk=1024, n_norm=float(p.N),
                           dw_accumulator=acc)
        loss.backward()
        total += float(loss.item())
        dHs.append(Hp.grad)
    torch.cuda.synchronize()
    assert Wp.grad is None  # the gradient went to the accumulator
    assert dHs[0].dtype == torch.bfloat16
    tol = TOL["bf16"]
    assert abs(total - ref["loss"]) <= tol["loss"] * ref["loss"]
    e_dh = rel_l2(host(torch.cat(dHs)), ref["dH"])
    e_dw = rel_l2(acc.double().cpu().numpy(), ref["dW"])
    say(f"  dH relL2 {e_dh:.2e}  dW (fp32 accumulator) relL2 {e_dw:.2e}")
    assert e_dh <= tol["grad"] and e_dw <= tol["grad"]
    # without the accumulator: W.grad in bf16, equal to the library's fp32 dW rounded
    Wq = W.clone().requires_grad_(True)
    loss = kd.fused_kl(H, Wq, idx, t, T=p.T, chunk=1024, low_memory=True)
    loss.backward()
    f = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=1024)
    _, dW = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=1024, flags=kd.KD_LOW_MEMORY)
    torch.cuda.synchronize()
    assert Wq.grad.dtype == torch.bfloat16
    assert torch.equal(Wq.grad.view(torch.int16), dW.to(torch.bfloat16).view(torch.int16))
