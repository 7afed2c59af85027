"""Seeded random problems: sizes, dtype, temperature, teacher recipe, id recipe, chunk,
normaliser and upstream weight are drawn per case, and each of the four formulations (and the
memory-lean fused backward) is compared in full with the fp64 oracle at the stated tolerances. The fixed edge list
elsewhere names the boundaries one at a time; here they are combined the way a caller might
combine them (a ragged chunk with K near its maximum, d just past a hidden tile, V below one
vocab tile).

The draws are fixed by the case number, so a failing case is reproduced by its id."""

import os

import numpy as np
import pytest
import torch

import datagen
import oracle
import lm_head_kl_amd as kd
from gpu_helpers import TOL, device_inputs, host, max_rel, rel_l2, say, lse_err, kl_input_bound, row_kl_err, assert_zk

pytestmark = pytest.mark.gpu

# More cases (new draws, same recipe) with KD_FUZZ_CASES=<n>.
N_CASES = int(os.environ.get("KD_FUZZ_CASES", "32"))


def draw_case(i: int) -> dict:
    g = np.random.Generator(np.random.PCG64([4242, i]))
    d = 8 * int(g.integers(1, 81))                        # 8 .. 648
    V = int(g.choice([int(g.integers(1, 256)), int(g.integers(256, 6000))]))
    kmax = min(V, 1024)
    K = int(g.choice([1, int(g.integers(1, kmax + 1)), kmax]))
    N = int(g.integers(1, 700))
    chunk = int(g.choice([1, int(g.integers(1, N + 1)), 64, 256, 512, 2048]))
    T = float(g.choice([0.5, 1.0, 1.7, 4.0]))
    teacher = str(g.choice(["normal", "peaked", "flat", "mix"]))
    # Zipf ids are drawn by rejection, so keep K well under V for them
    ids = str(g.choice(["uniform", "zipf", "mix"])) if 4 * K <= V else "uniform"
    dtype = str(g.choice(["fp32", "bf16"]))
    n_norm = float(g.choice([0.0, float(g.integers(1, 2 * N + 2))]))
    grad = float(g.choice([1.0, 0.37, -2.0]))
    return dict(N=N, d=d, V=V, K=K, chunk=chunk, T=T, teacher=teacher, ids=ids, dtype=dtype,
                n_norm=n_norm, grad=grad, seed=5000 + i)


def make_problem(c: dict) -> datagen.Problem:
    return datagen.make("tiny", N=c["N"], seed=c["seed"], d=c["d"], V=c["V"], K=c["K"], T=c["T"],
                        dtype=c["dtype"], chunk=c["chunk"], teacher=c["teacher"], ids=c["ids"])


def check(label, c, ref, loss, lse, row_kl, dH, dW=None, zk=None):
    tol = TOL[c["dtype"]]
    got = float(loss.item()) * c["grad"]  # the oracle's loss carries the upstream weight
    assert lse_err(host(lse), ref["lse"], c["T"]) <= tol["lse"], label
    if not np.any(ref["row_kl"]):
        # every KL_n is exactly 0 (V = 1): the loss is held to the bound its inputs carry
        ls = abs(c["grad"]) * c["T"] ** 2 / (c["n_norm"] or c["N"])
        assert abs(got) <= ls * kl_input_bound(ref, c["T"], tol["lse"]).sum(), (label, got)
    else:
        assert abs(got - ref["loss"]) <= tol["loss"] * abs(ref["loss"]), (label, got, ref["loss"])
    assert row_kl_err(host(row_kl), ref, c["T"], tol) <= 1.0, label
    if zk is not None:
        np.testing.assert_allclose(host(zk), ref["zk"], rtol=tol["lse"], atol=tol["lse"] * 4, err_msg=label)
    e_dh = rel_l2(host(dH), ref["dH"])
    e_dw = None if dW is None else rel_l2(host(dW), ref["dW"])
    say(f"  {label}: dH relL2 {e_dh:.2e}" + ("" if e_dw is None else f"  dW relL2 {e_dw:.2e}"))
    assert e_dh <= tol["grad"], label
    if e_dw is not None:
        assert e_dw <= tol["grad"], label


@pytest.mark.parametrize("i", range(N_CASES))
def test_fuzz_case(i):
    c = draw_case(i)
    say(f"fuzz case {i}:", {k: v for k, v in c.items()})
    p = make_problem(c)
    H, W, idx, t = device_inputs(p)
    nn = None if c["n_norm"] == 0.0 else c["n_norm"]
    ref = oracle.kl_chunked(p.f64("H"), p.f64("W"), p.idx, p.f64("tlog"), p.T, chunk=256, n_norm=nn, g=c["grad"])
    gt = torch.tensor(c["grad"], dtype=torch.float32, device=H.device)

    # the cache is sound: both forms of the id check pass it
    assert int(kd.validate_ids(idx, p.V).item()) == 0
    fv = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=c["chunk"], n_norm=c["n_norm"], flags=kd.KD_VALIDATE_IDX)

    # fused pair
    f = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=c["chunk"], n_norm=c["n_norm"], want_zk=True)
    dH, dW = kd.fused_kl_bwd(H, W, idx, t, f.lse, grad_loss=gt, T=p.T, chunk=c["chunk"], n_norm=c["n_norm"])
    torch.cuda.synchronize()
    check("fused", c, ref, f.loss, f.lse, f.row_kl, dH, dW, zk=f.zk)
    assert torch.equal(fv.lse, f.lse) and torch.equal(fv.loss, f.loss)

    # a second call gives the same bits (nothing depends on the plan's atomic fill order or on
    # which workgroup takes which tile)
    dH1, dW1 = kd.fused_kl_bwd(H, W, idx, t, f.lse, grad_loss=gt, T=p.T, chunk=c["chunk"], n_norm=c["n_norm"])
    torch.cuda.synchronize()
    assert torch.equal(dH1, dH) and torch.equal(dW1, dW), "the backward is not reproducible"

    # memory-lean backward (its own G_c layout and GEMM paths), against the oracle
    dHl, dWl = kd.fused_kl_bwd(H, W, idx, t, f.lse, grad_loss=gt, T=p.T, chunk=c["chunk"], n_norm=c["n_norm"],
                               flags=kd.KD_LOW_MEMORY)
    torch.cuda.synchronize()
    check("fused low-memory", c, ref, f.loss, f.lse, f.row_kl, dHl, dWl)

    # frozen head: the same dH, dW left alone
    dH2, none = kd.fused_kl_bwd(H, W, idx, t, f.lse, grad_loss=gt, T=p.T, chunk=c["chunk"], n_norm=c["n_norm"],
                                flags=kd.KD_SKIP_DW)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(dH2, dH), "frozen-head dH differs from the full backward's"

    # accumulate: a second backward added into the first dW doubles it, up to fp32 rounding of
    # the running sum where several dW passes add in turn
    dW_acc = dW.clone()
    kd.fused_kl_bwd(H, W, idx, t, f.lse, grad_loss=gt, T=p.T, chunk=c["chunk"], n_norm=c["n_norm"],
                    dW=dW_acc, flags=kd.KD_ACCUMULATE_DW)
    torch.cuda.synchronize()
    assert rel_l2(host(dW_acc), 2.0 * host(dW)) <= 1e-6, "accumulated dW is not twice the overwritten one"

    # the other three formulations
    for name, fn in (("chunked", kd.chunked_kl), ("fwdbwd", kd.fused_kl_fwdbwd)):
        loss, lse, row_kl, dHx, dWx = fn(H, W, idx, t, T=p.T, chunk=c["chunk"], grad_loss=gt, n_norm=c["n_norm"])
        torch.cuda.synchronize()
        check(name, c, ref, loss, lse, row_kl, dHx, dWx)
    loss, lse, row_kl, dHx, dWx = kd.dense_kl(H, W, idx, t, T=p.T, grad_loss=gt, n_norm=c["n_norm"])
    torch.cuda.synchronize()
    check("dense", c, ref, loss, lse, row_kl, dHx, dWx)


def test_fuzz_draws_cover_the_boundaries():
    """The fixed draws reach both dtypes, K = 1, K at min(V, 1024), V below one vocab tile,
    chunk = 1, and a non-default normaliser."""
    cs = [draw_case(i) for i in range(N_CASES)]
    assert {c["dtype"] for c in cs} == {"fp32", "bf16"}
    assert any(c["K"] == 1 for c in cs)
    assert any(c["K"] == min(c["V"], 1024) and c["K"] > 1 for c in cs)
    assert any(c["V"] < 256 for c in cs)
    assert any(c["chunk"] == 1 for c in cs)
    assert any(c["n_norm"] != 0.0 for c in cs)


# Medium shapes: more tiles than the chip has workgroup slots, so the persistent loops, the
# forward's vocabulary split and the dW chunk groups all take their general paths. Every row's
# lse, zk, KL_n and dH row is compared; dW on 64 vocabulary rows (ids 0-3, V-1 and seeded).
N_MEDIUM = int(os.environ.get("KD_FUZZ_MEDIUM", "6"))  # more with KD_FUZZ_MEDIUM=<n>


def draw_medium(i: int) -> dict:
    g = np.random.Generator(np.random.PCG64([4243, i]))
    N = int(g.integers(1000, 3000))
    d = 8 * int(g.integers(16, 97))                       # 128 .. 768
    V = int(g.integers(16000, 48000))
    K = int(g.choice([int(g.integers(1, 129)), int(g.integers(129, 1025))]))
    chunk = int(g.choice([int(g.integers(100, N)), 256, 512, 1024, 4096]))
    T = float(g.choice([0.5, 1.0, 2.0]))
    teacher = str(g.choice(["peaked", "flat", "mix"]))
    ids = str(g.choice(["uniform", "zipf", "mix"]))
    dtype = "fp32" if i % 3 == 2 else "bf16"
    return dict(N=N, d=d, V=V, K=K, chunk=chunk, T=T, teacher=teacher, ids=ids, dtype=dtype,
                n_norm=0.0, grad=1.0, seed=6000 + i)


@pytest.mark.parametrize("i", range(N_MEDIUM))
def test_fuzz_medium(i):
    c = draw_medium(i)
    say(f"medium case {i}:", {k: v for k, v in c.items()})
    p = make_problem(c)
    H, W, idx, t = device_inputs(p)
    tol = TOL[c["dtype"]]
    f = kd.fused_kl_fwd(H, W, idx, t, T=p.T, chunk=c["chunk"], want_zk=True)
    dH, dW = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=c["chunk"])
    torch.cuda.synchronize()
    Hf, Wf, tl = p.f64("H"), p.f64("W"), p.f64("tlog")
    ref = {k: [] for k in ("lse", "row_kl", "zk", "dH")}
    for r0 in range(0, p.N, 512):
        rows = np.arange(r0, min(p.N, r0 + 512))
        part = oracle.kl_rows(Hf, Wf, p.idx, tl, p.T, rows, n_norm=p.N)
        for k in ref:
            ref[k].append(part[k])
    ref = {k: np.concatenate(v) for k, v in ref.items()}
    loss = p.T * p.T / p.N * float(np.sum(ref["row_kl"]))
    assert abs(f.loss.item() - loss) <= tol["loss"] * abs(loss)
    assert lse_err(host(f.lse), ref["lse"], p.T) <= tol["lse"]
    assert row_kl_err(host(f.row_kl), ref, p.T, tol) <= 1.0
    assert_zk(host(f.zk), ref["zk"], tol["lse"], Hf, Wf, p.idx)
    e_dh = rel_l2(host(dH), ref["dH"])
    vocab = datagen.sample_vocab(p.V, 64, c["seed"])
    want = oracle.dw_rows(Hf, Wf, p.idx, tl, p.T, vocab, ref["lse"], n_norm=p.N)
    e_dw = rel_l2(host(dW[torch.from_numpy(vocab).to(dW.device)]), want)
    say(f"  dH relL2 {e_dh:.2e}  dW rows relL2 {e_dw:.2e}")
    assert e_dh <= tol["grad"] and e_dw <= tol["grad"]
    # the memory-lean backward on the same shapes
    dHl, dWl = kd.fused_kl_bwd(H, W, idx, t, f.lse, T=p.T, chunk=c["chunk"], flags=kd.KD_LOW_MEMORY)
    torch.cuda.synchronize()
    e_dh = rel_l2(host(dHl), ref["dH"])
    e_dw = rel_l2(host(dWl[torch.from_numpy(vocab).to(dWl.device)]), want)
    say(f"  low-memory: dH relL2 {e_dh:.2e}  dW rows relL2 {e_dw:.2e}")
    assert e_dh <= tol["grad"] and e_dw <= tol["grad"]
