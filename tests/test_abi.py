"""The C ABI of libkdkl without a GPU: symbols, status strings, workspace queries, and the
host-side argument checks that must reject bad calls before anything is enqueued."""

import ctypes
import os
import re
import subprocess

import pytest

from lm_head_kl_amd import _lib
from lm_head_kl_amd._lib import KD_BF16, KD_FP32, KdProblem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kdkl.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libkdkl.so not built")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kd_[a-z_0-9]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert header_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for fn in header_functions():
        assert fn in exported, fn
    L = _lib.lib()
    for fn in header_functions():
        assert hasattr(L, fn)


def test_abi_version_matches_header():
    v = int(re.search(r"#define KDKL_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert _lib.lib().kd_abi_version() == v


def test_status_strings():
    L = _lib.lib()
    for code in range(0, 9):
        s = L.kd_status_str(code)
        assert s and len(s) > 1
    assert L.kd_status_str(99) == b"unknown status"


def prob(**kw):
    base = dict(N=4096, d=1024, V=32000, K=100, chunk=1024, T=1.0, n_norm=0.0, act=KD_BF16, tlogit=KD_BF16,
                flags=0, reserved=0)
    base.update(kw)
    return KdProblem(**base)


def ws_bytes(**kw):
    return _lib.lib().kd_fused_workspace_bytes(ctypes.byref(prob(**kw)))


def test_workspace_queries():
    L = _lib.lib()
    assert ws_bytes() > 0
    assert L.kd_fused_workspace_bytes(None) == 0
    assert ws_bytes(K=0) == 0 and ws_bytes(T=-1.0) == 0
    # The gradient tile grows with chunk ...
    sizes = [ws_bytes(chunk=c) for c in (256, 512, 1024, 2048, 4096)]
    assert all(a < b for a, b in zip(sizes, sizes[1:]))
    # ... and is at least chunk x V in the activation dtype.
    assert ws_bytes(chunk=2048) >= 2048 * 32000 * 2
    # N enters only through O(N*K) and O(N) terms: second differences vanish once N > chunk.
    a, b, c = (ws_bytes(N=n, chunk=1024) for n in (8192, 16384, 24576))
    assert abs((c - b) - (b - a)) <= 4096
    per_row = (b - a) / 8192
    assert per_row < 100 * 4 * 3 + 64  # a few words per cached entry, nothing per vocab entry
    # Dense: two fp32 N x V grids.
    dn = L.kd_dense_workspace_bytes(ctypes.byref(prob(N=512)))
    assert dn >= 2 * 512 * 32000 * 4


def test_stored_logit_workspaces():
    """The forward-chunked path keeps every logit, so its workspace grows by at least 4 V bytes
    per row; the single-pass path keeps one chunk's logits, so N enters only through O(N*K)."""
    L = _lib.lib()

    def ch(**kw):
        return L.kd_chunked_workspace_bytes(ctypes.byref(prob(**kw)))

    def sp(**kw):
        return L.kd_fused_fwdbwd_workspace_bytes(ctypes.byref(prob(**kw)))

    assert L.kd_chunked_workspace_bytes(None) == 0 and L.kd_fused_fwdbwd_workspace_bytes(None) == 0
    assert ch(K=0) == 0 and sp(T=0.0) == 0
    a, b = ch(N=8192), ch(N=16384)
    assert b - a >= 8192 * 32000 * 4
    a, b, c = (sp(N=n, chunk=1024) for n in (8192, 16384, 24576))
    assert abs((c - b) - (b - a)) <= 4096 and (b - a) / 8192 < 100 * 4 * 4 + 64
    # one chunk of fp32 logits: each further row of chunk adds at least 4 V bytes
    assert sp(chunk=2048) - sp(chunk=1024) >= 1024 * 32000 * 4


# ------------------------------------------------------------------ argument checks
# These pass fake device addresses; the checks must reject the call before any launch.
# They are skipped where a GPU is visible, so that a checking bug can never turn into a
# kernel launch on made-up pointers.

nogpu = pytest.mark.skipif(
    __import__("torch").cuda.is_available(), reason="fake pointers are only passed when no GPU is visible")

F = ctypes.c_void_p(0x10000)  # 16- and 256-byte aligned, never dereferenced


def fwd(p, H=F, W=F, idx=F, t=F, loss=F, lse=F, ws=F, nbytes=None):
    L = _lib.lib()
    if nbytes is None:
        nbytes = max(1, L.kd_fused_workspace_bytes(ctypes.byref(p)))
    return L.kd_fused_kl_fwd(ctypes.byref(p), H, W, idx, t, loss, lse, None, None, ws, nbytes, None)


def bwd(p, H=F, W=F, idx=F, t=F, lse=F, dH=F, dW=F, ws=F, nbytes=None):
    L = _lib.lib()
    if nbytes is None:
        nbytes = max(1, L.kd_fused_workspace_bytes(ctypes.byref(p)))
    return L.kd_fused_kl_bwd(ctypes.byref(p), H, W, idx, t, lse, None, dH, dW, ws, nbytes, None)


def dense(p, H=F, dH=F, ws=F, nbytes=None):
    L = _lib.lib()
    if nbytes is None:
        nbytes = max(1, L.kd_dense_workspace_bytes(ctypes.byref(p)))
    return L.kd_dense_kl(ctypes.byref(p), H, F, F, F, None, F, F, None, dH, F, ws, nbytes, None)


@nogpu
@pytest.mark.parametrize("bad,code", [
    (dict(N=0), 2), (dict(d=0), 2), (dict(d=12), 2), (dict(V=0), 2), (dict(K=0), 2), (dict(K=1025, V=4000), 2),
    (dict(V=50, K=60), 2), (dict(chunk=0), 2), (dict(V=256 * 16384 + 1), 2), (dict(N=1 << 30, d=8), 2),
    (dict(d=(1 << 20) + 8, V=1000, N=1000), 2),
    (dict(act=2), 3), (dict(tlogit=-1), 3),
    (dict(T=0.0), 4), (dict(T=-1.0), 4), (dict(T=float("nan")), 4), (dict(T=float("inf")), 4),
    (dict(n_norm=float("nan")), 4), (dict(flags=16), 4), (dict(reserved=1), 4),
])
def test_bad_problem_rejected(bad, code):
    p = prob(**bad)
    assert fwd(p) == code
    assert bwd(p) == code
    assert dense(p) == code


@nogpu
def test_null_pointers_rejected():
    p = prob()
    L = _lib.lib()
    assert L.kd_fused_kl_fwd(None, F, F, F, F, F, F, None, None, F, 1 << 40, None) == 1
    for kw in ("H", "W", "idx", "t", "loss", "lse", "ws"):
        assert fwd(p, **{kw: None}) == 1, kw
    for kw in ("H", "W", "idx", "t", "lse", "dH", "dW", "ws"):
        assert bwd(p, **{kw: None}) == 1, kw
    assert dense(p, H=None) == 1 and dense(p, dH=None) == 1


@nogpu
def test_workspace_and_alignment_rejected():
    p = prob()
    need = ws_bytes()
    assert fwd(p, nbytes=need - 1) == 5
    assert bwd(p, nbytes=need - 1) == 5
    assert fwd(p, ws=ctypes.c_void_p(0x10000 + 128)) == 5  # not 256-byte aligned
    assert fwd(p, H=ctypes.c_void_p(0x10008)) == 4          # vector loads need 16-byte alignment
    assert bwd(p, dH=ctypes.c_void_p(0x10004)) == 4
    assert bwd(p, dW=ctypes.c_void_p(0x10008)) == 4
    dn = _lib.lib().kd_dense_workspace_bytes(ctypes.byref(p))
    assert dense(p, nbytes=dn - 1) == 5


def test_fp32_problem_is_valid():
    assert ws_bytes(act=KD_FP32, tlogit=KD_FP32, d=128, V=2048, K=16, N=256, chunk=64) > 0


@nogpu
@pytest.mark.parametrize("args,code", [
    (dict(logits=None), 1), (dict(idx=None), 1), (dict(values=None), 1),
    (dict(dtype=2), 3),
    (dict(N=0), 2), (dict(V=0), 2), (dict(K=0), 2), (dict(K=1025, V=2000), 2), (dict(K=11, V=10), 2),
    (dict(V=(1 << 22) + 1), 2), (dict(ld=99), 2),
])
def test_topk_bad_arguments(args, code):
    a = dict(logits=F, dtype=KD_BF16, N=4, V=100, ld=100, K=10, idx=F, values=F)
    a.update(args)
    L = _lib.lib()
    assert L.kd_topk_cache(a["logits"], a["dtype"], a["N"], a["V"], a["ld"], a["K"], a["idx"], a["values"],
                           None) == code


@nogpu
def test_skip_dw_flag_rules():
    """KD_SKIP_DW: only the fused backward may leave dW out; with KD_ACCUMULATE_DW it is
    rejected by every call; without it the fused backward still needs dW."""
    L = _lib.lib()
    both = prob(flags=_lib.KD_SKIP_DW | _lib.KD_ACCUMULATE_DW)
    assert fwd(both) == 4 and bwd(both) == 4 and dense(both) == 4
    p = prob(flags=_lib.KD_SKIP_DW)
    assert dense(p) == 4
    for fn, query in (("kd_chunked_kl", "kd_chunked_workspace_bytes"),
                      ("kd_fused_kl_fwdbwd", "kd_fused_fwdbwd_workspace_bytes")):
        nb = max(1, getattr(L, query)(ctypes.byref(p)))
        assert getattr(L, fn)(ctypes.byref(p), F, F, F, F, None, F, F, None, F, F, F, nb, None) == 4
    assert bwd(prob(), dW=None) == 1


def test_low_memory_workspace():
    """KD_LOW_MEMORY drops the transposed copies of W, G_c and H_c from the fused backward's
    workspace: what is left is about the gradient tile G_c plus the dH partials and the
    O(N*K) cache terms. The forward's part is unchanged."""
    d, V, C = 2880, 201088, 2048
    full = ws_bytes(N=32768, d=d, V=V, chunk=C)
    lean = ws_bytes(N=32768, d=d, V=V, chunk=C, flags=_lib.KD_LOW_MEMORY)
    vp = (V + 255) // 256 * 256
    gc = C * vp * 2
    assert gc <= lean < gc + 8 * C * d * 4 + 32768 * 100 * 12 + (1 << 24)
    # the default adds W^T (V*d) and a four-chunk G^T slab (4*C*V) in bf16
    assert full - lean >= (vp * d + 4 * C * vp) * 2
    # N still enters only through O(N*K) terms
    a, b, c = (ws_bytes(N=n, chunk=1024, flags=_lib.KD_LOW_MEMORY) for n in (8192, 16384, 24576))
    assert abs((c - b) - (b - a)) <= 4096 and (b - a) / 8192 < 100 * 4 * 3 + 64


@nogpu
def test_wide_dh_vocabulary_limit():
    """The backward paths that read W^T stage-tiled in 320-row blocks stop where its last stage
    would leave a buffer descriptor's 32-bit range: V = 3,355,392 in bf16, 1,677,568 in fp32
    (KD_ERR_SHAPE before anything is enqueued); the memory-lean backward and the forward go on,
    the bf16 memory-lean backward up to V = 4,194,048."""
    L = _lib.lib()
    for act, vmax in ((KD_BF16, 3355392), (KD_FP32, 1677568)):
        for V, ok in ((vmax, True), (vmax + 256, False)):
            p = prob(N=256, d=8, V=V, K=4, chunk=256, act=act, tlogit=act)
            code = bwd(p, nbytes=1)  # too small a workspace: past the shape check it is error 5
            assert code == (5 if ok else 2), (act, V, code)
            for fn in ("kd_chunked_kl", "kd_fused_kl_fwdbwd"):
                assert (getattr(L, fn)(ctypes.byref(p), F, F, F, F, None, F, F, None, F, F, F, 1, None)
                        == (5 if ok else 2)), (fn, act, V)
            lean = prob(N=256, d=8, V=V, K=4, chunk=256, act=act, tlogit=act, flags=_lib.KD_LOW_MEMORY)
            assert bwd(lean, nbytes=1) == 5
            assert fwd(p, nbytes=1) == 5
    # the bf16 memory-lean backward reads its stage-tiled G_c (256-row blocks) the same way: up to
    # V = 4,194,048; fp32 goes on to the largest vocabulary the calls take
    for act, V, ok in ((KD_BF16, 4194048, True), (KD_BF16, 4194304, False), (KD_FP32, 4194304, True)):
        lean = prob(N=256, d=8, V=V, K=4, chunk=256, act=act, tlogit=act, flags=_lib.KD_LOW_MEMORY)
        assert bwd(lean, nbytes=1) == (5 if ok else 2), (act, V)


@nogpu
def test_low_memory_flag_rules():
    """KD_LOW_MEMORY belongs to the fused calls; the other loss calls reject it."""
    L = _lib.lib()
    p = prob(flags=_lib.KD_LOW_MEMORY)
    assert dense(p) == 4
    for fn, query in (("kd_chunked_kl", "kd_chunked_workspace_bytes"),
                      ("kd_fused_kl_fwdbwd", "kd_fused_fwdbwd_workspace_bytes")):
        nb = max(1, getattr(L, query)(ctypes.byref(p)))
        assert getattr(L, fn)(ctypes.byref(p), F, F, F, F, None, F, F, None, F, F, F, nb, None) == 4
    # a workspace sized for the lean backward is too small for the default one
    lean = L.kd_fused_workspace_bytes(ctypes.byref(p))
    assert bwd(prob(), nbytes=lean) == 5


def test_chunked_logits_view():
    """kd_chunked_logits is host-only: it places z^T [Vp][ldzt] fp32 inside the workspace and
    checks its arguments like the loss call."""
    L = _lib.lib()
    p = prob(N=1000, d=64, V=3000, K=10, chunk=256)
    need = L.kd_chunked_workspace_bytes(ctypes.byref(p))
    base = 0x100000
    zp, ld = ctypes.c_void_p(0), ctypes.c_int64(0)
    assert L.kd_chunked_logits(ctypes.byref(p), ctypes.c_void_p(base), need, ctypes.byref(zp), ctypes.byref(ld)) == 0
    assert ld.value >= 1000 and ld.value % 4 == 0
    off = zp.value - base
    assert off % 256 == 0 and off + 3072 * ld.value * 4 <= need
    assert L.kd_chunked_logits(ctypes.byref(p), ctypes.c_void_p(base), need - 1, ctypes.byref(zp),
                               ctypes.byref(ld)) == 5
    assert L.kd_chunked_logits(ctypes.byref(p), None, need, ctypes.byref(zp), ctypes.byref(ld)) == 1
    assert L.kd_chunked_logits(ctypes.byref(prob(K=0)), ctypes.c_void_p(base), need, ctypes.byref(zp),
                               ctypes.byref(ld)) == 2


@pytest.mark.parametrize("K", [0, -3, 11, 2000])
def test_topk_binding_checks_k(K):
    """The binding rejects K outside 1 .. min(V, 1024) before it allocates or calls anything."""
    import torch

    import lm_head_kl_amd as kd

    with pytest.raises(kd.KdError) as e:
        kd.topk_cache(torch.zeros((4, 10)), K)
    assert e.value.code == 2


def test_chunk_is_capped_at_2_20_rows():
    """Chunks longer than 2^20 rows are taken as 2^20 (the dW product's chunk-strided operands
    stay within 32-bit buffer offsets): the workspace stops growing there."""
    big = dict(N=1 << 22, d=8, V=256, K=1)
    a = ws_bytes(chunk=1 << 20, **big)
    assert a > 0
    assert ws_bytes(chunk=(1 << 20) + 1, **big) == a
    assert ws_bytes(chunk=1 << 22, **big) == a
    assert ws_bytes(chunk=(1 << 20) - 8, **big) < a


@nogpu
def test_dense_vocabulary_limit():
    """The dense path reads 256-row tiles of grids whose rows are 4 * Vp bytes through 32-bit
    buffer offsets, so it stops at V = 2^21; the fused calls take the full range."""
    L = _lib.lib()
    ok, over = prob(N=8, d=8, V=1 << 21, K=4), prob(N=8, d=8, V=(1 << 21) + 1, K=4)
    assert L.kd_dense_workspace_bytes(ctypes.byref(ok)) > 0
    assert L.kd_dense_workspace_bytes(ctypes.byref(over)) == 0
    assert dense(over) == 2
    assert ws_bytes(N=8, d=8, V=(1 << 21) + 1, K=4) > 0


@nogpu
@pytest.mark.parametrize("args,code", [
    (dict(idx=None), 1), (dict(status=None), 1),
    (dict(N=0), 2), (dict(K=0), 2), (dict(K=1025), 2), (dict(V=0), 2), (dict(N=1 << 31), 2),
])
def test_validate_ids_bad_arguments(args, code):
    a = dict(idx=F, N=4, K=10, V=100, status=F)
    a.update(args)
    assert _lib.lib().kd_validate_ids(a["idx"], a["N"], a["K"], a["V"], a["status"], None) == code
