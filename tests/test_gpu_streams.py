"""The library keeps no state between calls and enqueues nothing but kernel launches, so
(1) calls on different streams with their own buffers may overlap and give exactly the
results they give alone, and (2) a fused forward + backward can be captured into a HIP graph
and replayed. Both are compared bit for bit with eager calls (the path is deterministic)."""

import numpy as np
import pytest
import torch

import datagen
import lm_head_kl_amd as kd
from gpu_helpers import device_inputs, say, to_torch

pytestmark = pytest.mark.gpu

CHUNK = 512


def bits(x: torch.Tensor) -> torch.Tensor:
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


def same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return a.shape == b.shape and a.dtype == b.dtype and torch.equal(bits(a), bits(b))


class Step:
    """One fused forward + backward with every buffer allocated up front."""

    def __init__(self, p: datagen.Problem):
        self.p = p
        self.H, self.W, self.idx, self.t = device_inputs(p)
        prob = kd.make_problem(self.H, self.W, self.idx, self.t, p.T, CHUNK)
        self.ws = torch.empty(kd.fused_workspace_bytes(prob), dtype=torch.uint8, device=self.H.device)
        self.dW = torch.empty(self.W.shape, dtype=torch.float32, device=self.H.device)

    def __call__(self):
        f = kd.fused_kl_fwd(self.H, self.W, self.idx, self.t, T=self.p.T, chunk=CHUNK, want_zk=True,
                            workspace=self.ws)
        dH, dW = kd.fused_kl_bwd(self.H, self.W, self.idx, self.t, f.lse, T=self.p.T, chunk=CHUNK, dW=self.dW,
                                 workspace=self.ws)
        return [f.loss, f.lse, f.row_kl, f.zk, dH, dW]


def snapshot(outs):
    return [o.clone() for o in outs]


def test_concurrent_streams_match_sequential():
    say("two problems on two streams at once vs one at a time")
    a = Step(datagen.make("small", N=1536))
    b = Step(datagen.make("small", N=1024, seed=77))
    ref_a = snapshot(a())
    torch.cuda.synchronize()
    ref_b = snapshot(b())
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        with torch.cuda.stream(s1):
            out_a = a()
        with torch.cuda.stream(s2):
            out_b = b()
        torch.cuda.synchronize()
        for x, y in zip(out_a, ref_a):
            assert same(x, y), f"stream 1, repeat {rep}"
        for x, y in zip(out_b, ref_b):
            assert same(x, y), f"stream 2, repeat {rep}"


def make_case(case: str, seed: int | None = None) -> datagen.Problem:
    if case == "small":
        return datagen.make("small", N=1024, seed=seed)
    # 8448 rows: the calls copy W and H into the stage-tiled layout first
    return datagen.make("tiny", N=8448, d=264, V=3000, dtype="bf16", seed=seed)


@pytest.mark.parametrize("case", ["small", "tiled"])
def test_graph_capture_and_replay(case):
    say("fused forward + backward captured into a HIP graph, replayed", case)
    p = make_case(case)
    st = Step(p)
    eager = snapshot(st())
    torch.cuda.synchronize()
    # warm up on a side stream, as torch asks before a capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        static_out = st()
    other = Step(datagen.make("small", N=512, seed=5))
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(static_out, eager):
            assert same(x, y), f"replay {rep}"
        other()  # eager work of the program between replays
        torch.cuda.synchronize()
    # the graph reads its input buffers at replay: new values in place give the new results
    p2 = make_case(case, seed=99)
    st.H.copy_(to_torch(p2.H))
    st.t.copy_(to_torch(p2.tlog))
    st.idx.copy_(torch.from_numpy(p2.idx))
    g.replay()
    torch.cuda.synchronize()
    got = snapshot(static_out)
    fresh = Step(p2)
    fresh.W.copy_(st.W)
    want = fresh()
    torch.cuda.synchronize()
    for x, y in zip(got, want):
        assert same(x, y), "replay on new inputs"
    assert not same(got[1], eager[1])


def _timed(fn):
    kd.timing_reset()
    kd.timing_enable(True)
    try:
        fn()
        torch.cuda.synchronize()
        return kd.timing_read()
    finally:
        kd.timing_enable(False)
        kd.timing_reset()


def test_timing_counts_launches_per_kind():
    """The per-kernel HIP-event timing counts each launch of a fused forward + backward once:
    one forward, and per 512-row chunk one gradient tile and one dH, one dW pass per four chunks."""
    say("per-kernel timing, one thread")
    st = Step(datagen.make("small", N=2048))  # 4 chunks of 512
    k = _timed(st)
    assert k["fwd"][0] == 1 and k["combine"][0] == 1
    assert k["bwd_grad"][0] == 4 and k["dh"][0] == 4 and k["dw"][0] == 1
    assert all(ms > 0.0 for _, ms in k.values())


def test_timing_from_two_threads():
    """Two threads calling the library at once, each on its own stream, with timing on: every
    launch is counted once (each thread brackets its own launches)."""
    import threading

    say("per-kernel timing, two threads on two streams")
    steps = [Step(datagen.make("small", N=2048)), Step(datagen.make("small", N=1024, seed=3))]
    torch.cuda.synchronize()
    errors = []

    def work(st):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    st()
            s.synchronize()
        except Exception as e:  # surfaced below
            errors.append(e)

    def both():
        th = [threading.Thread(target=work, args=(st,)) for st in steps]
        for x in th:
            x.start()
        for x in th:
            x.join()

    k = _timed(both)
    assert not errors, errors
    # 3 calls each: 4 + 2 chunks of 512 per call pair
    assert k["fwd"][0] == 6
    assert k["bwd_grad"][0] == 3 * (4 + 2) and k["dh"][0] == 3 * (4 + 2)
    assert k["dw"][0] == 6


@pytest.mark.parametrize("path", ["chunked", "fwdbwd", "topk"])
def test_other_calls_capture_and_replay(path):
    """The forward-chunked and single-pass calls and the top-K producer enqueue kernels only as
    well: captured into a graph, each of three replays (with eager library calls between them)
    gives the eager result bit for bit."""
    say("graph capture", path)
    p = datagen.make("small", N=1024, seed=21)
    H, W, idx, t = device_inputs(p)
    if path == "topk":
        logits = (H[:256].float() @ W.float().t()).to(torch.bfloat16).contiguous()

        def call():
            return list(kd.topk_cache(logits, 100))
    else:
        fn = kd.chunked_kl if path == "chunked" else kd.fused_kl_fwdbwd
        prob = kd.make_problem(H, W, idx, t, p.T, CHUNK)
        nb = (kd.chunked_workspace_bytes if path == "chunked" else kd.fused_fwdbwd_workspace_bytes)(prob)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        dW = torch.empty(W.shape, dtype=torch.float32, device="cuda")

        def call():
            return list(fn(H, W, idx, t, T=p.T, chunk=CHUNK, dW=dW, workspace=ws))
    eager = snapshot(call())
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        static_out = call()
    other = Step(datagen.make("small", N=512, seed=5))
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(static_out, eager):
            assert same(x, y), f"{path} replay {rep}"
        other()
        torch.cuda.synchronize()
