"""The top-K truncation study on the GPU path: the library's cache producer and fused loss give
the per-row losses against the cached teacher that the oracle recorded in
tests/golden/topk_truncation_study.json (written by make_truncation_study.py), for peaked and
flat teachers at V = 201,088 and K in {10, 50, 100, 500}."""

import json
import os

import numpy as np
import pytest
import torch

import datagen
import oracle
import lm_head_kl_amd as kd
from gpu_helpers import say, to_torch

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "topk_truncation_study.json")


@pytest.mark.parametrize("kind", ["peaked", "flat"])
def test_truncation_study_on_gpu(kind):
    st = json.load(open(GOLD))
    V, D, R, T, seed = st["V"], st["d"], st["rows_per_kind"], st["T"], st["seed"]
    say("truncation study", kind, f"rows={R} V={V} d={D}")
    H = datagen.normal_rows(R, D, 1.0, seed, 0, dtype="fp32")
    W = datagen.normal_rows(V, D, 1.0 / np.sqrt(D), seed, 1, dtype="fp32")
    t = datagen.full_teacher_logits(kind, R, V, seed)
    Hd, Wd, td = to_torch(H), to_torch(W), to_torch(t)
    for K in st["K"]:
        idx, vals = kd.topk_cache(td, K)
        f = kd.fused_kl_fwd(Hd, Wd, idx, vals, T=T, chunk=R)
        torch.cuda.synchronize()
        want_idx, _ = oracle.topk_cache(t, K)
        assert np.array_equal(idx.cpu().numpy(), want_idx)
        got = f.row_kl.cpu().numpy().astype(np.float64)
        ref = np.array(st["kinds"][kind][str(K)]["kl_topk_rows"])
        say(f"  K={K} max rel {np.max(np.abs(got - ref) / np.abs(ref)):.2e}")
        np.testing.assert_allclose(got, ref, rtol=1e-5)
        assert abs(got.mean() - ref.mean()) <= 1e-6 * abs(ref.mean())
