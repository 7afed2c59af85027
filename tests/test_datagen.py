"""The seeded input generators: shapes, ranges, distinct ids, determinism and the
distributions the workloads are meant to have (CPU only)."""

import json
import os

import numpy as np
import pytest

import datagen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rounding():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e-3, 65504.0], np.float32)
    b = datagen.bf16_bits(x)
    back = datagen.bf16_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to even (1.0)
    assert back[0] == 1.0 and back[1] == 1.0
    assert back[2] == np.float32(1.0078125)
    assert back[3] == -2.5
    assert abs(back[4] - 3.0e-3) <= 2 ** -8 * 3.0e-3  # half an ulp of an 8-bit significand
    assert np.all(datagen.bf16_to_f32(datagen.bf16_bits(back)) == back)


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_shapes_and_ids(name):
    p = datagen.make(name)
    assert p.H.shape == (p.N, p.d) and p.W.shape == (p.V, p.d)
    assert p.idx.shape == (p.N, p.K) and p.tlog.shape == (p.N, p.K)
    assert p.idx.dtype == np.int32
    assert p.idx.min() >= 0 and p.idx.max() < p.V
    s = np.sort(p.idx, axis=1)
    assert not np.any(s[:, 1:] == s[:, :-1])
    t = p.f64("tlog")
    assert np.all(np.diff(t, axis=1) <= 0)  # sorted descending


def test_deterministic_and_prefix_stable():
    a = datagen.make("small")
    b = datagen.make("small", N=300)
    np.testing.assert_array_equal(a.H[:300], b.H)
    np.testing.assert_array_equal(a.idx[:300], b.idx)
    np.testing.assert_array_equal(a.tlog[:300], b.tlog)
    np.testing.assert_array_equal(a.W, b.W)
    c = datagen.make("small", seed=5)
    assert not np.array_equal(a.H, c.H)


def test_peaked_rows_top1_is_0p6():
    p = datagen.make("small", N=2048)
    t = p.f64("tlog") / p.T
    pt = np.exp(t - t.max(1, keepdims=True))
    pt /= pt.sum(1, keepdims=True)
    # exact 0.6 before bf16 rounding of the stored logits
    assert abs(pt[:, 0].mean() - 0.6) < 0.01
    assert np.all(np.abs(pt[:, 0] - 0.6) < 0.05)


def test_flat_rows_spread_mass():
    p = datagen.make("qwen", N=1024)
    t = p.f64("tlog") / p.T
    pt = np.exp(t - t.max(1, keepdims=True))
    pt /= pt.sum(1, keepdims=True)
    assert pt.max(1).mean() < 0.05


def test_zipf_rank_frequency_slope():
    """log-frequency vs log-rank of drawn ids has slope about -1.1 on the head ranks
    (without replacement flattens the very top, so fit ranks 20..2000)."""
    g = np.random.Generator(np.random.PCG64(3))
    ids = datagen.zipf_distinct(4000, 1, 32000, g)  # K = 1: plain Zipf draws
    cnt = np.bincount(ids[:, 0], minlength=32000).astype(float)
    g2 = np.random.Generator(np.random.PCG64(4))
    more = datagen.zipf_distinct(200000, 1, 32000, g2)[:, 0]
    cnt += np.bincount(more, minlength=32000)
    r = np.arange(20, 2000)
    y = np.log(cnt[r - 1] + 0.5)
    slope = np.polyfit(np.log(r), y, 1)[0]
    assert -1.25 < slope < -0.95


def test_mix_rows_and_uniform_ids():
    p = datagen.make("gptoss", N=4096, V=201088)
    assert 0.45 < p.peaked.mean() < 0.55
    flat_ids = p.idx[~p.peaked]
    # uniform ids: mean near V/2; Zipf ids: heavily skewed to small ids
    assert abs(flat_ids.mean() / p.V - 0.5) < 0.02
    assert np.median(p.idx[p.peaked]) < 2000


def test_sampled_rows_and_vocab():
    r = datagen.sample_rows(131072, 256, 1004)
    assert len(np.unique(r)) == 256 and r.max() < 131072
    v = datagen.sample_vocab(201088, 256, 1004)
    assert len(np.unique(v)) == 256
    assert {0, 1, 2, 3, 201087} <= set(v.tolist())


def test_pages_workload_shape():
    """The gpt-oss-120b workload the pages print (vocabulary, sequence length, batch, K) and
    their byte accounting for the dense bf16 teacher tensor."""
    with open(os.path.join(GOLDEN, "pages_workload.json")) as f:
        gold = json.load(f)
    cfg = datagen.CONFIGS["full"]
    assert cfg["V"] == gold["vocab"] and cfg["S"] == gold["seq_len"] and cfg["B"] == gold["batch"]
    assert cfg["K"] == gold["top_k"]
    dense_bytes = gold["batch"] * gold["vocab"] * gold["seq_len"] * 2
    assert abs(dense_bytes / 1e9 - gold["dense_teacher_gb_bf16"]) / gold["dense_teacher_gb_bf16"] < 0.1
    g2 = datagen.CONFIGS["gptoss"]
    assert g2["V"] == gold["vocab"] and g2["S"] == gold["seq_len"]



def test_truncation_study_fixture():
    """The committed study shows the restriction the pages describe: for peaked teachers the
    top-100 cache keeps nearly all of the mass and moves the loss and gradient by a few percent;
    for flat teachers it keeps a fraction of a percent and the gradient is dominated by the
    truncation. More cached entries always help."""
    import json
    st = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "topk_truncation_study.json")))
    pk, fl = st["kinds"]["peaked"], st["kinds"]["flat"]
    assert pk["100"]["mass_mean"] > 0.95 and pk["100"]["grad_rel_mean"] < 0.05
    assert fl["100"]["mass_mean"] < 0.01 and fl["100"]["grad_rel_mean"] > 1.0
    for kind in (pk, fl):
        g = [kind[str(k)]["grad_rel_mean"] for k in st["K"]]
        m = [kind[str(k)]["mass_mean"] for k in st["K"]]
        assert all(a > b for a, b in zip(g, g[1:])) and all(a < b for a, b in zip(m, m[1:]))
