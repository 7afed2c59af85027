"""Writes topk_truncation_study.json: the top-K truncation study on synthetic teachers.

For 64 peaked and 64 flat full-vocabulary teacher rows at V = 201,088 (the gpt-oss-120b
vocabulary) and a random student head (d = 256, z ~ N(0, 1)), it records what caching only the
top K teacher logits changes, for K in {10, 50, 100, 500}: the kept teacher mass, the loss
against the whole teacher and against the cached one, and the relative error of the logit
gradient. Every number comes from oracle.truncation_terms; inputs from datagen.

The study quantifies the restriction the pages name (the top-K approximation drops the tail;
harmless for peaked positions, lossy where the mass is spread over hundreds of candidates):
"Making knowledge distillation cheap enough to run in production", paragraph on the remaining
restriction. No dataset or teacher model is involved.

Run from the repository root: python tests/golden/make_truncation_study.py
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import datagen  # noqa: E402
import oracle  # noqa: E402

V, D, ROWS, T, SEED = 201088, 256, 64, 1.0, 2024
KS = (10, 50, 100, 500)


def student(seed):
    H = datagen.normal_rows(ROWS, D, 1.0, seed, 0, dtype="fp32")
    W = datagen.normal_rows(V, D, 1.0 / np.sqrt(D), seed, 1, dtype="fp32")
    return H, W


def main():
    out = {"V": V, "d": D, "rows_per_kind": ROWS, "T": T, "seed": SEED, "K": list(KS), "kinds": {},
           "source": "oracle.truncation_terms on datagen.full_teacher_logits and datagen.normal_rows"}
    for kind in ("peaked", "flat"):
        H, W = student(SEED)
        t = datagen.full_teacher_logits(kind, ROWS, V, SEED)
        per = {}
        for K in KS:
            r = oracle.truncation_terms(H, W, t, K, T)
            per[str(K)] = {
                "mass_mean": float(r["mass"].mean()),
                "mass_min": float(r["mass"].min()),
                "kl_full_mean": float(r["kl_full"].mean()),
                "kl_topk_mean": float(r["kl_topk"].mean()),
                "kl_rel_gap_mean": float(np.mean(np.abs(r["kl_topk"] - r["kl_full"]) / r["kl_full"])),
                "grad_rel_mean": float(r["grad_rel"].mean()),
                "grad_rel_max": float(r["grad_rel"].max()),
                "kl_topk_rows": [float(x) for x in r["kl_topk"]],
            }
            print(kind, K, {k: round(v, 6) for k, v in per[str(K)].items() if k != "kl_topk_rows"}, flush=True)
        out["kinds"][kind] = per
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "topk_truncation_study.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
