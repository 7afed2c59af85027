"""Writes <config>_lse.npy: the fp64 log-sum-exp of z/T for every row of a large workload
(seeded inputs from datagen), computed by oracle.lse_all_rows. Configs: "gptoss" (N = 32768)
and "full" (the pages' shape, N = 131072), both at d = 2880, V = 201,088, T = 1; "qwen"
(N = 8192, d = 2048, V = 151,936, T = 2).

With it, a GPU test checks the full-batch lse of the fused forward at every row and derives
sampled rows of the full-batch dW on the host (oracle.dw_rows needs every row's lse, which
takes minutes of fp64 matrix products and so is stored here instead of recomputed).

Run from the repository root: python tests/golden/make_lse.py gptoss full qwen
"""

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import datagen  # noqa: E402
import oracle  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def main(names):
    for name in names:
        p = datagen.make(name)
        t0 = time.time()
        lse = oracle.lse_all_rows(p.f32("H"), p.f64("W"), p.T, block=512)
        out = os.path.join(HERE, f"{name}_lse.npy")
        np.save(out, lse.astype(np.float64))
        print(f"wrote {out}: {lse.shape[0]} rows (config seed {p.extra['seed']}), {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["gptoss", "full", "qwen"])
