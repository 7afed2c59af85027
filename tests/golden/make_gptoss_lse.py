"""Writes gptoss_lse.npy: the fp64 log-sum-exp of z/T for every row of the gpt-oss head
workload (N = 32768, d = 2880, V = 201,088, T = 1, seeded inputs from datagen's "gptoss"
config), computed by oracle.lse_all_rows.

With it, a GPU test checks the full-batch lse of the fused forward at every row and derives
sampled rows of the full-batch dW on the host (oracle.dw_rows needs every row's lse, which
takes a few minutes of fp64 matrix products and so is stored here instead of recomputed).

Run from the repository root: python tests/golden/make_gptoss_lse.py
"""

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import datagen  # noqa: E402
import oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gptoss_lse.npy")


def main():
    p = datagen.make("gptoss")
    t0 = time.time()
    lse = oracle.lse_all_rows(p.f32("H"), p.f64("W"), p.T, block=512)
    np.save(OUT, lse.astype(np.float64))
    print(f"wrote {OUT}: {lse.shape[0]} rows (config seed {p.extra['seed']}), {time.time() - t0:.0f} s")


if __name__ == "__main__":
    main()
