"""Writes <config>_rowkl.npy: the fp64 KL_n of every row of a large workload (seeded inputs
from datagen), computed by oracle.kl_rows_all: each row's logits over the whole vocabulary,
its teacher softmax over the K cached entries, KL(p_t || p_s). Configs: "gptoss" (N = 32768),
"full" (the pages' shape, N = 131072), both at d = 2880, V = 201,088, T = 1; "qwen" (N = 8192,
d = 2048, V = 151,936, T = 2).

With it, a GPU test compares the fused forward's KL_n at every row, and its scalar loss with
the oracle's T^2/N sum of these values. The same pass recomputes every row's lse, which must
agree with <config>_lse.npy (written by make_lse.py from the same definition).

Run from the repository root: python tests/golden/make_rowkl.py gptoss full qwen
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
        out = oracle.kl_rows_all(p.f32("H"), p.f64("W"), p.idx, p.f64("tlog"), p.T, block=512)
        lse_path = os.path.join(HERE, f"{name}_lse.npy")
        if os.path.exists(lse_path):
            stored = np.load(lse_path, allow_pickle=False)
            err = float(np.max(np.abs(out["lse"] - stored) / np.abs(stored)))
            if err > 1e-13:
                raise SystemExit(f"{name}: lse differs from {lse_path} by {err:.2e}")
        path = os.path.join(HERE, f"{name}_rowkl.npy")
        np.save(path, out["row_kl"].astype(np.float64))
        print(f"wrote {path}: {p.N} rows (config seed {p.extra['seed']}), {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["gptoss", "full", "qwen"])
