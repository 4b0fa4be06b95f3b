"""Write the float64 oracle's complete MaxSim score matrix of a full-size workload to
tests/golden/oracle_scores_<name>.npz, for the GPU test that compares every score, top-k set and
weight at that size (tests/test_gpu_parity_full.py).

    python tests/golden/make_oracle_scores.py [long]

The oracle computes every ordered split pair from its definition: the sum over the target
split's valid tokens of the maximum cosine to the candidate split's valid tokens, the diagonal
-inf (paperlayer.ai "Avey-B" summary, section 3; papernotes.org Avey-B note, 方法详解/整体框架).
At the 32K-token workload that is 32 512 ordered pairs, a few minutes on 8 cores; the GPU machine
would need the same time inside a test. The inputs are the seeded synthetic ones of synth/, and
the file records a digest of x so that the test can check it still holds the same inputs.

Only oracle/ and the seeded input generator are used here: no value comes from the GPU path.
"""
import hashlib
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import avey_oracle as O  # noqa: E402
from synth import CONFIGS, make_inputs  # noqa: E402

_X = None


def x_digest(x: np.ndarray) -> str:
    """sha256 of the input tensor's bytes (its exact values, shape and dtype)."""
    h = hashlib.sha256()
    h.update(str((x.dtype.str, x.shape)).encode())
    h.update(np.ascontiguousarray(x).tobytes())
    return h.hexdigest()


def _row(args):
    b, i, S = args
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        return b, i, O.score_row(_X[b], S, i)


def main(name: str = "long") -> str:
    global _X
    cfg = CONFIGS[name]
    inp = make_inputs(cfg)
    _X = {b: inp.x_f64(b) for b in range(cfg.B)}
    n_s = cfg.n_s
    scores = np.empty((cfg.B, n_s, n_s), dtype=np.float64)
    t0 = time.time()
    jobs = [(b, i, cfg.S) for b in range(cfg.B) for i in range(n_s)]
    with mp.get_context("fork").Pool(min(8, os.cpu_count() or 1)) as pool:
        for done, (b, i, row) in enumerate(pool.imap_unordered(_row, jobs, chunksize=2), 1):
            scores[b, i] = row
            if done % 32 == 0:
                print(f"{done}/{len(jobs)} rows, {time.time() - t0:.0f} s", flush=True)
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"oracle_scores_{name}.npz")
    np.savez(out, scores=scores, x_sha256=np.array(x_digest(inp.x)), config=np.array(repr(cfg)))
    print(f"wrote {out} ({os.path.getsize(out)} bytes) in {time.time() - t0:.0f} s", flush=True)
    return out


if __name__ == "__main__":
    main(*(sys.argv[1:] or ["long"]))
