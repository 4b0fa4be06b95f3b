"""The stored full-size oracle score matrices (tests/golden/oracle_scores_*.npz, written by
tests/golden/make_oracle_scores.py from oracle/ alone) still belong to today's seeded inputs and
to the oracle: the digest of x matches, sampled rows recomputed by the oracle match bit for bit,
and the matrix has the structure MaxSim fixes (paperlayer.ai "Avey-B" summary, section 3): a -inf
diagonal and, off it, finite scores no larger than the target split's token count."""
import os
import sys

import numpy as np
import pytest

from oracle import avey_oracle as O
from synth import CONFIGS, make_inputs

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
from make_oracle_scores import x_digest  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("name,rows", [("base", [(0, 0), (7, 31)]), ("long", [(0, 0), (1, 64), (1, 127)]),
                                       ("extreme", [(0, 5), (0, 383)]), ("wide", [(0, 3), (3, 31)])])
def test_stored_scores_are_the_oracles(name, rows):
    cfg = CONFIGS[name]
    gold = np.load(os.path.join(GOLDEN, f"oracle_scores_{name}.npz"))
    s = gold["scores"]
    assert s.shape == (cfg.B, cfg.n_s, cfg.n_s) and s.dtype == np.float64
    inp = make_inputs(cfg)
    assert str(gold["x_sha256"]) == x_digest(inp.x)
    diag = np.eye(cfg.n_s, dtype=bool)[None].repeat(cfg.B, 0)
    assert np.all(s[diag] == -np.inf)
    off = s[~diag]
    assert np.isfinite(off).all() and off.max() <= cfg.S and off.min() > 0
    for b, i in rows:
        np.testing.assert_allclose(s[b, i], O.score_row(inp.x_f64(b), cfg.S, i), rtol=1e-12, atol=0)
