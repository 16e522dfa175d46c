"""The stitching used by the GPU test of every rank (tests/stitch.py), run
with the oracle itself as the per-rank computation (CPU only). The oracle's
rank shares, put back through the zigzag permutation and with the partial
dK/dV summed over ranks, must equal the oracle on the whole batch as one rank
(invariants I4 and I7: the split over ranks and ring steps is exact, ai.info
summary, Methodology). This checks the stitching code, so that a GPU failure
of that test points at the library and not at the bookkeeping."""

import numpy as np
import pytest

import workloads

from helpers import oracle_grouped
from stitch import stitch_and_compare


def _oracle_rank(wr, lay, br, raw):
    dec = {k: workloads.as_f32(wr, v).astype(np.float64) for k, v in raw.items()}
    r = oracle_grouped(lay, br, *(dec[k] for k in ("q", "k", "v", "qb", "kb", "vb")),
                       dec["do"], dec["dob"], dtype=np.float64, threads=4)
    return {k: v.astype(np.float64) for k, v in r.items()}


@pytest.mark.slow
@pytest.mark.parametrize("name", ["dspark_r"])
def test_oracle_ranks_stitch_to_the_full_batch(name):
    w = workloads.make(name)
    errs = stitch_and_compare(w, _oracle_rank, seed=w.seed + 500)
    for key, e in errs.items():
        # fp32 full-batch oracle against fp64 rank shares: rounding only
        assert e[0] < 1e-4, (key, e)
