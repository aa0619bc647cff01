"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The float64 oracle cannot evaluate every output of these workloads in seconds,
so it checks a seeded sample of (query row, head) outputs one by one; block
tables are still compared in full.  The sample always includes the first and
last rows.
"""

import numpy as np
import pytest

from workloads import recipes

from _gpu_common import assert_close, run_both

pytestmark = pytest.mark.gpu


def _sampler(per_op, seed=0):
    def sample(op, nrows):
        rng = np.random.default_rng(seed + op[1])
        wl_heads = sample.heads
        rows = rng.integers(0, nrows, per_op)
        heads = rng.integers(0, wl_heads, per_op)
        pts = list(zip(rows.tolist(), heads.tolist()))
        pts += [(0, 0), (nrows - 1, wl_heads - 1)]
        return sorted(set(pts))
    return sample


@pytest.mark.parametrize("name,per_op", [("llama_fork", 48), ("mcts_tree", 48), ("spec_verify", 64),
                                         ("full_depth", 6)])
def test_standard_workload_sampled(name, per_op):
    wl = recipes.STANDARD[name]()
    s = _sampler(per_op)
    s.heads = wl.q_heads
    assert_close(run_both(wl, sample=s), wl.dtype)
