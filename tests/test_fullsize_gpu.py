"""Parity at the named workloads' full sizes, through the same entry points and launch
configuration the bench times.  The oracle computes whole (batch, kv-head) groups -- every
output element of the sampled groups (their G query heads' O, LSE and dQ, and the group's dK
and dV) is compared; the sample is the first and the last group of each workload (one group
for the 16384-long causal case, whose single head takes the oracle ~10 s)."""
import pytest

import workloads
from parity_helpers import check_end_to_end

pytestmark = pytest.mark.gpu


def sample_groups(w):
    last = (w.B - 1, w.H_kv - 1)
    if w.Sq * w.Sk > 1 << 26:
        return [last]
    return [(0, 0), last] if last != (0, 0) else [(0, 0)]


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_fullsize_sampled_groups(fab, name):
    w = workloads.get(name)
    check_end_to_end(fab, w, groups=sample_groups(w), jobs=1)
