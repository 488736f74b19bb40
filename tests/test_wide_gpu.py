"""GPU parity of the wide dK/dV workgroups (256 keys, 32-row query tiles), which the launcher
takes at head dims up to 128 when the grid of 256-key tiles still gives every CU of the
device at least two workgroups: batch x kv heads x ceil(Sk / 256) >= 2 x CUs (512 on
MI355X).  Many short sequences reach that grid at sizes the oracle finishes quickly; sampled
(batch, kv head) groups are compared whole, at the usual tolerances.  Cases cover ragged
sequences, grouped-query heads, causal and not, windows, and head dims 32 to 128."""
import pytest

import workloads
from parity_helpers import check_end_to_end

pytestmark = pytest.mark.gpu

CASES = [
    # (dtype, B, H, H_kv, Sq, Sk, D, causal, window)
    ("bf16", 32, 16, 16, 300, 300, 128, True, 0),
    ("fp16", 64, 16, 8, 200, 520, 128, False, 90),
    ("bf16", 128, 4, 4, 257, 257, 64, True, 33),
    ("fp16", 32, 32, 16, 190, 400, 96, True, 0),
    ("bf16", 128, 8, 4, 333, 280, 32, False, 0),
    ("bf16", 64, 8, 8, 500, 500, 128, True, 300),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_wide_dkdv_parity(fab, case):
    dt, B, H, H_kv, Sq, Sk, D, causal, W = case
    assert B * H_kv * -(-Sk // 256) >= 512  # the grid that selects the wide workgroups
    w = workloads.Workload(f"wide_{dt}", dt, B, H, H_kv, Sq, Sk, D, causal,
                           seed=7300 + Sq + Sk + D + W, window=W)
    groups = [(0, 0), (B // 2, H_kv // 2), (B - 1, H_kv - 1)]
    check_end_to_end(fab, w, groups=groups, jobs=1)
