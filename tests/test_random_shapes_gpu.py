"""GPU parity over random shapes: a fixed list of cases drawn once from a seeded generator
(dtype, head dim, query heads per kv head, kv heads, Sq and Sk from 1 to 400, causal or not,
a window or none), each run end to end (HIP forward then backward) against the fp64 oracle at
the usual tolerances.  The draws reach combinations the hand-picked cases do not: Sq or Sk of
1, windows wider than the sequence, rectangular causal with Sq > Sk, head dim 256 with a
window, and so on.  Every case is printed before it runs."""
import numpy as np
import pytest

import workloads
from parity_helpers import check_end_to_end

pytestmark = pytest.mark.gpu


def draw_cases(n=24, seed=20261202):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dt = ["bf16", "fp16", "fp32"][rng.integers(3)]
        dims = [32, 64, 96, 128] + ([256] if dt != "fp32" else [])
        D = int(dims[rng.integers(len(dims))])
        G = int([1, 2, 4][rng.integers(3)])
        H_kv = int(rng.integers(1, 3))
        # mostly mid-sized, sometimes tiny
        Sq = int(rng.integers(1, 9) if rng.random() < 0.15 else rng.integers(9, 401))
        Sk = int(rng.integers(1, 9) if rng.random() < 0.15 else rng.integers(9, 401))
        causal = bool(rng.random() < 0.6)
        W = 0 if rng.random() < 0.5 else int(rng.integers(1, max(Sq, Sk) + 20))
        cases.append((dt, 1, G * H_kv, H_kv, Sq, Sk, D, causal, W, 9000 + i))
    return cases


CASES = draw_cases()


@pytest.mark.parametrize("store_ds", [True, False], ids=["stored_ds", "recompute"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_random_shape_parity(fab, case, store_ds):
    dt, B, H, H_kv, Sq, Sk, D, causal, W, seed = case
    w = workloads.Workload(f"rand_{dt}", dt, B, H, H_kv, Sq, Sk, D, causal, seed=seed, window=W)
    check_end_to_end(fab, w, store_ds=store_ds)
