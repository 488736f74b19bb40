"""Parity at the named workloads' full sizes, through the same entry points and launch
configuration the bench times, over every (batch, kv-head) group: every output element (O,
LSE, dQ, dK, dV) of the whole tensors is compared against the fp64 oracle, in both modes of
the backward (stored dS, which the bench times, and recompute).  The oracle runs one group per
worker process on all host cores the test may use, in spawned interpreters (they never touch
the GPU runtime of this process)."""
import os

import numpy as np
import pytest

import oracle
import workloads
from parity_helpers import assert_close, run_gpu, say, to_np64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_fullsize_all_groups(fab, name):
    w = workloads.get(name)
    jobs = len(os.sched_getaffinity(0))
    groups = [(b, g) for b in range(w.B) for g in range(w.H_kv)]
    say(f"[case] full size {w.name}: dtype={w.dtype} B={w.B} H={w.H} H_kv={w.H_kv} Sq={w.Sq} "
        f"Sk={w.Sk} D={w.D} causal={w.causal} window={w.window}; {len(groups)} groups, {jobs} oracle workers")
    q, k, v, do = workloads.make_inputs(w)
    outs = {}
    for store_ds in (True, False):
        out = run_gpu(fab, q, k, v, do, w.causal, w.scale, w.window, store_ds=store_ds)
        outs[store_ds] = {key: to_np64(t) for key, t in out.items()}
        del out
    res = oracle.grads_for_groups(q, k, v, do, w.causal, w.scale, groups, jobs=jobs,
                                  window=w.window, start_method="spawn")
    G = w.group
    exp = {key: np.empty(outs[True][key].shape) for key in ("o", "lse", "dq", "dk", "dv")}
    for (b, g), r in res.items():
        hs = slice(g * G, (g + 1) * G)
        exp["o"][b, hs], exp["lse"][b, hs], exp["dq"][b, hs] = r["o"], r["lse"], r["dq"]
        exp["dk"][b, g], exp["dv"][b, g] = r["dk"], r["dv"]
    for store_ds, got in outs.items():
        say(f"  mode={'stored-dS' if store_ds else 'recompute'}")
        for key in ("o", "lse", "dq", "dk", "dv"):
            assert got[key].size == exp[key].size
            say(f"    {key}: {got[key].size} elements compared (whole tensor)")
            assert_close(key, got[key], exp[key], "fp32" if key == "lse" and w.dtype != "fp32" else w.dtype)
