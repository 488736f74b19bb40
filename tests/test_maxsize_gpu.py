"""GPU parity at the largest sizes the library accepts: 2**31 - 1 elements in the biggest
tensor (Q, O, dO, dQ), where the byte size of a kv group's query rows comes within 100 KB of
2**32 and every 32-bit offset is at its limit.  Sequences are ragged (not a tile multiple).

The oracle cannot take such a sequence whole, so a causal sliding window of W keys makes a
short span exact: for positions [c, e), a row i >= c + W - 1 sees only keys inside the span
(the window starts at i - W + 1), and a key j in [c + W - 1, e - W + 1) receives gradient
only from rows in [j, j + W - 1], all of which are such rows.  At the sequence's ends the
bounds relax (nothing lies before 0 or after S).  The oracle runs on the span's rounded
inputs; O, LSE, dQ of its exact rows and dK, dV of its exact keys are compared, at the usual
tolerances, for spans at the start, the middle and the end of the sequence.  Inputs are drawn
on the GPU from a seeded generator (2**31 host draws would take minutes).
"""
import numpy as np
import pytest

import oracle
import workloads
from parity_helpers import assert_close, say, to_np64, window_span_ranges

pytestmark = pytest.mark.gpu

MAX_ELEMS = 2 ** 31 - 1

CASES = [
    # (dtype, H, H_kv, D, window): the tiled 16-bit kernels at D = 128 (grouped-query heads)
    # and D = 256, and the fp32 kernels
    ("bf16", 4, 1, 128, 192),
    ("fp16", 2, 1, 256, 160),
    ("fp32", 1, 1, 128, 96),
]


def spans(S, W):
    n = 3 * W + 5
    mid = S // 2 - 1001
    return [(0, n), (mid, mid + n), (S - n - 11, S)]


def compare_spans(tensors, S, W, scale, dt):
    """Compare O, LSE, dQ on the exact rows and dK, dV on the exact keys of three spans
    (start, middle, end) with the oracle run on each span's inputs."""
    q, k, v, do, o, lse, dq, dk, dv = tensors
    got = {key: [] for key in ("o", "lse", "dq", "dk", "dv")}
    exp = {key: [] for key in got}
    for c, e in spans(S, W):
        rows, keys = window_span_ranges(c, e, S, W)
        cut = lambda t: t[:, :, c:e].cpu()
        ref = oracle.attention_grads(cut(q), cut(k), cut(v), cut(do), True, scale, window=W)
        r0, r1 = rows[0] - c, rows[1] - c
        k0, k1 = keys[0] - c, keys[1] - c
        for key, t, a, b in (("o", o, r0, r1), ("lse", lse, r0, r1), ("dq", dq, r0, r1),
                             ("dk", dk, k0, k1), ("dv", dv, k0, k1)):
            got[key].append(to_np64(t[:, :, c + a:c + b]).ravel())
            exp[key].append(np.asarray(ref[key])[:, :, a:b].ravel())
    return got, exp


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_max_size_parity(fab, case):
    import torch
    dt, H, H_kv, D, W = case
    S = MAX_ELEMS // (H * D) - 37
    assert H * S * D <= MAX_ELEMS
    w = workloads.Workload(f"max_{dt}_d{D}", dt, 1, H, H_kv, S, S, D, True, seed=7100 + D, window=W)
    dev = torch.device("cuda:0")
    say(f"[case] max size {dt} B=1 H={H} H_kv={H_kv} S={S} D={D} window={W} "
        f"({H * S * D} elements per query tensor)")
    q, k, v, do = workloads.make_inputs_device(w, dev)
    o, lse = fab.fwd(q, k, v, causal=True, scale=w.scale, window_size=W)
    dq, dk, dv = fab.bwd(do, q, k, v, o, lse, causal=True, scale=w.scale, window_size=W)
    torch.cuda.synchronize()
    say("    GPU forward and backward done")
    got, exp = compare_spans((q, k, v, do, o, lse, dq, dk, dv), S, W, w.scale, dt)
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    for key in got:
        assert_close(key, np.concatenate(got[key]), np.concatenate(exp[key]),
                     "fp32" if key == "lse" else dt)


def test_stored_ds_largest_slab(fab):
    """The stored-dS mode at the largest dS slab it takes: 2**31 bytes for one (batch, head)
    (ragged Sq = Sk = 32731, rounded up to 32768 rows and keys), one query head per kv head, so
    the group's dS buffer resource spans 2**31 bytes and the fragments near the slab's end sit
    at 32-bit offsets just below it.  Spans of a causal sliding window are compared with the
    oracle as in the maximum-size test."""
    import torch
    dt, H, H_kv, D, W = "bf16", 1, 1, 128, 192
    S = 32768 - 37
    code = fab.DTYPE_CODES["bfloat16"]
    nb = fab.bwd_workspace_bytes(1, H, H_kv, S, S, D, code, store_ds=True)
    assert nb > 2 ** 31 and fab.bwd_plan(1, H, H_kv, S, S, D, code, nb) == "stored_ds"
    w = workloads.Workload("max_ds_slab", dt, 1, H, H_kv, S, S, D, True, seed=7301, window=W)
    dev = torch.device("cuda:0")
    say(f"[case] stored dS, largest slab: {dt} B=1 H={H} S={S} D={D} window={W}, workspace {nb} bytes")
    q, k, v, do = workloads.make_inputs_device(w, dev)
    o, lse = fab.fwd(q, k, v, causal=True, scale=w.scale, window_size=W)
    dq, dk, dv = fab.bwd(do, q, k, v, o, lse, causal=True, scale=w.scale, window_size=W, store_ds=True)
    torch.cuda.synchronize()
    say("    GPU forward and backward done")
    got, exp = compare_spans((q, k, v, do, o, lse, dq, dk, dv), S, W, w.scale, dt)
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    for key in got:
        assert_close(key, np.concatenate(got[key]), np.concatenate(exp[key]),
                     "fp32" if key == "lse" else dt)
