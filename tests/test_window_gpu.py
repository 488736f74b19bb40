"""GPU parity with a sliding window (``window_size``): the HIP forward and backward through
the C ABI against the fp64 oracle, at the same tolerances as the other parity tests.

Cases span several tiles in both directions with ragged tails, windows narrower and wider
than a tile, W = 1, windows that leave rows without keys (O = 0, LSE = -inf, dQ = 0), and a
window wide enough to cut nothing, which must give exactly the results of no window.
"""
import numpy as np
import pytest

import oracle
import workloads
from parity_helpers import assert_close, check_end_to_end, run_gpu, say, to_np64

pytestmark = pytest.mark.gpu

CASES = [
    # (dtype, B, H, H_kv, Sq, Sk, D, causal, window)
    ("bf16", 1, 4, 2, 333, 333, 128, True, 100),
    ("fp16", 1, 2, 2, 300, 260, 64, False, 50),
    ("bf16", 1, 2, 1, 200, 200, 128, True, 1),
    ("bf16", 2, 2, 2, 512, 512, 64, True, 128),    # window and sequence on tile multiples
    ("fp16", 1, 4, 1, 190, 330, 128, False, 70),   # Sk > Sq, several kv tiles per query tile
    ("bf16", 1, 2, 1, 400, 100, 128, True, 64),    # rows 163.. keep no key
    ("fp16", 1, 2, 2, 300, 64, 64, False, 20),     # rows 83.. keep no key
    ("fp32", 1, 2, 1, 150, 150, 64, True, 37),
    ("fp32", 1, 2, 2, 100, 90, 128, False, 64),
    ("fp32", 1, 2, 1, 120, 30, 64, True, 16),      # fp32 with rows that keep no key
]


@pytest.mark.parametrize("store_ds", [True, False], ids=["stored_ds", "recompute"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_window_parity(fab, case, store_ds):
    """Both modes (fp32 has one path, which either flag selects)."""
    dt, B, H, H_kv, Sq, Sk, D, causal, W = case
    w = workloads.Workload(f"win_{dt}", dt, B, H, H_kv, Sq, Sk, D, causal,
                           seed=3000 + Sq + 3 * Sk + W, window=W)
    out, _ = check_end_to_end(fab, w, store_ds=store_ds)
    if Sq - Sk >= W:  # rows without keys: exact zeros and -inf
        first = Sk + W - 1
        assert float(out["o"][:, :, first:].abs().max()) == 0.0
        assert float(out["dq"][:, :, first:].abs().max()) == 0.0
        assert bool(np.all(np.isneginf(to_np64(out["lse"][:, :, first:]))))


def test_window_long_sequence(fab):
    """A Mistral-like shape at a size the oracle still finishes quickly: causal GQA with a
    window of 256 keys over 2048 positions."""
    w = workloads.Workload("win_long", "bf16", 1, 4, 1, 2048, 2048, 128, True, seed=3100, window=256)
    check_end_to_end(fab, w)


@pytest.mark.parametrize("causal", [False, True])
def test_wide_window_equals_no_window(fab, causal):
    """A window of max(Sq, Sk) keys cuts nothing: every output bit equals the no-window run."""
    import torch
    w = workloads.Workload("win_wide", "bf16", 1, 4, 2, 190, 250, 128, causal, seed=3200)
    q, k, v, do = workloads.make_inputs(w)
    a = run_gpu(fab, q, k, v, do, causal, w.scale, 0)
    b = run_gpu(fab, q, k, v, do, causal, w.scale, 250)
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[key], b[key]), key


def test_window_autograd(fab):
    """torch.autograd through flash_attention(..., window_size=W) against the oracle."""
    import torch
    from flashattention_backward_amd.autograd import flash_attention
    w = workloads.Workload("win_autograd", "bf16", 1, 4, 2, 260, 260, 64, True, seed=3300, window=90)
    q, k, v, do = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev).requires_grad_(True) for x in (q, k, v))
    say("[case] autograd window=90 bf16 D=64")
    out = flash_attention(qd, kd, vd, causal=True, window_size=90)
    out.backward(do.to(dev))
    ref = oracle.attention_grads(q, k, v, do, True, w.scale, window=90)
    assert_close("o", to_np64(out), ref["o"], "bf16")
    for name, t in (("dq", qd), ("dk", kd), ("dv", vd)):
        assert_close(name, to_np64(t.grad), ref[name], "bf16")
