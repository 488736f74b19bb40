"""GPU parity at the head dims served by the generic kernels: 32 and 96 in every dtype, 256 in
bf16 and fp16 (64 and 128 are covered by the other parity tests).  Same tolerances and
comparison as the other parity tests; shapes span several tiles with ragged tails, causal and
not, grouped-query heads, and a window."""
import pytest

import oracle
import workloads
from parity_helpers import assert_close, check_end_to_end, say, to_np64

pytestmark = pytest.mark.gpu

CASES = [
    # (dtype, B, H, H_kv, Sq, Sk, D, causal, window)
    ("bf16", 1, 4, 2, 300, 300, 32, True, 0),
    ("fp16", 2, 2, 1, 190, 333, 32, False, 0),
    ("fp32", 1, 2, 2, 130, 170, 32, True, 0),
    ("bf16", 1, 4, 1, 257, 257, 96, True, 0),
    ("fp16", 1, 2, 2, 140, 260, 96, False, 0),
    ("fp32", 1, 2, 1, 150, 120, 96, True, 0),
    ("bf16", 1, 4, 2, 300, 300, 256, True, 0),
    ("fp16", 1, 2, 2, 100, 290, 256, False, 0),
    ("bf16", 1, 2, 1, 330, 330, 96, True, 70),
    ("fp16", 1, 2, 1, 260, 200, 256, False, 40),
    ("fp32", 1, 2, 2, 120, 120, 32, False, 25),
]


@pytest.mark.parametrize("store_ds", [True, False], ids=["stored_ds", "recompute"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_head_dim_parity(fab, case, store_ds):
    """Both modes (fp32 has one path, which either flag selects)."""
    dt, B, H, H_kv, Sq, Sk, D, causal, W = case
    w = workloads.Workload(f"hd{D}_{dt}", dt, B, H, H_kv, Sq, Sk, D, causal,
                           seed=5000 + D + Sq + W, window=W)
    check_end_to_end(fab, w, store_ds=store_ds)


def test_head_dim_256_isolated_backward(fab):
    """The backward alone on the oracle's O (rounded to bf16) and LSE at head dim 256."""
    import torch
    w = workloads.Workload("hd256_iso", "bf16", 1, 2, 1, 200, 200, 256, True, seed=5300)
    q, k, v, do = workloads.make_inputs(w)
    o64, lse64 = oracle.attention_forward(q, k, v, True, w.scale)
    o = torch.from_numpy(o64).to(q.dtype)
    lse = torch.from_numpy(lse64).float()
    ref = oracle.attention_backward(do, q, k, v, o, lse.double(), True, w.scale)
    dev = torch.device("cuda:0")
    say("[case] isolated backward bf16 D=256")
    dq, dk, dv = fab.bwd(do.to(dev), q.to(dev), k.to(dev), v.to(dev), o.to(dev), lse.to(dev),
                         causal=True, scale=w.scale)
    for name, g, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        assert_close(name, to_np64(g), r, "bf16")
