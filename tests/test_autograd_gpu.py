"""torch.autograd integration: gradients through flash_attention() against the fp64 oracle
(same tolerances as the parity tests) and against a direct call of the backward."""
import numpy as np
import pytest

import oracle
import workloads
from parity_helpers import assert_close, say, to_np64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt,causal,D", [("bf16", True, 128), ("fp16", False, 64), ("fp32", True, 64)])
def test_autograd_matches_oracle(fab, dt, causal, D):
    import torch
    from flashattention_backward_amd.autograd import flash_attention
    w = workloads.Workload(f"autograd_{dt}", dt, 2, 4, 2, 150, 170, D, causal, seed=41)
    say(f"[case] autograd {dt} causal={causal} D={D}")
    q, k, v, do = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev).requires_grad_(True) for x in (q, k, v))
    out = flash_attention(qd, kd, vd, causal=causal)
    out.backward(do.to(dev))
    torch.cuda.synchronize()
    ref = oracle.attention_grads(q, k, v, do, causal, w.scale)
    assert_close("o", to_np64(out.detach()), ref["o"], dt)
    for name, t in (("dq", qd), ("dk", kd), ("dv", vd)):
        assert_close(name, to_np64(t.grad), ref[name], dt)


def test_autograd_equals_direct_backward_and_noncontiguous_grad(fab):
    import torch
    from flashattention_backward_amd.autograd import flash_attention
    w = workloads.Workload("autograd_direct", "bf16", 1, 4, 1, 96, 96, 128, True, seed=43)
    say("[case] autograd vs direct backward")
    q, k, v, do = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev).requires_grad_(True) for x in (q, k, v))
    out, lse = flash_attention(qd, kd, vd, causal=True, return_lse=True)
    assert not lse.requires_grad
    # an incoming gradient that is a non-contiguous view with the same values
    g = do.to(dev).transpose(2, 3).contiguous().transpose(2, 3)
    assert not g.is_contiguous()
    out.backward(g)
    dq, dk, dv = fab.bwd(do.to(dev), qd.detach(), kd.detach(), vd.detach(), out.detach(), lse,
                         causal=True)
    torch.cuda.synchronize()
    for a, b in ((qd.grad, dq), (kd.grad, dk), (vd.grad, dv)):
        assert torch.equal(a, b)
