"""fab_bwd_noalloc (the backward without a workspace, for callers that cannot allocate)
against fab_bwd through the C ABI: two calls in a row on the same GPU, the second with a
smaller input, so that the second call runs on scratch that still holds the first call's
statistics.  Each result must match fab_bwd's on the same inputs within the parity
tolerances (bf16: max|err| <= 2e-2 max|ref|, relative Frobenius <= 1e-2; fp32: 1e-4)."""
import ctypes

import pytest

import workloads
from parity_helpers import assert_close, say, to_np64

pytestmark = pytest.mark.gpu

CASES = [  # (dtype, B, H, H_kv, Sq, Sk, D, causal, window, seed): the second is smaller
    ("bf16", 2, 8, 2, 700, 700, 128, True, 0, 101),
    ("bf16", 1, 2, 1, 77, 93, 64, False, 0, 102),
    ("fp32", 1, 2, 2, 50, 40, 64, True, 0, 103),
]


def _run(fab, w, noalloc):
    import torch
    dev = torch.device("cuda:0")
    q, k, v, do = (x.to(dev) for x in workloads.make_inputs(w))
    o, lse = fab.fwd(q, k, v, causal=w.causal, scale=w.scale, window_size=w.window)
    if noalloc:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        torch.cuda.synchronize()
        L = fab.lib()
        code = fab.DTYPE_CODES[str(q.dtype).replace("torch.", "")]
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        st = L.fab_bwd_noalloc(do.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               lse.data_ptr(), out[0].data_ptr(), out[1].data_ptr(), out[2].data_ptr(),
                               w.B, w.H, w.H_kv, w.Sq, w.Sk, w.D, code, int(w.causal), w.window,
                               float(w.scale), stream)
        assert st == 0, L.fab_last_error().decode()
    else:
        out = fab.bwd(do, q, k, v, o, lse, causal=w.causal, scale=w.scale, window_size=w.window)
    torch.cuda.synchronize()
    return out


def test_noalloc_matches_fab_bwd_on_consecutive_calls(fab):
    for dt, B, H, H_kv, Sq, Sk, D, causal, win, seed in CASES:
        w = workloads.Workload(f"noalloc_{dt}_{Sq}x{Sk}_d{D}", dt, B, H, H_kv, Sq, Sk, D, causal,
                               seed=seed, window=win)
        say(f"[case] fab_bwd_noalloc vs fab_bwd: {w.name} B={B} H={H} H_kv={H_kv} causal={causal}")
        got = _run(fab, w, noalloc=True)
        ref = _run(fab, w, noalloc=False)
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            assert_close(name, to_np64(g), to_np64(r), dt)
