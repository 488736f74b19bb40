"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by element.

Tolerances (per output tensor, over all compared elements): fp32 max|err| <= 1e-4 max|ref|;
bf16/fp16 max|err| <= 2e-2 max|ref| and relative Frobenius error <= 1e-2.  LSE is float32
in every dtype and is held to the fp32 bound... relative to max|LSE|.
"""
import numpy as np
import pytest

import oracle
import workloads
from parity_helpers import assert_close, check_end_to_end, run_gpu, say, to_np64

pytestmark = pytest.mark.gpu

# Every named workload at a reduced size that the oracle finishes in seconds but that still
# spans several tiles in both directions and ends in a ragged tail.
REDUCED = {
    "fp32_h2_s128_d64": {},  # already small: the full workload
    "bf16_causal_h8_s1024_d64": dict(B=1, H=3, H_kv=3, Sq=333, Sk=333),
    "bf16_causal_h16_s2048_d128": dict(B=1, H=2, H_kv=2, Sq=300, Sk=300),
    "bf16_gqa4_causal_h32_s4096_d128": dict(B=1, H=8, H_kv=2, Sq=272, Sk=272),
    "fp16_causal_h16_s16384_d128": dict(B=1, H=2, H_kv=2, Sq=513, Sk=513),
    "fp16_gqa4_h16_sq512_sk8192_d128": dict(B=2, H=4, H_kv=1, Sq=77, Sk=700),
}


MODES = [True, False]  # store_ds: the stored-dS mode, then the recompute mode
MODE_IDS = ["stored_ds", "recompute"]


@pytest.mark.parametrize("store_ds", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("name", list(REDUCED))
def test_named_workloads_reduced(fab, name, store_ds):
    w = workloads.scaled(workloads.get(name), **REDUCED[name])
    check_end_to_end(fab, w, store_ds=store_ds)


SHAPES = [
    # (dtype, B, H, H_kv, Sq, Sk, D, causal)
    ("bf16", 1, 2, 1, 1, 1, 64, False),
    ("bf16", 1, 2, 1, 1, 1, 128, True),
    ("fp16", 1, 1, 1, 5, 3, 64, False),
    ("bf16", 2, 4, 2, 129, 257, 128, True),    # causal, Sk > Sq: keys past Sq-1 get zero grad
    ("bf16", 1, 4, 1, 260, 70, 64, True),      # causal, Sq > Sk
    ("fp16", 1, 8, 8, 200, 200, 128, False),
    ("fp16", 2, 4, 4, 64, 128, 64, True),      # exact tile multiples
    ("fp32", 1, 2, 1, 100, 150, 128, True),
    ("fp32", 2, 2, 2, 65, 33, 64, False),
    ("bf16", 1, 16, 2, 96, 96, 128, False),    # 8 query heads per kv head
    ("bf16", 1, 6, 2, 300, 280, 128, True),    # 3 query heads per kv head (odd group)
    ("fp16", 1, 5, 1, 140, 333, 96, False),    # 5 query heads per kv head, head dim 96
]


@pytest.mark.parametrize("store_ds", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_shapes_and_edges(fab, shape, store_ds):
    dt, B, H, H_kv, Sq, Sk, D, causal = shape
    w = workloads.Workload(f"edge_{dt}", dt, B, H, H_kv, Sq, Sk, D, causal, seed=1000 + Sq + 7 * Sk)
    check_end_to_end(fab, w, store_ds=store_ds)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 1e-3, 0.5])
@pytest.mark.parametrize("dt,D", [("bf16", 128), ("fp16", 64)])
def test_scale_values(fab, dt, D, scale):
    """Softmax scales of either sign, zero and tiny: a masked score is replaced by a value
    whose exponent is -inf for the sign of the scale, and a zero scale runs with the smallest
    normal exponent scale.  Causal, with ragged tails, so masked steps are exercised."""
    w = workloads.Workload(f"scale_{dt}", dt, 1, 4, 2, 150, 170, D, True, seed=31)
    say(f"[case] scale={scale} {dt} D={D}")
    q, k, v, do = workloads.make_inputs(w)
    out = run_gpu(fab, q, k, v, do, True, scale)
    ref = oracle.attention_grads(q, k, v, do, True, scale)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert_close(name, to_np64(out[name]), ref[name], "fp32" if name == "lse" else dt)


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
def test_isolated_backward(fab, dt):
    """Diagnostic mode: the GPU backward fed the oracle's O (rounded to the dtype) and LSE."""
    import torch
    w = workloads.Workload(f"iso_{dt}", dt, 1, 4, 2, 190, 230, 128, True, seed=77)
    say(f"[case] isolated backward {dt}")
    q, k, v, do = workloads.make_inputs(w)
    o64, lse64 = oracle.attention_forward(q, k, v, w.causal, w.scale)
    tdt = q.dtype
    o = torch.from_numpy(o64).to(tdt)
    lse = torch.from_numpy(lse64).float()
    ref = oracle.attention_backward(do, q, k, v, o, lse.double(), w.causal, w.scale)
    dev = torch.device("cuda:0")
    dq, dk, dv = fab.bwd(do.to(dev), q.to(dev), k.to(dev), v.to(dev), o.to(dev), lse.to(dev),
                         causal=True, scale=w.scale)
    delta, _ = fab.bwd_preprocess(do.to(dev), o.to(dev), lse.to(dev))
    torch.cuda.synchronize()
    assert_close("delta", to_np64(delta), ref[3], "fp32" if dt == "fp32" else "bf16")
    for name, g, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        assert_close(name, to_np64(g), r, dt)


@pytest.mark.parametrize("store_ds", MODES, ids=MODE_IDS)
def test_deterministic(fab, store_ds):
    import torch
    w = workloads.Workload("det", "bf16", 1, 8, 2, 300, 300, 128, True, seed=5)
    say(f"[case] determinism store_ds={store_ds}")
    q, k, v, do = workloads.make_inputs(w)
    a = run_gpu(fab, q, k, v, do, True, w.scale, store_ds=store_ds)
    b = run_gpu(fab, q, k, v, do, True, w.scale, store_ds=store_ds)
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("B,H,H_kv,S", [(2, 8, 2, 333), (2, 16, 4, 1100)])
def test_modes_agree(fab, B, H, H_kv, S):
    """Where both modes run the same dK/dV kernel (the recompute plan's separate launches),
    dV depends only on P and is bitwise equal.  The small problem's one-launch recompute plan
    runs another dK/dV kernel, whose dV sums in another order.  dK also depends on D, which the
    two modes sum in different orders (the preprocess kernel, or the recomputing dQ kernel's
    prologue), and dQ is formed differently: all agree with the other mode to the tolerances."""
    import torch
    w = workloads.Workload("modes", "bf16", B, H, H_kv, S, S, 128, True, seed=15)
    say(f"[case] stored dS vs recompute: B={B} H={H} H_kv={H_kv} S={S}")
    q, k, v, do = workloads.make_inputs(w)
    a = run_gpu(fab, q, k, v, do, True, w.scale, store_ds=True)
    b = run_gpu(fab, q, k, v, do, True, w.scale, store_ds=False)
    code = fab.DTYPE_CODES["bfloat16"]
    nb = fab.bwd_workspace_bytes(B, H, H_kv, S, S, 128, code, store_ds=False)
    if fab.bwd_plan(B, H, H_kv, S, S, 128, code, nb) == "recompute":
        assert torch.equal(a["dv"], b["dv"])
    else:
        assert_close("dv", to_np64(a["dv"]), to_np64(b["dv"]), "bf16")
    assert_close("dk", to_np64(a["dk"]), to_np64(b["dk"]), "bf16")
    assert_close("dq", to_np64(a["dq"]), to_np64(b["dq"]), "bf16")


@pytest.mark.parametrize("dt,D,causal,win", [("bf16", 128, True, 0), ("fp16", 64, False, 0),
                                             ("bf16", 96, True, 70), ("fp16", 256, True, 0)])
def test_step_entry_points_stored_ds(fab, dt, D, causal, win):
    """fab_bwd_preprocess, fab_bwd_dkdv and fab_bwd_dq called one by one with the stored-dS
    workspace (the route bench.py times kernel by kernel): dkdv stores dS, dq reads it."""
    import ctypes
    import torch
    w = workloads.Workload(f"steps_{dt}", dt, 1, 4, 2, 211, 245, D, causal, seed=61, window=win)
    say(f"[case] step entry points, stored dS: {dt} D={D} causal={causal} window={win}")
    q, k, v, do = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    o, lse = fab.fwd(qd, kd, vd, causal=causal, scale=w.scale, window_size=win)
    L = fab.lib()
    code = fab.DTYPE_CODES[str(qd.dtype).replace("torch.", "")]
    nb = fab.bwd_workspace_bytes(w.B, w.H, w.H_kv, w.Sq, w.Sk, D, code, store_ds=True)
    assert nb > fab.bwd_workspace_bytes(w.B, w.H, w.H_kv, w.Sq, w.Sk, D, code, store_ds=False)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    dims = (w.B, w.H, w.H_kv, w.Sq, w.Sk, D, code, int(causal), win, float(w.scale))
    assert L.fab_bwd_preprocess(dod.data_ptr(), o.data_ptr(), lse.data_ptr(), ws.data_ptr(), nb,
                                w.B, w.H, w.Sq, D, code, st) == 0
    assert L.fab_bwd_dkdv(dod.data_ptr(), qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), ws.data_ptr(),
                          nb, dk.data_ptr(), dv.data_ptr(), *dims, st) == 0
    assert L.fab_bwd_dq(dod.data_ptr(), qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), ws.data_ptr(),
                        nb, dq.data_ptr(), *dims, st) == 0
    torch.cuda.synchronize()
    ref = oracle.attention_grads(q, k, v, do, causal, w.scale, window=win)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_close(name, to_np64(g), ref[name], dt)


def test_causal_zero_rows_and_invariants(fab):
    """Exact zeros where the mask cuts every path; shift and row-stochastic invariants."""
    import torch
    w = workloads.Workload("inv", "fp32", 1, 4, 2, 150, 190, 64, True, seed=9)
    say("[case] invariants")
    q, k, v, do = workloads.make_inputs(w)
    out = run_gpu(fab, q, k, v, do, True, w.scale)
    dk, dv, dq = to_np64(out["dk"]), to_np64(out["dv"]), to_np64(out["dq"])
    # keys 150..189 are beyond the last query row: no query attends them
    assert np.all(dk[:, :, 150:] == 0.0) and np.all(dv[:, :, 150:] == 0.0)
    # the first query row attends only key 0: dq row 0 ~ 0
    assert np.max(np.abs(dq[:, :, 0])) <= 1e-5 * max(1.0, np.max(np.abs(dq)))
    # sum_j dK_j = 0 (shift invariance), sum_j dV_j = sum over the group of dO
    assert np.max(np.abs(dk.sum(axis=2))) <= 1e-4 * np.abs(dk).sum(axis=2).max()
    do64 = to_np64(do)
    np.testing.assert_allclose(dv.sum(axis=2), do64.reshape(1, 2, 2, 150, 64).sum(axis=(2, 3)),
                               rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("dt,D,causal,window", [("bf16", 128, True, 0), ("fp16", 64, False, 40),
                                                ("fp32", 64, True, 0)])
def test_step_entry_points(fab, dt, D, causal, window):
    """fab_bwd_preprocess, then fab_bwd_dkdv and fab_bwd_dq on their own (the calls the bench
    times per kernel), against the oracle; fab_bwd itself folds step 1 into its dQ kernel on
    the 16-bit path, so this route is checked separately."""
    import ctypes
    import torch
    w = workloads.Workload(f"steps_{dt}", dt, 1, 4, 2, 230, 190, D, causal, seed=91, window=window)
    say(f"[case] step entry points {dt} D={D} causal={causal} window={window}")
    q, k, v, do = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    o, lse = fab.fwd(qd, kd, vd, causal=causal, scale=w.scale, window_size=window)
    code = fab._dtype_code(qd)
    nb = fab.bwd_workspace_bytes(w.B, w.H, w.H_kv, w.Sq, w.Sk, D, code)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    L = fab.lib()
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    dims = (w.B, w.H, w.H_kv, w.Sq, w.Sk, D, code, int(causal), window, float(w.scale), st)
    assert L.fab_bwd_preprocess(dod.data_ptr(), o.data_ptr(), lse.data_ptr(), ws.data_ptr(), nb,
                                w.B, w.H, w.Sq, D, code, st) == 0
    assert L.fab_bwd_dkdv(dod.data_ptr(), qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), ws.data_ptr(),
                          nb, dk.data_ptr(), dv.data_ptr(), *dims) == 0
    assert L.fab_bwd_dq(dod.data_ptr(), qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), ws.data_ptr(),
                        nb, dq.data_ptr(), *dims) == 0
    torch.cuda.synchronize()
    ref = oracle.attention_grads(q, k, v, do, causal, w.scale, window=window)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_close(name, to_np64(g), ref[name], dt)


@pytest.mark.parametrize("dt,D,causal,window", [("bf16", 128, True, 0), ("fp16", 64, False, 0),
                                                ("bf16", 96, True, 50), ("fp32", 64, True, 0)])
def test_peaked_softmax(fab, dt, D, causal, window):
    """Q and K scaled by 4: scores with a standard deviation near 16, so most rows' softmax is
    close to one-hot and row maxima jump across key tiles (the forward's rescaling)."""
    import torch
    w = workloads.Workload(f"peaked_{dt}", dt, 1, 4, 2, 300, 260, D, causal, seed=211, window=window)
    q, k, v, do = workloads.make_inputs(w)
    tdt = q.dtype
    q = (q.float() * 4).to(tdt)
    k = (k.float() * 4).to(tdt)
    say(f"[case] peaked softmax {dt} D={D} causal={causal} window={window}")
    out = run_gpu(fab, q, k, v, do, causal, w.scale, window)
    ref = oracle.attention_grads(q, k, v, do, causal, w.scale, window=window)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert_close(name, to_np64(out[name]), ref[name], "fp32" if name == "lse" else dt)
