"""Shared helpers for the GPU parity tests: run the HIP path, run the oracle, compare."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import workloads

TOL = {  # per output tensor: (max|err| / max|ref|, relative Frobenius error)
    "fp32": (1e-4, 1e-4),
    "bf16": (2e-2, 1e-2),
    "fp16": (2e-2, 1e-2),
}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np64(t) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


# Where the exact gradient is identically zero (closed forms such as a single key, whose dQ
# and dK vanish), a relative bound would demand bit-exact zeros from float arithmetic; the
# denominators are therefore floored at REF_FLOOR (max|ref|) and REF_FLOOR * sqrt(n)
# (Frobenius).  Gradients of the N(0, 1) workloads are orders of magnitude above the floor,
# so it only acts on those degenerate cases.
REF_FLOOR = 1e-3


def errors(got: np.ndarray, ref: np.ndarray):
    err = np.abs(got - ref)
    mx = max(float(np.max(np.abs(ref))), REF_FLOOR)
    rel_max = float(np.max(err)) / mx
    fro_ref = max(float(np.linalg.norm(ref.ravel())), REF_FLOOR * np.sqrt(ref.size))
    fro = float(np.linalg.norm((got - ref).ravel())) / fro_ref
    return rel_max, fro


def assert_close(name: str, got: np.ndarray, ref: np.ndarray, dtype: str):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    empty = np.isneginf(ref)  # the LSE of a row that keeps no key (a window can leave one)
    if np.any(empty):
        assert np.array_equal(np.isneginf(got), empty), f"{name}: -inf at other positions"
        got, ref = got[~empty], ref[~empty]
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    tmax, tfro = TOL[dtype]
    rel_max, fro = errors(got, ref)
    say(f"    {name:6s} max|err|/max|ref| = {rel_max:.3e} (tol {tmax:g})   rel-Frobenius = {fro:.3e} (tol {tfro:g})")
    assert rel_max <= tmax, f"{name}: max relative error {rel_max:.3e} > {tmax:g}"
    assert fro <= tfro, f"{name}: relative Frobenius error {fro:.3e} > {tfro:g}"


def window_span_ranges(c: int, e: int, S: int, W: int):
    """For causal attention with a window of W keys over S positions, the rows and the keys of
    the span [c, e) whose results the span's inputs alone determine: a row i sees keys
    [i - W + 1, i], inside the span from i = c + W - 1 on (from 0 at the sequence's start);
    a key j gets gradient from rows [j, j + W - 1], all such rows below e - W + 1 (below S at
    the sequence's end).  Returns ((row_lo, row_hi), (key_lo, key_hi)), half-open."""
    lo = c + W - 1 if c > 0 else 0
    return (lo, e), (lo, e - W + 1 if e < S else S)


def run_gpu(fab, q, k, v, do, causal, scale, window=0, store_ds=None):
    """End-to-end HIP path: fwd then bwd, all inputs resident on cuda:0.  store_ds selects the
    backward's mode through its workspace size: None the recommended one, True stored dS
    (where it can run), False recompute."""
    import torch
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    o, lse = fab.fwd(qd, kd, vd, causal=causal, scale=scale, window_size=window)
    dq, dk, dv = fab.bwd(dod, qd, kd, vd, o, lse, causal=causal, scale=scale, window_size=window,
                         store_ds=store_ds)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def check_end_to_end(fab, w: workloads.Workload, groups=None, jobs: int = 1, check_fwd=True,
                     store_ds=None):
    """GPU fwd+bwd against oracle fwd+bwd on the same rounded inputs.  With ``groups`` only
    those (b, kv head) groups are compared (full-size runs)."""
    say(f"[case] {w.name} dtype={w.dtype} B={w.B} H={w.H} H_kv={w.H_kv} Sq={w.Sq} Sk={w.Sk} "
        f"D={w.D} causal={w.causal} window={w.window} seed={w.seed} groups={groups} "
        f"mode={ {None: 'recommended', True: 'stored-dS', False: 'recompute'}[store_ds] }")
    q, k, v, do = workloads.make_inputs(w)
    out = run_gpu(fab, q, k, v, do, w.causal, w.scale, w.window, store_ds=store_ds)
    if groups is None:
        ref = oracle.attention_grads(q, k, v, do, w.causal, w.scale, window=w.window)
        pairs = [("dq", out["dq"], ref["dq"]), ("dk", out["dk"], ref["dk"]), ("dv", out["dv"], ref["dv"])]
        if check_fwd:
            pairs = [("o", out["o"], ref["o"]), ("lse", out["lse"], ref["lse"])] + pairs
        for name, g, r in pairs:
            assert_close(name, to_np64(g), r, "fp32" if name == "lse" and w.dtype != "fp32" else w.dtype)
        return out, ref
    res = oracle.grads_for_groups(q, k, v, do, w.causal, w.scale, groups, jobs=jobs, window=w.window)
    G = w.group
    got = {key: [] for key in ("o", "lse", "dq", "dk", "dv")}
    exp = {key: [] for key in got}
    for (b, g), r in res.items():
        hs = slice(g * G, (g + 1) * G)
        for key, t in (("o", out["o"][b, hs]), ("lse", out["lse"][b, hs]), ("dq", out["dq"][b, hs]),
                       ("dk", out["dk"][b, g]), ("dv", out["dv"][b, g])):
            got[key].append(to_np64(t).ravel())
            exp[key].append(r[key].ravel())
    names = ("o", "lse", "dq", "dk", "dv") if check_fwd else ("dq", "dk", "dv")
    for key in names:
        assert_close(key, np.concatenate(got[key]), np.concatenate(exp[key]),
                     "fp32" if key == "lse" and w.dtype != "fp32" else w.dtype)
    return out, res
