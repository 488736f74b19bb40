"""The C ABI on the CPU: the library loads, exports every symbol include/fab.h declares, and
rejects invalid arguments before touching the GPU (no device is needed for these paths)."""
import ctypes
import os
import re

import pytest

import flashattention_backward_amd as fab

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fab.h")).read()
    return sorted(set(re.findall(r"\b(fab_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = fab.lib()
    names = declared_functions()
    assert {"fab_fwd", "fab_bwd", "fab_bwd_preprocess", "fab_bwd_workspace_bytes",
            "fab_last_error", "fab_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert b"gfx950" in L.fab_version()


def test_workspace_bytes():
    L = fab.lib()
    # recompute mode: {lse * log2(e), D} per row, rows padded to 64, bytes rounded up to 256
    assert L.fab_bwd_workspace_bytes_min(2, 32, 8, 4096, 4096, 128, 2) == 2 * 32 * 4096 * 8
    assert L.fab_bwd_workspace_bytes_min(1, 1, 1, 3, 5, 64, 2) == 512
    # stored dS: the statistics to a 4 KB boundary, then per (b, h) Sq rounded up to 128 times
    # Sk rounded up to 256 16-bit values
    assert L.fab_bwd_workspace_bytes_ds(2, 32, 8, 4096, 4096, 128, 2) == 2 * 32 * 4096 * 8 + 64 * 4096 * 4096 * 2
    assert L.fab_bwd_workspace_bytes_ds(1, 3, 1, 130, 300, 64, 1) == 8192 + 3 * 256 * 512 * 2  # 4608 B of statistics
    assert L.fab_bwd_workspace_bytes_ds(1, 1, 1, 3, 5, 64, 0) == 0                        # no stored dS in fp32
    # recommended: stored dS from head dim 96 up, unless both recomputing grids fit one launch
    assert L.fab_bwd_workspace_bytes(2, 32, 8, 4096, 4096, 128, 2) == L.fab_bwd_workspace_bytes_ds(2, 32, 8, 4096, 4096, 128, 2)
    assert L.fab_bwd_workspace_bytes(2, 32, 8, 4096, 4096, 96, 2) == L.fab_bwd_workspace_bytes_ds(2, 32, 8, 4096, 4096, 96, 2)
    assert L.fab_bwd_workspace_bytes(2, 32, 8, 4096, 4096, 64, 2) == L.fab_bwd_workspace_bytes_min(2, 32, 8, 4096, 4096, 64, 2)
    assert L.fab_bwd_workspace_bytes(1, 8, 2, 300, 300, 128, 2) == L.fab_bwd_workspace_bytes_min(1, 8, 2, 300, 300, 128, 2)
    # float32 has no stored-dS mode; too large a dS buffer (here 64 GiB) falls back as well
    assert L.fab_bwd_workspace_bytes(1, 1, 1, 3, 5, 64, 0) == 512
    assert L.fab_bwd_workspace_bytes(1, 3, 3, 65, 5, 64, 0) == 3 * 128 * 8
    assert L.fab_bwd_workspace_bytes_ds(1, 2, 2, 131072, 131072, 128, 2) == 0  # a 64 GiB dS buffer
    assert L.fab_bwd_workspace_bytes(1, 2, 2, 131072, 131072, 128, 2) == L.fab_bwd_workspace_bytes_min(1, 2, 2, 131072, 131072, 128, 2)
    assert L.fab_bwd_workspace_bytes(1, 3, 2, 3, 5, 64, 0) == 0    # H % H_kv != 0
    assert L.fab_bwd_workspace_bytes(1, 1, 1, 3, 5, 80, 0) == 0    # head dim
    assert L.fab_bwd_workspace_bytes(1, 1, 1, 3, 5, 256, 0) == 0   # head dim 256 in fp32
    assert L.fab_bwd_workspace_bytes(1, 1, 1, 3, 5, 256, 2) > 0    # ... but not in bf16
    assert L.fab_bwd_workspace_bytes(1, 1, 1, 3, 5, 96, 1) > 0
    assert L.fab_bwd_workspace_bytes(1, 1, 1, 3, 5, 64, 9) == 0    # dtype


def test_plan():
    """The launch sequence follows the workspace size, the dtype and the problem size."""
    L = fab.lib()
    big = (2, 32, 8, 4096, 4096, 128, 2)
    assert L.fab_bwd_plan(*big, L.fab_bwd_workspace_bytes_ds(*big)) == 2            # stored dS
    assert L.fab_bwd_plan(*big, L.fab_bwd_workspace_bytes_min(*big)) == 0           # recompute
    assert L.fab_bwd_plan(*big, L.fab_bwd_workspace_bytes(*big)) == 2               # recommended
    small = (1, 8, 8, 1024, 1024, 64, 2)                                            # 64 + 64 workgroups
    assert L.fab_bwd_plan(*small, L.fab_bwd_workspace_bytes(*small)) == 1
    assert L.fab_bwd_plan(*small, L.fab_bwd_workspace_bytes_ds(*small)) == 2
    assert L.fab_bwd_plan(1, 2, 2, 128, 128, 64, 0, 1 << 20) == 3                   # float32
    assert L.fab_bwd_plan(*big, 16) == -1                                           # too small
    assert L.fab_bwd_plan(1, 3, 2, 8, 8, 64, 2, 1 << 20) == -1                      # H % H_kv
    assert fab.bwd_plan(*big, L.fab_bwd_workspace_bytes(*big)) == "stored_ds"


P = 1 << 20  # a fake, 16-byte aligned address: validation must fail before using it


def bwd(**kw):
    a = dict(dO=P, q=P, k=P, v=P, o=P, lse=P, dq=P, dk=P, dv=P, ws=P, ws_bytes=1 << 40,
             B=1, H=4, H_kv=2, Sq=16, Sk=16, D=64, dtype=2, causal=1, window=0, scale=0.125)
    a.update(kw)
    L = fab.lib()
    st = L.fab_bwd(a["dO"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["dq"], a["dk"], a["dv"],
                   a["ws"], a["ws_bytes"], a["B"], a["H"], a["H_kv"], a["Sq"], a["Sk"], a["D"],
                   a["dtype"], a["causal"], a["window"], a["scale"], None)
    return st, L.fab_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dtype=3), 2, "dtype"),
    (dict(D=80), 2, "head_dim"),
    (dict(D=256, dtype=0), 2, "head_dim"),
    (dict(D=0), 1, "dims"),
    (dict(B=0), 1, "dims"),
    (dict(Sq=0), 1, "dims"),
    (dict(Sk=-1), 1, "dims"),
    (dict(H=3), 1, "num_kv_heads"),
    (dict(q=0), 1, "q: null"),
    (dict(dv=0), 1, "dv: null"),
    (dict(lse=P + 4), 1, "lse: pointer"),
    (dict(k=P + 8), 1, "k: pointer"),
    (dict(ws_bytes=10), 1, "workspace"),
    (dict(scale=float("inf")), 1, "scale"),
    (dict(scale=float("nan")), 1, "scale"),
    (dict(window=-1), 1, "window_size"),
    (dict(B=4096, Sq=65536, D=128, H=8, H_kv=8), 1, "2^31"),
])
def test_bwd_rejects_invalid_arguments(kw, status, needle):
    st, msg = bwd(**kw)
    assert st == status, (st, msg)
    assert needle in msg, msg


def test_fwd_and_preprocess_reject_invalid_arguments():
    L = fab.lib()
    st = L.fab_fwd(P, P, 0, P, P, 1, 2, 1, 8, 8, 64, 1, 0, 0, 0.1, None)
    assert st == 1 and "v: null" in L.fab_last_error().decode()
    st = L.fab_fwd(P, P, P, P, P, 1, 2, 1, 8, 8, 64, 1, 0, 0, float("nan"), None)
    assert st == 1 and "scale" in L.fab_last_error().decode()
    st = L.fab_fwd(P, P, P, P, P, 1, 2, 1, 8, 8, 64, 1, 1, -3, 0.1, None)
    assert st == 1 and "window_size" in L.fab_last_error().decode()
    st = L.fab_bwd_preprocess(P, P, P + 2, P, 1 << 30, 1, 2, 8, 128, 0, None)
    assert st == 1 and "lse" in L.fab_last_error().decode()
    st = L.fab_bwd_preprocess(P, P, P, P, 16, 1, 2, 8, 128, 0, None)
    assert st == 1 and "workspace" in L.fab_last_error().decode()
    st = L.fab_bwd_preprocess(P, P, P, P, 1 << 30, 1, 2, 8, 48, 0, None)
    assert st == 2
    st = L.fab_bwd_dkdv(P, P, P, P, P, 1 << 30, P, 0, 1, 2, 1, 8, 8, 64, 2, 1, 0, 0.1, None)
    assert st == 1 and "dv: null" in L.fab_last_error().decode()
    st = L.fab_bwd_dkdv(P, P, P, P, P, 1 << 30, P, P, 1, 2, 1, 8, 8, 64, 2, 1, -1, 0.1, None)
    assert st == 1 and "window_size" in L.fab_last_error().decode()
    st = L.fab_bwd_dq(P, P, P, P, P, 8, P, 1, 2, 1, 8, 8, 64, 2, 1, 0, 0.1, None)
    assert st == 1 and "workspace" in L.fab_last_error().decode()


def test_error_message_is_thread_local():
    import threading
    L = fab.lib()
    bwd(dtype=3)
    seen = {}

    def other():
        seen["msg"] = L.fab_last_error().decode()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "dtype" in L.fab_last_error().decode()


def bwd_noalloc(**kw):
    a = dict(dO=P, q=P, k=P, v=P, o=P, lse=P, dq=P, dk=P, dv=P,
             B=1, H=4, H_kv=2, Sq=16, Sk=16, D=64, dtype=2, causal=1, window=0, scale=0.125)
    a.update(kw)
    L = fab.lib()
    st = L.fab_bwd_noalloc(a["dO"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["dq"], a["dk"],
                           a["dv"], a["B"], a["H"], a["H_kv"], a["Sq"], a["Sk"], a["D"], a["dtype"],
                           a["causal"], a["window"], a["scale"], None)
    return st, L.fab_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    # 2^21 + 64 padded rows of statistics: one row group past the static scratch
    (dict(B=1, H=1, H_kv=1, Sq=(1 << 21) + 1, Sk=16, D=64), 1, "static scratch"),
    (dict(B=33, H=64, H_kv=8, Sq=1000, Sk=1000, D=128), 1, "static scratch"),
    (dict(dtype=3), 2, "dtype"),
    (dict(H=3), 1, "num_kv_heads"),
    (dict(dq=0), 1, "dq: null"),
    (dict(o=P + 4), 1, "o: pointer"),
    (dict(scale=float("nan")), 1, "scale"),
])
def test_bwd_noalloc_rejects_invalid_arguments(kw, status, needle):
    """The no-allocation entry point validates before touching the GPU, including its limit:
    B * num_heads * (Sq rounded up to 64) <= 2^21 rows of statistics."""
    st, msg = bwd_noalloc(**kw)
    assert st == status, (st, msg)
    assert needle in msg, msg


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 2, 8, 64)
    with pytest.raises(ValueError, match="GPU"):
        fab.fwd(q, q, q)
    with pytest.raises(ValueError, match="4-D"):
        fab.bwd(q, q[0], q, q, q, q[..., 0])


def test_binding_fails_loudly_without_the_library(monkeypatch):
    """No fallback: with libfab.so absent, every entry point raises instead of computing."""
    import flashattention_backward_amd as fab
    monkeypatch.setattr(fab, "_lib", None)
    monkeypatch.setattr(fab, "LIB_PATH", os.path.join(os.path.dirname(fab.LIB_PATH), "absent", "libfab.so"))
    with pytest.raises(RuntimeError, match="missing"):
        fab.lib()
    with pytest.raises(RuntimeError, match="missing"):
        fab.bwd_workspace_bytes(1, 1, 1, 8, 8, 64, 2)
