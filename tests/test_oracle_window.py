"""Pins for the oracle's sliding window (``window_size``), each against something other than
the oracle's own mask: finite differences of a pure-Python forward, PyTorch's band
matrices (``tril``/``triu``) under fp64 autograd, closed forms, and invariants.

Reading pinned (the pages pass the argument but do not define it): W > 0 keeps W keys per
query row i, keys j with i - W < j (and j < i + W without the causal mask); rows left with no
key get O = 0, LSE = -inf and no gradient.
"""
import math

import numpy as np
import pytest

from oracle import attention_forward, attention_grads


def rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def inputs(B, H, H_kv, Sq, Sk, D, seed):
    return (rand((B, H, Sq, D), seed), rand((B, H_kv, Sk, D), seed + 1),
            rand((B, H_kv, Sk, D), seed + 2), rand((B, H, Sq, D), seed + 3))


def brute_forward(q, k, v, causal, scale, window):
    """Pure-Python loops: each row's key list is built by walking back (and, without the causal
    mask, forward) at most window - 1 positions from the row's own index."""
    B, H, Sq, D = q.shape
    H_kv, Sk = k.shape[1], k.shape[2]
    G = H // H_kv
    o = np.zeros((B, H, Sq, D))
    lse = np.full((B, H, Sq), -math.inf)
    for b in range(B):
        for h in range(H):
            g = h // G
            for i in range(Sq):
                back = range(i, i - window, -1)
                ahead = range(i + 1, i + window) if not causal else range(0)
                keys = [j for j in list(back) + list(ahead) if 0 <= j < Sk]
                if not keys:
                    continue
                s = [scale * sum(q[b, h, i, d] * k[b, g, j, d] for d in range(D)) for j in keys]
                mx = max(s)
                lse[b, h, i] = mx + math.log(sum(math.exp(x - mx) for x in s))
                for d in range(D):
                    o[b, h, i, d] = sum(math.exp(x - lse[b, h, i]) * v[b, g, j, d]
                                        for x, j in zip(s, keys))
    return o, lse


FD_CASES = [
    # (B, H, H_kv, Sq, Sk, D, causal, window)
    (1, 2, 1, 6, 6, 3, True, 2),
    (1, 2, 2, 5, 7, 2, False, 2),
    (1, 2, 1, 7, 3, 2, True, 3),   # rectangular: rows 5 and 6 keep no key
]


@pytest.mark.parametrize("case", FD_CASES)
def test_window_forward_matches_brute_force(case):
    B, H, H_kv, Sq, Sk, D, causal, W = case
    q, k, v, _ = inputs(B, H, H_kv, Sq, Sk, D, 200)
    o, lse = attention_forward(q, k, v, causal, 0.7, row_block=2, window=W)
    o2, lse2 = brute_forward(q, k, v, causal, 0.7, W)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(lse2))
    fin = np.isfinite(lse2)
    np.testing.assert_allclose(lse[fin], lse2[fin], rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", FD_CASES)
def test_window_backward_central_finite_differences(case):
    """L = sum(W_o * O); every element of dQ, dK, dV against central differences of the
    pure-Python forward."""
    B, H, H_kv, Sq, Sk, D, causal, W = case
    q, k, v, wo = inputs(B, H, H_kv, Sq, Sk, D, 210)
    r = attention_grads(q, k, v, wo, causal, 0.8, window=W)
    eps = 1e-6

    def loss(q, k, v):
        return float(np.sum(wo * brute_forward(q, k, v, causal, 0.8, W)[0]))

    for name, x, g in (("q", q, r["dq"]), ("k", k, r["dk"]), ("v", v, r["dv"])):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args_p, args_m = {"q": q, "k": k, "v": v}, {"q": q, "k": k, "v": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(**args_p) - loss(**args_m)) / (2 * eps)
        assert np.all(np.abs(num - g) <= 1e-7 * np.maximum(1.0, np.abs(g))), name


@pytest.mark.parametrize("causal,W", [(True, 1), (True, 5), (False, 3), (False, 8)])
def test_window_against_torch_band_matrix(causal, W):
    """PyTorch fp64 CPU autograd with the band built by tril/triu: keys up to W - 1 behind the
    row (and up to W - 1 ahead without the causal mask)."""
    torch = pytest.importorskip("torch")
    B, H, H_kv, Sq, Sk, D = 1, 4, 2, 17, 21, 6
    G = H // H_kv
    q, k, v, do = inputs(B, H, H_kv, Sq, Sk, D, 220)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    band = torch.ones(Sq, Sk, dtype=torch.bool).triu(-(W - 1))
    band = band.tril(0) if causal else band.tril(W - 1)
    s = 0.35 * torch.matmul(tq, tk.repeat_interleave(G, 1).transpose(-1, -2).contiguous())
    s = s.masked_fill(~band, float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), tv.repeat_interleave(G, 1))
    o.backward(torch.tensor(do))
    r = attention_grads(q, k, v, do, causal, 0.35, window=W)
    np.testing.assert_allclose(r["o"], o.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(r["lse"], torch.logsumexp(s, dim=-1).detach().numpy(), atol=1e-12)
    for key, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        np.testing.assert_allclose(r[key], t.grad.numpy(), atol=1e-12, err_msg=key)


def test_window_of_one_closed_form():
    """Causal, W = 1, Sq = Sk: every row sees only its own key, so O_i = V_i,
    LSE_i = scale q_i . k_i, dQ = dK = 0 and dV_i = sum over the group's heads of dO_i."""
    B, H, H_kv, S, D = 2, 4, 2, 9, 5
    q, k, v, do = inputs(B, H, H_kv, S, S, D, 230)
    r = attention_grads(q, k, v, do, True, 0.6, window=1)
    ke, ve = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    np.testing.assert_allclose(r["o"], ve, atol=1e-14)
    np.testing.assert_allclose(r["lse"], 0.6 * np.sum(q * ke, axis=-1), atol=1e-13)
    np.testing.assert_allclose(r["dq"], 0.0, atol=1e-13)
    np.testing.assert_allclose(r["dk"], 0.0, atol=1e-13)
    np.testing.assert_allclose(r["dv"], do.reshape(B, H_kv, 2, S, D).sum(axis=2), atol=1e-13)


@pytest.mark.parametrize("causal,W", [(True, 3), (False, 3), (True, 1)])
def test_window_identical_keys_counts_the_window(causal, W):
    """All keys equal: P is uniform over the row's keys, so LSE_i = scale q_i.k + log n_i and
    O_i is the mean of those keys' V rows, n_i = the number of keys the window keeps."""
    S, D = 11, 3
    q, v = rand((1, 1, S, D), 240), rand((1, 1, S, D), 241)
    k = np.broadcast_to(rand((1, 1, 1, D), 242), (1, 1, S, D)).copy()
    o, lse = attention_forward(q, k, v, causal, 1.0, window=W)
    for i in range(S):
        lo = max(0, i - W + 1)
        hi = i if causal else min(S - 1, i + W - 1)
        n = hi - lo + 1
        np.testing.assert_allclose(lse[0, 0, i], q[0, 0, i] @ k[0, 0, 0] + math.log(n), atol=1e-13)
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, lo:hi + 1].mean(axis=0), atol=1e-13)


def test_window_boundary_locality():
    """Row i depends on key i - W + 1 but not on key i - W (or anything older)."""
    S, D, W = 12, 4, 4
    q, k, v, _ = inputs(1, 1, 1, S, S, D, 250)
    o, _ = attention_forward(q, k, v, True, 0.5, window=W)
    i = 9
    k_old, v_old = k.copy(), v.copy()
    k_old[0, 0, :i - W + 1] += 3.0
    v_old[0, 0, :i - W + 1] -= 2.0
    o_old, _ = attention_forward(q, k_old, v_old, True, 0.5, window=W)
    np.testing.assert_array_equal(o_old[0, 0, i], o[0, 0, i])
    k_edge = k.copy()
    k_edge[0, 0, i - W + 1] += 3.0
    o_edge, _ = attention_forward(q, k_edge, v, True, 0.5, window=W)
    assert np.max(np.abs(o_edge[0, 0, i] - o[0, 0, i])) > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_wide_window_is_no_window(causal):
    B, H, H_kv, Sq, Sk, D = 1, 2, 1, 9, 13, 4
    q, k, v, do = inputs(B, H, H_kv, Sq, Sk, D, 260)
    r0 = attention_grads(q, k, v, do, causal, 0.5)
    rw = attention_grads(q, k, v, do, causal, 0.5, window=max(Sq, Sk))
    for key in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_array_equal(rw[key], r0[key], err_msg=key)
    # the narrowest window that still cuts a pair: causal rows see at most Sq keys
    rn = attention_grads(q, k, v, do, causal, 0.5, window=(Sq if causal else max(Sq, Sk)) - 1)
    assert np.max(np.abs(rn["dk"] - r0["dk"])) > 1e-6


@pytest.mark.parametrize("causal", [False, True])
def test_rows_without_keys(causal):
    """Sq - Sk >= W leaves rows i >= Sk + W - 1 without keys: O = 0, LSE = -inf, dQ = 0, and
    dK, dV equal those of the same problem with those rows removed."""
    B, H, H_kv, Sq, Sk, D, W = 1, 2, 1, 10, 4, 3, 3
    q, k, v, do = inputs(B, H, H_kv, Sq, Sk, D, 270)
    r = attention_grads(q, k, v, do, causal, 0.5, window=W)
    first_empty = Sk + W - 1
    assert np.all(r["o"][:, :, first_empty:] == 0.0)
    assert np.all(np.isneginf(r["lse"][:, :, first_empty:]))
    assert np.all(np.isfinite(r["lse"][:, :, :first_empty]))
    assert np.all(r["dq"][:, :, first_empty:] == 0.0)
    cut = attention_grads(q[:, :, :first_empty], k, v, do[:, :, :first_empty], causal, 0.5, window=W)
    np.testing.assert_allclose(r["dk"], cut["dk"], atol=1e-14)
    np.testing.assert_allclose(r["dv"], cut["dv"], atol=1e-14)
    np.testing.assert_allclose(r["dq"][:, :, :first_empty], cut["dq"], atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_window_invariants(causal):
    """Shift invariance (sum_j dK_j = 0), row-stochastic P (sum_j dV_j = sum of dO over rows
    that keep a key), Q/K scaling symmetry."""
    B, H, H_kv, Sq, Sk, D, W = 1, 4, 2, 15, 9, 5, 4
    q, k, v, do = inputs(B, H, H_kv, Sq, Sk, D, 280)
    r = attention_grads(q, k, v, do, causal, 0.4, window=W)
    G = H // H_kv
    np.testing.assert_allclose(r["dk"].sum(axis=2), 0.0, atol=1e-12)
    kept = np.isfinite(r["lse"])[..., None]
    np.testing.assert_allclose(r["dv"].sum(axis=2),
                               (do * kept).reshape(B, H_kv, G, Sq, D).sum(axis=(2, 3)), atol=1e-12)
    lhs = (q * r["dq"]).reshape(B, H_kv, G, Sq, D).sum(axis=(2, 3, 4))
    np.testing.assert_allclose(lhs, (k * r["dk"]).sum(axis=(2, 3)), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("W", [1, 7, 16])
def test_window_span_determines_its_rows_and_keys(W):
    """What the maximum-size GPU test relies on: for causal attention with a window, the
    oracle on a span of positions gives the full sequence's O, LSE, dQ on the span's exact
    rows and dK, dV on its exact keys (window_span_ranges), at the start, inside, and at the
    end of the sequence."""
    from parity_helpers import window_span_ranges
    B, H, H_kv, S, D = 1, 4, 2, 90, 8
    q, k, v, do = inputs(B, H, H_kv, S, S, D, 290 + W)
    full = attention_grads(q, k, v, do, True, 0.35, window=W)
    n = 3 * W + 5
    for c, e in ((0, n), (31, 31 + n), (S - n, S)):
        (r0, r1), (k0, k1) = window_span_ranges(c, e, S, W)
        assert r1 > r0 and k1 > k0
        part = attention_grads(q[:, :, c:e], k[:, :, c:e], v[:, :, c:e], do[:, :, c:e], True, 0.35,
                               window=W)
        for key, a, b in (("o", r0, r1), ("lse", r0, r1), ("dq", r0, r1), ("dk", k0, k1), ("dv", k0, k1)):
            np.testing.assert_allclose(part[key][:, :, a - c:b - c], full[key][:, :, a:b],
                                       rtol=1e-12, atol=1e-13, err_msg=f"{key} span {c}:{e}")
    # with W > 1, the row before and the key after those ranges differ: the ranges are tight
    # (with W = 1 a row sees only its own key and every row and key of a span is exact)
    if W > 1:
        c, e = 31, 31 + n
        (r0, _), (_, k1) = window_span_ranges(c, e, S, W)
        part = attention_grads(q[:, :, c:e], k[:, :, c:e], v[:, :, c:e], do[:, :, c:e], True, 0.35,
                               window=W)
        assert not np.allclose(part["o"][:, :, r0 - 1 - c], full["o"][:, :, r0 - 1])
        assert not np.allclose(part["dv"][:, :, k1 - c], full["dv"][:, :, k1])
