"""Pins for the fp64 oracle: each check ties it to something other than itself.

A plausible slip anywhere in the oracle (a dropped ``scale``, a wrong sign in dS, a
transposed operand, a wrong causal direction, natural-vs-base-2 LSE, interleaved instead of
contiguous kv-head groups, a row-blocking bug) fails at least one of these.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention_backward, attention_forward, attention_grads, grads_for_groups

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def brute_forward(q, k, v, causal, scale):
    """Pure-Python loops over the definition: the independent forward used for FD."""
    B, H, Sq, D = q.shape
    H_kv, Sk = k.shape[1], k.shape[2]
    G = H // H_kv
    o = np.zeros((B, H, Sq, D))
    lse = np.zeros((B, H, Sq))
    for b in range(B):
        for h in range(H):
            g = h // G
            for i in range(Sq):
                keys = [j for j in range(Sk) if (not causal) or j <= i]
                s = [scale * sum(q[b, h, i, d] * k[b, g, j, d] for d in range(D)) for j in keys]
                mx = max(s)
                z = sum(math.exp(x - mx) for x in s)
                lse[b, h, i] = mx + math.log(z)
                for d in range(D):
                    o[b, h, i, d] = sum(math.exp(x - lse[b, h, i]) * v[b, g, j, d]
                                        for x, j in zip(s, keys))
    return o, lse


FD_CASES = [
    # (B, H, H_kv, Sq, Sk, D, causal)
    (1, 2, 1, 4, 6, 3, False),
    (2, 2, 2, 5, 5, 4, True),
    (1, 4, 2, 6, 3, 2, True),
]


@pytest.mark.parametrize("case", FD_CASES)
def test_forward_matches_brute_force(case):
    B, H, H_kv, Sq, Sk, D, causal = case
    q, k, v = rand((B, H, Sq, D), 1), rand((B, H_kv, Sk, D), 2), rand((B, H_kv, Sk, D), 3)
    scale = 0.7
    o, lse = attention_forward(q, k, v, causal, scale, row_block=2)
    o2, lse2 = brute_forward(q, k, v, causal, scale)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", FD_CASES)
def test_backward_central_finite_differences(case):
    """(N1) L = sum(W * O(Q, K, V)); dO = W.  Every element of dQ, dK, dV against
    (L(x + e) - L(x - e)) / 2e evaluated with the brute-force loop forward."""
    B, H, H_kv, Sq, Sk, D, causal = case
    q, k, v = rand((B, H, Sq, D), 11), rand((B, H_kv, Sk, D), 12), rand((B, H_kv, Sk, D), 13)
    w = rand((B, H, Sq, D), 14)
    scale = 0.8
    r = attention_grads(q, k, v, w, causal, scale)
    eps = 1e-6

    def loss(qq, kk, vv):
        return float(np.sum(w * brute_forward(qq, kk, vv, causal, scale)[0]))

    for name, x, g in (("q", q, r["dq"]), ("k", k, r["dk"]), ("v", v, r["dv"])):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                        loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
        tol = 1e-7 * np.maximum(1.0, np.abs(g))
        assert np.all(np.abs(num - g) <= tol), (name, np.max(np.abs(num - g)))


def test_preprocess_identity():
    """(N2) D_i = rowsum(dO * O) equals sum_j P_ij dP_ij (because O = P V)."""
    B, H, H_kv, Sq, Sk, D = 1, 2, 1, 7, 9, 5
    q, k, v, do = (rand((B, H, Sq, D), 21), rand((B, H_kv, Sk, D), 22),
                   rand((B, H_kv, Sk, D), 23), rand((B, H, Sq, D), 24))
    for causal in (False, True):
        r = attention_grads(q, k, v, do, causal, 0.5)
        o_bf, lse_bf = brute_forward(q, k, v, causal, 0.5)
        for h in range(H):
            s = 0.5 * q[0, h] @ k[0, h // 2].T
            ok = np.tril(np.ones((Sq, Sk), bool)) if causal else np.ones((Sq, Sk), bool)
            p = np.where(ok, np.exp(s - lse_bf[0, h][:, None]), 0.0)
            dp = do[0, h] @ v[0, h // 2].T
            np.testing.assert_allclose(r["delta"][0, h], (p * dp).sum(1), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_expanded_heads(causal):
    """(N3) GQA dK/dV equal the per-group sums of a run with K, V repeated per query head
    (query head h holding kv head h // G); dQ identical."""
    B, H, H_kv, Sq, Sk, D = 2, 6, 2, 9, 11, 4
    G = H // H_kv
    q, k, v, do = (rand((B, H, Sq, D), 31), rand((B, H_kv, Sk, D), 32),
                   rand((B, H_kv, Sk, D), 33), rand((B, H, Sq, D), 34))
    r = attention_grads(q, k, v, do, causal, 0.45)
    ke, ve = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    re = attention_grads(q, ke, ve, do, causal, 0.45)
    np.testing.assert_allclose(r["dq"], re["dq"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["o"], re["o"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dk"], re["dk"].reshape(B, H_kv, G, Sk, D).sum(2), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["dv"], re["dv"].reshape(B, H_kv, G, Sk, D).sum(2), rtol=1e-11, atol=1e-12)


def test_causal_masked_positions_get_zero_gradient():
    """(N4) With dO rows i >= m zeroed, causal dK and dV rows j >= m are exactly zero; and the
    first query row (which sees only key 0) gets dQ = 0 and O = V_0."""
    B, H, H_kv, Sq, Sk, D, m = 1, 2, 2, 10, 10, 4, 6
    q, k, v, do = (rand((B, H, Sq, D), 41), rand((B, H_kv, Sk, D), 42),
                   rand((B, H_kv, Sk, D), 43), rand((B, H, Sq, D), 44))
    do[:, :, m:] = 0.0
    r = attention_grads(q, k, v, do, True, 0.6)
    assert np.all(r["dk"][:, :, m:] == 0.0)
    assert np.all(r["dv"][:, :, m:] == 0.0)
    np.testing.assert_allclose(r["o"][:, :, 0], v[:, :, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(r["dq"][:, :, 0], 0.0, atol=1e-14)
    # the non-causal run does give those rows gradient: the mask is what zeroes them
    rn = attention_grads(q, k, v, do, False, 0.6)
    assert np.max(np.abs(rn["dk"][:, :, m:])) > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    """Shift invariance (sum_j dK_j = 0), row-stochastic P (sum_j dV_j = sum of dO over the
    group), and the Q/K scaling symmetry (sum <Q, dQ> = sum <K, dK> per group)."""
    B, H, H_kv, Sq, Sk, D = 2, 4, 2, 13, 17, 6
    q, k, v, do = (rand((B, H, Sq, D), 51), rand((B, H_kv, Sk, D), 52),
                   rand((B, H_kv, Sk, D), 53), rand((B, H, Sq, D), 54))
    r = attention_grads(q, k, v, do, causal, 0.4)
    G = H // H_kv
    np.testing.assert_allclose(r["dk"].sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(r["dv"].sum(axis=2), do.reshape(B, H_kv, G, Sq, D).sum(axis=(2, 3)),
                               rtol=1e-12, atol=1e-12)
    lhs = (q * r["dq"]).reshape(B, H_kv, G, Sq, D).sum(axis=(2, 3, 4))
    rhs = (k * r["dk"]).sum(axis=(2, 3))
    np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-12)


def test_closed_form_single_key():
    """Sk = 1: O = V_0, LSE = scale q.k_0, dQ = dK = 0, dV_0 = sum_i dO_i."""
    B, H, Sq, D = 1, 3, 5, 4
    q, k, v, do = rand((B, H, Sq, D), 61), rand((B, H, 1, D), 62), rand((B, H, 1, D), 63), rand((B, H, Sq, D), 64)
    r = attention_grads(q, k, v, do, False, 0.3)
    np.testing.assert_allclose(r["o"], np.broadcast_to(v, r["o"].shape), atol=1e-15)
    np.testing.assert_allclose(r["lse"], 0.3 * np.einsum("bhid,bhd->bhi", q, k[:, :, 0]), atol=1e-14)
    np.testing.assert_allclose(r["dq"], 0.0, atol=1e-14)
    np.testing.assert_allclose(r["dk"], 0.0, atol=1e-14)
    np.testing.assert_allclose(r["dv"][:, :, 0], do.sum(axis=2), atol=1e-14)


def test_closed_form_identical_keys():
    """All keys equal: P is uniform over the allowed keys, so O_i is the mean of the allowed
    V rows and LSE_i = scale q_i.k + log(number of allowed keys)."""
    B, H, Sq, Sk, D = 1, 1, 6, 6, 3
    q, v = rand((B, H, Sq, D), 71), rand((B, H, Sk, D), 72)
    k = np.broadcast_to(rand((1, 1, 1, D), 73), (B, H, Sk, D)).copy()
    for causal in (False, True):
        o, lse = attention_forward(q, k, v, causal, 1.0)
        for i in range(Sq):
            n = i + 1 if causal else Sk
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n].mean(axis=0), atol=1e-14)
            np.testing.assert_allclose(lse[0, 0, i], q[0, 0, i] @ k[0, 0, 0] + math.log(n), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_fp64_autograd(causal):
    """Library cross-check: PyTorch fp64 CPU autograd of the explicit matmul/softmax formula."""
    torch = pytest.importorskip("torch")
    B, H, H_kv, Sq, Sk, D = 2, 4, 2, 19, 23, 8
    G = H // H_kv
    q, k, v, do = (rand((B, H, Sq, D), 81), rand((B, H_kv, Sk, D), 82),
                   rand((B, H_kv, Sk, D), 83), rand((B, H, Sq, D), 84))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    ke = tk.repeat_interleave(G, dim=1)
    ve = tv.repeat_interleave(G, dim=1)
    s = 0.35 * torch.matmul(tq, ke.transpose(-1, -2).contiguous())
    if causal:
        s = s.masked_fill(~torch.ones(Sq, Sk, dtype=torch.bool).tril(), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), ve)
    o.backward(torch.tensor(do))
    r = attention_grads(q, k, v, do, causal, 0.35)
    np.testing.assert_allclose(r["o"], o.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse"], torch.logsumexp(s, dim=-1).detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(r["dq"], tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(r["dk"], tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(r["dv"], tv.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("case", ["noncausal", "causal"])
def test_handworked_golden(case):
    with open(os.path.join(GOLDEN, "handworked_two_keys.json")) as f:
        g = json.load(f)[case]
    arr = {key: np.array(val, dtype=np.float64) for key, val in g.items() if isinstance(val, list)}
    r = attention_grads(arr["q"], arr["k"], arr["v"], arr["do"], g["causal"], g["scale"])
    for key in ("o", "lse", "delta", "dq", "dk", "dv"):
        np.testing.assert_allclose(r[key], arr[key], rtol=0, atol=1e-14, err_msg=key)


def test_row_blocking_does_not_change_results():
    B, H, H_kv, Sq, Sk, D = 1, 2, 1, 37, 29, 5
    q, k, v, do = (rand((B, H, Sq, D), 91), rand((B, H_kv, Sk, D), 92),
                   rand((B, H_kv, Sk, D), 93), rand((B, H, Sq, D), 94))
    o1, l1 = attention_forward(q, k, v, True, 0.5, row_block=5)
    o2, l2 = attention_forward(q, k, v, True, 0.5, row_block=1000)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    g1 = attention_backward(do, q, k, v, o1, l1, True, 0.5, row_block=3)
    g2 = attention_backward(do, q, k, v, o2, l2, True, 0.5, row_block=1000)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(a, b, atol=1e-13)


def test_group_subset_matches_full_run():
    """grads_for_groups (used at full sizes and by the CPU baseline) agrees with the full run,
    both serially and in a process pool."""
    B, H, H_kv, Sq, Sk, D = 2, 4, 2, 11, 13, 4
    q, k, v, do = (rand((B, H, Sq, D), 101), rand((B, H_kv, Sk, D), 102),
                   rand((B, H_kv, Sk, D), 103), rand((B, H, Sq, D), 104))
    full = attention_grads(q, k, v, do, True, 0.5)
    groups = [(0, 1), (1, 0)]
    for jobs in (1, 2):
        sub = grads_for_groups(q, k, v, do, True, 0.5, groups, jobs=jobs)
        for (b, g), r in sub.items():
            hs = slice(2 * g, 2 * g + 2)
            np.testing.assert_allclose(r["dq"], full["dq"][b, hs], atol=1e-14)
            np.testing.assert_allclose(r["dk"], full["dk"][b, g], atol=1e-14)
            np.testing.assert_allclose(r["dv"], full["dv"][b, g], atol=1e-14)
            np.testing.assert_allclose(r["lse"], full["lse"][b, hs], atol=1e-14)
