"""Plain fp64 forward and backward of (grouped-query, optionally causal) attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Deliberately slow and obvious:
NumPy float64, queries processed in row blocks only so that an Sq x Sk score matrix never
has to exist whole; no fusion, no reordering beyond what the definitions state.

Definitions followed (cited by page title and section):

* boostr 0.1.0, ``src/ops/cuda/attention/flash_bwd.rs`` (docs.rs), doc comment of
  ``flash_attention_bwd_impl``: the backward is two steps -- (1) a preprocessing step that
  forms D = rowsum(dO * O) for every query row, stored as fp32 ``[B, H, Sq]`` ("Step 1"
  block), and (2) a main step producing dQ, dK and dV ("Step 2" block).  Its allocation
  block fixes the output shapes: dQ like Q, dK and dV ``[B, num_kv_heads, Sk, D]``.  Its
  launch block fixes the default softmax scale 1/sqrt(head_dim) and passes a causal flag.
* boostr 0.1.0, ``src/ops/autograd_attention.rs`` (docs.rs), ``var_flash_attention`` and
  ``FlashAttentionBackward``: the forward returns (output, lse); the backward consumes the
  saved q, k, v, output and lse plus the incoming dO and returns (dq, dk, dv).
* The problem statement this library implements: P = exp(scale * Q K^T - LSE),
  dS = P * (dP - D) with dP = dO V^T, and the contractions dV = P^T dO, dK = scale dS^T Q,
  dQ = scale dS K.

Readings where the pages are silent (each also listed in the design notes):

* LSE is the natural-log log-sum-exp of the scaled scores.
* Causal masking is top-left aligned: query i may attend key j iff j <= i.
* Sliding window.  The autograd_attention.rs page passes a ``window_size`` to both the
  forward and the backward, and flash_bwd.rs's backward rejects any value but 0; neither
  page says what the window keeps.  Read here as: W > 0 keeps W keys per query row i, the
  keys j with i - W < j (the W most recent ones, i itself included, under the causal mask)
  and, without the causal mask, also j < i + W; W = 0 is no window.
* A row with no allowed key (only possible with a window and Sq - Sk >= W) has the empty
  sum's LSE = log 0 = -inf and O = 0; P and dS are 0 on it, so its dQ is 0 and it adds
  nothing to dK, dV.
* Grouped-query heads are contiguous: query head h uses kv head h // (H / H_kv), and dK, dV
  sum the contributions of all query heads of a group.
* dQ and dK carry the factor ``scale`` (the gradient of the function actually computed).
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 512


def kv_head_of(h: int, H: int, H_kv: int) -> int:
    """kv head used by query head ``h`` (contiguous groups of H / H_kv query heads)."""
    if H % H_kv:
        raise ValueError("H must be a multiple of H_kv")
    return h // (H // H_kv)


def allowed_mask(rows: np.ndarray, Sk: int, causal: bool, window: int = 0) -> np.ndarray:
    """Boolean [len(rows), Sk]: True where query row i may attend key j (top-left causal;
    with window W > 0 also i - W < j, and j < i + W when not causal)."""
    if window < 0:
        raise ValueError("window must be >= 0")
    i = np.asarray(rows)[:, None]
    j = np.arange(Sk)[None, :]
    ok = np.ones((len(rows), Sk), dtype=bool)
    if causal:
        ok &= j <= i
    if window > 0:
        ok &= j > i - window
        if not causal:
            ok &= j < i + window
    return ok


def _as64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    B, H, Sq, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k and v must be [B, H_kv, Sk, D] matching q")
    H_kv = k.shape[1]
    if H % H_kv:
        raise ValueError("H must be a multiple of H_kv")
    return B, H, H_kv, Sq, k.shape[2], D


def attention_forward(q, k, v, causal: bool, scale: float, heads=None, row_block: int = ROW_BLOCK,
                      window: int = 0):
    """O = softmax(scale Q K^T restricted to allowed keys) V and the row LSE (natural log).
    A row with no allowed key gets O = 0 and LSE = -inf.

    ``heads``: optional iterable of (b, h) pairs to compute; other rows are left as NaN.
    Returns (O [B,H,Sq,D] float64, LSE [B,H,Sq] float64).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, H_kv, Sq, Sk, D = _check_shapes(q, k, v)
    o = np.full((B, H, Sq, D), np.nan)
    lse = np.full((B, H, Sq), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    for b, h in pairs:
        g = kv_head_of(h, H, H_kv)
        for i0 in range(0, Sq, row_block):
            rows = np.arange(i0, min(Sq, i0 + row_block))
            s = scale * (q[b, h, rows] @ k[b, g].T)                 # scaled scores
            ok = allowed_mask(rows, Sk, causal, window)
            s = np.where(ok, s, -np.inf)
            has = ok.any(axis=1, keepdims=True)                      # rows with >= 1 key
            m = np.where(has, s.max(axis=1, keepdims=True), 0.0)
            l = np.exp(s - m).sum(axis=1, keepdims=True)             # 0 for a row with no key
            with np.errstate(divide="ignore"):
                row_lse = m + np.log(l)                              # log 0 = -inf there
            p = np.where(ok, np.exp(np.where(ok, s, 0.0) - np.where(has, row_lse, 0.0)), 0.0)
            o[b, h, rows] = p @ v[b, g]
            lse[b, h, rows] = row_lse[:, 0]
    return o, lse


def attention_backward(do, q, k, v, o, lse, causal: bool, scale: float, groups=None,
                       row_block: int = ROW_BLOCK, window: int = 0):
    """The two-step backward: D = rowsum(dO * O), then dQ, dK, dV from P recomputed via LSE.

    ``groups``: optional iterable of (b, g) kv-head groups to compute; rows of other groups
    are left as NaN.  Returns (dQ [B,H,Sq,D], dK [B,H_kv,Sk,D], dV [B,H_kv,Sk,D],
    D [B,H,Sq]), all float64.
    """
    do, q, k, v, o, lse = (_as64(x) for x in (do, q, k, v, o, lse))
    B, H, H_kv, Sq, Sk, D = _check_shapes(q, k, v)
    G = H // H_kv
    # Step 1 (preprocessing): D_i = sum_d dO_{i,d} O_{i,d}
    delta = np.sum(do * o, axis=-1)
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    glist = [(b, g) for b in range(B) for g in range(H_kv)] if groups is None else list(groups)
    for b, g in glist:
        dk[b, g] = 0.0
        dv[b, g] = 0.0
        for h in range(g * G, (g + 1) * G):
            for i0 in range(0, Sq, row_block):
                rows = np.arange(i0, min(Sq, i0 + row_block))
                ok = allowed_mask(rows, Sk, causal, window)
                s = scale * (q[b, h, rows] @ k[b, g].T)
                # P on allowed pairs only; a row with no allowed key (LSE = -inf) is all zero
                lse_r = lse[b, h, rows][:, None]
                p = np.where(ok, np.exp(np.where(ok, s - lse_r, 0.0)), 0.0)
                dp = do[b, h, rows] @ v[b, g].T
                ds = p * (dp - delta[b, h, rows][:, None])
                dv[b, g] += p.T @ do[b, h, rows]
                dk[b, g] += scale * (ds.T @ q[b, h, rows])
                dq[b, h, rows] = scale * (ds @ k[b, g])
    return dq, dk, dv, delta


def attention_grads(q, k, v, do, causal: bool, scale: float, groups=None, window: int = 0):
    """Forward then backward on the same inputs (the end-to-end comparison).

    Returns a dict with o, lse, dq, dk, dv, delta (float64).  With ``groups`` only the
    listed (b, g) kv-head groups (and their query heads) are computed.
    """
    q64, k64, v64, do64 = (_as64(x) for x in (q, k, v, do))
    B, H, H_kv, Sq, Sk, D = _check_shapes(q64, k64, v64)
    G = H // H_kv
    heads = None
    if groups is not None:
        groups = list(groups)
        heads = [(b, h) for b, g in groups for h in range(g * G, (g + 1) * G)]
    o, lse = attention_forward(q64, k64, v64, causal, scale, heads=heads, window=window)
    if heads is not None:
        # rows outside the requested groups stay NaN; give the backward finite placeholders
        o = np.where(np.isnan(o), 0.0, o)
        lse = np.where(np.isnan(lse), 0.0, lse)
    dq, dk, dv, delta = attention_backward(do64, q64, k64, v64, o, lse, causal, scale,
                                           groups=groups, window=window)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "delta": delta}


def _worker(args):
    q, k, v, do, causal, scale, group, window = args
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        return group, attention_grads(q, k, v, do, causal, scale, groups=[group], window=window)


def _serial(args):
    q, k, v, do, causal, scale, group, window = args
    return group, attention_grads(q, k, v, do, causal, scale, groups=[group], window=window)


def grads_for_groups(q, k, v, do, causal: bool, scale: float, groups, jobs: int = 1,
                     window: int = 0, start_method: str = "fork"):
    """attention_grads over several (b, g) groups, optionally in a process pool.

    With jobs > 1 each worker process receives only its group's slices and uses one BLAS
    thread ("spawn" starts clean interpreters, for callers whose process holds state a
    forked child should not inherit); with jobs <= 1 the groups run one after another in
    this process.  Returns
    {(b, g): result dict with the group's slices: o, lse, delta [G,Sq(,D)], dq [G,Sq,D],
    dk, dv [Sk,D]}.
    """
    q64, k64, v64, do64 = (_as64(x) for x in (q, k, v, do))
    B, H, H_kv, Sq, Sk, D = _check_shapes(q64, k64, v64)
    G = H // H_kv
    tasks = []
    for b, g in groups:
        hs = slice(g * G, (g + 1) * G)
        tasks.append((q64[b:b + 1, hs], k64[b:b + 1, g:g + 1], v64[b:b + 1, g:g + 1],
                      do64[b:b + 1, hs], causal, scale, (0, 0), window))
    if jobs <= 1:
        outs = [_serial(t)[1] for t in tasks]  # one process, BLAS threads as configured
    else:
        import multiprocessing as mp
        ctx = mp.get_context(start_method)
        pool = ctx.Pool(jobs)
        try:
            outs = [r[1] for r in pool.map(_worker, tasks)]
        finally:
            pool.close()  # let the workers exit on their own (no SIGTERM from terminate())
            pool.join()
    res = {}
    for (b, g), out in zip(groups, outs):
        res[(b, g)] = {"o": out["o"][0], "lse": out["lse"][0], "delta": out["delta"][0],
                       "dq": out["dq"][0], "dk": out["dk"][0, 0], "dv": out["dv"][0, 0]}
    return res
