"""Plain token-by-token FP64 oracle for the GDN-2 backward pass (numpy).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``). Pinned by
``tests/test_oracle_bwd_pins.py``: central finite differences of the forward
oracle (itself pinned by ``tests/test_oracle_pins.py``), and the closed-form
gradients of ungated linear attention.

What is differentiated: the forward recurrence of the FlashInfer
``chunk_gated_delta_rule2`` docs (recurrence display equation), exactly as
:mod:`oracle.recurrence` runs it, per value head and token t:

    Sd_t   = diag(exp(g_t)) S_{t-1}          decayed state
    e_t    = Sd_t^T (beta_t * k_t)           erase read
    vnew_t = w_t * v_t - e_t
    S_t    = Sd_t + k_t vnew_t^T
    o_t    = scale * S_t^T q_t

For a scalar loss with dL/do_t = do_t and dL/dS_T = dS_T, the reverse sweep
(chain rule through the five lines above, last line first) is, with dS the
gradient with respect to S_t accumulated from later tokens:

    dS      += scale * q_t do_t^T             ;  dq_t  = scale * S_t do_t
    dvnew    = dS^T k_t                       ;  dk_t  = dS vnew_t
    dw_t     = dvnew * v_t ;  dv_t = dvnew * w_t ;  de = -dvnew
    dbk      = Sd_t de                        ;  dbeta_t = dbk * k_t ;  dk_t += dbk * beta_t
    dSd      = dS + (beta_t * k_t) de^T
    dg_t     = rowsum(dSd * Sd_t)             (d exp(g)/dg = exp(g))
    dS       = diag(exp(g_t)) dSd             (the gradient with respect to S_{t-1})

and dS after the first token is the gradient of the initial state. Grouped
value heads: dq and dk of a q/k head are the sums over the value heads that
read it (contiguous groups, as in the forward oracle).
"""

from __future__ import annotations

import numpy as np

from .recurrence import _f64, resolve_scale


def gdn2_sequence_bwd(q, k, v, g, beta, w, scale, S0, do, dST):
    """Gradients of ONE sequence, all value heads at once (float64 arrays,
    already gathered per value head).

    Shapes: q, k, g, beta [L, HV, K]; v, w, do [L, HV, V]; S0, dST [HV, K, V].
    Returns dq, dk, dg, dbeta [L, HV, K], dv, dw [L, HV, V], dS0 [HV, K, V]
    (dq, dk per value head).
    """
    L = q.shape[0]
    # forward, keeping the state entering every token
    S_prev = np.empty((L,) + S0.shape)
    S = S0.copy()
    for t in range(L):
        S_prev[t] = S
        Sd = S * np.exp(g[t])[:, :, None]
        vnew = w[t] * v[t] - np.einsum("hk,hkv->hv", beta[t] * k[t], Sd)
        S = Sd + k[t][:, :, None] * vnew[:, None, :]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dg = np.zeros_like(g)
    dbeta = np.zeros_like(beta)
    dv = np.zeros_like(v)
    dw = np.zeros_like(w)
    dS = dST.copy()
    for t in range(L - 1, -1, -1):
        a = np.exp(g[t])
        Sd = S_prev[t] * a[:, :, None]
        bk = beta[t] * k[t]
        vnew = w[t] * v[t] - np.einsum("hk,hkv->hv", bk, Sd)
        St = Sd + k[t][:, :, None] * vnew[:, None, :]
        # o_t = scale * S_t^T q_t
        dq[t] = scale * np.einsum("hkv,hv->hk", St, do[t])
        dS = dS + scale * q[t][:, :, None] * do[t][:, None, :]
        # S_t = Sd + k vnew^T
        dvnew = np.einsum("hkv,hk->hv", dS, k[t])
        dk[t] = np.einsum("hkv,hv->hk", dS, vnew)
        # vnew = w * v - Sd^T (beta * k)
        dw[t] = dvnew * v[t]
        dv[t] = dvnew * w[t]
        de = -dvnew
        dbk = np.einsum("hkv,hv->hk", Sd, de)
        dbeta[t] = dbk * k[t]
        dk[t] += dbk * beta[t]
        dSd = dS + bk[:, :, None] * de[:, None, :]
        # Sd = diag(exp(g)) S_{t-1}
        dg[t] = np.sum(dSd * Sd, axis=2)
        dS = dSd * a[:, :, None]
    return dq, dk, dg, dbeta, dv, dw, dS


def gdn2_recurrence_bwd(q, k, v, g, beta, w, scale, initial_state, cu_seqlens, d_out,
                        d_final_state=None):
    """FP64 oracle of the GDN-2 backward over packed (varlen) sequences.

    Arguments as :func:`oracle.recurrence.gdn2_recurrence` (g, beta, w
    required here), plus d_out [T, HV, V] and d_final_state [N, HV, K, V] or
    None (zero). Returns a dict of float64 arrays: dq, dk [T, H, K] (summed
    over the value heads of each q/k head), dv, dw [T, HV, V], dg, dbeta
    [T, HV, K], d_initial_state [N, HV, K, V].
    """
    q, k, v, g, beta, w = (_f64(x) for x in (q, k, v, g, beta, w))
    do = _f64(d_out)
    T, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    if HV % H != 0:
        raise ValueError("HV must be a multiple of H")
    m = HV // H
    scale = resolve_scale(scale, K)
    cu = np.array([0, T], dtype=np.int64) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    S0_all = np.zeros((N, HV, K, V)) if initial_state is None else _f64(initial_state)
    dST_all = np.zeros((N, HV, K, V)) if d_final_state is None else _f64(d_final_state)
    hk = np.arange(HV) // m
    res = {"dq": np.zeros((T, H, K)), "dk": np.zeros((T, H, K)), "dv": np.zeros((T, HV, V)),
           "dw": np.zeros((T, HV, V)), "dg": np.zeros((T, HV, K)), "dbeta": np.zeros((T, HV, K)),
           "d_initial_state": np.zeros((N, HV, K, V))}
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        dq, dk, dg, dbeta, dv, dw, dS0 = gdn2_sequence_bwd(
            q[a:b][:, hk], k[a:b][:, hk], v[a:b], g[a:b], beta[a:b], w[a:b], scale,
            S0_all[n], do[a:b], dST_all[n])
        for h in range(H):
            res["dq"][a:b, h] = dq[:, h * m:(h + 1) * m].sum(axis=1)
            res["dk"][a:b, h] = dk[:, h * m:(h + 1) * m].sum(axis=1)
        res["dv"][a:b], res["dw"][a:b] = dv, dw
        res["dg"][a:b], res["dbeta"][a:b] = dg, dbeta
        res["d_initial_state"][n] = dS0
    return res
