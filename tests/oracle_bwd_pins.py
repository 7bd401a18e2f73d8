"""Pins of the FP64 backward oracle against facts fixed outside its own code.

Each ``pin_*`` takes a callable with the signature of
``oracle.recurrence_bwd.gdn2_recurrence_bwd`` and raises AssertionError when
it disagrees with the fact:

* central finite differences of the (separately pinned) forward oracle, for
  every input, over varlen sequences with grouped value heads;
* the closed-form gradients of ungated linear attention (g = 0, beta = 0,
  w = 1), written with matrix products and prefix / suffix sums instead of a
  reverse recurrence;
* linearity of every gradient in (d_out, d_final_state).
"""

from __future__ import annotations

import numpy as np

from oracle.recurrence import gdn2_recurrence

NAMES = ("q", "k", "v", "g", "beta", "w", "initial_state")
GRADS = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "w": "dw",
         "initial_state": "d_initial_state"}


def rand_case(seed, lengths=(4, 0, 5), H=1, HV=2, K=3, V=2, beta_max=2.0):
    r = np.random.default_rng(seed)
    T = sum(lengths)
    N = len(lengths)
    x = {
        "q": r.standard_normal((T, H, K)) * 0.7,
        "k": r.standard_normal((T, H, K)) * 0.7,
        "v": r.standard_normal((T, HV, V)),
        "g": -r.random((T, HV, K)) * 0.8 + 0.1 * r.standard_normal((T, HV, K)),
        "beta": beta_max * r.random((T, HV, K)),
        "w": r.random((T, HV, V)) * 1.5,
        "initial_state": 0.5 * r.standard_normal((N, HV, K, V)),
    }
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    d_out = r.standard_normal((T, HV, V))
    d_final = r.standard_normal((N, HV, K, V))
    return x, cu, d_out, d_final


def _loss(x, cu, scale, d_out, d_final):
    o, S = gdn2_recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], x["w"], scale,
                           x["initial_state"], cu)
    return float(np.sum(o * d_out) + np.sum(S * d_final))


def pin_finite_differences(bwd, seed=3, eps=1e-6, tol=1e-6):
    """Every gradient against central differences of the forward oracle."""
    x, cu, d_out, d_final = rand_case(seed)
    scale = 0.6
    got = bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["w"], scale, x["initial_state"], cu,
              d_out, d_final)
    for name in NAMES:
        num = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp = {n: a.copy() for n, a in x.items()}
            xm = {n: a.copy() for n, a in x.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            num[idx] = (_loss(xp, cu, scale, d_out, d_final) - _loss(xm, cu, scale, d_out, d_final)) / (2 * eps)
        err = np.max(np.abs(got[GRADS[name]] - num))
        ref = max(1.0, np.max(np.abs(num)))
        assert err <= tol * ref, f"d{name}: max |analytic - finite difference| {err:.3e}"


def pin_linear_attention(bwd, seed=5, T=9, K=4, V=3, tol=1e-11):
    """g = 0, beta = 0, w = 1 is linear attention with a state:
    o = scale (tril(Q K^T) V + Q S0), S_T = S0 + K^T V. Its gradients in
    closed form, with M = tril(dO V^T) and D the gradient of the value update:
      dQ = scale (M K + dO S0^T)        dK = scale M^T Q + V dS_T^T
      D  = scale tril(Q K^T)^T dO + K dS_T        dV = D,  dw = D * V
      dS0 = scale Q^T dO + dS_T
      dbeta_t = -k_t * (S_{t-1} D_t)    dg_t = rowsum(G_t * S_{t-1})
    where S_{t-1} = S0 + sum_{s<t} k_s v_s^T (prefix sum) and
    G_t = dS_T + scale sum_{r>=t} q_r do_r^T (suffix sum)."""
    r = np.random.default_rng(seed)
    Q, Kk, Vv = r.standard_normal((T, K)), r.standard_normal((T, K)), r.standard_normal((T, V))
    S0, dO, dST = r.standard_normal((K, V)), r.standard_normal((T, V)), r.standard_normal((K, V))
    scale = 0.45
    got = bwd(Q[:, None], Kk[:, None], Vv[:, None], np.zeros((T, 1, K)), np.zeros((T, 1, K)),
              np.ones((T, 1, V)), scale, S0[None, None], None, dO[:, None], dST[None, None])
    M = np.tril(dO @ Vv.T)
    dQ = scale * (M @ Kk + dO @ S0.T)
    dK = scale * M.T @ Q + Vv @ dST.T
    D = scale * np.tril(Q @ Kk.T).T @ dO + Kk @ dST
    dS0 = scale * Q.T @ dO + dST
    Sprev = S0[None] + np.concatenate([np.zeros((1, K, V)),
                                       np.cumsum(Kk[:, :, None] * Vv[:, None, :], axis=0)[:-1]])
    G = dST[None] + scale * np.cumsum((Q[:, :, None] * dO[:, None, :])[::-1], axis=0)[::-1]
    dbeta = -Kk * np.einsum("tkv,tv->tk", Sprev, D)
    dg = np.sum(G * Sprev, axis=2)
    for name, want in (("dq", dQ), ("dk", dK), ("dv", D), ("dw", D * Vv), ("dbeta", dbeta), ("dg", dg)):
        a = got[name][:, 0]
        err = np.max(np.abs(a - want))
        assert err <= tol * max(1.0, np.max(np.abs(want))), f"{name}: {err:.3e}"
    err = np.max(np.abs(got["d_initial_state"][0, 0] - dS0))
    assert err <= tol * max(1.0, np.max(np.abs(dS0))), f"d_initial_state: {err:.3e}"


def pin_linearity_in_cotangents(bwd, seed=7, tol=1e-11):
    """Gradients are linear in (d_out, d_final_state)."""
    x, cu, d1, f1 = rand_case(seed)
    r = np.random.default_rng(seed + 1)
    d2, f2 = r.standard_normal(d1.shape), r.standard_normal(f1.shape)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["w"], 0.8, x["initial_state"], cu)
    a, b = bwd(*args, d1, f1), bwd(*args, d2, f2)
    c = bwd(*args, 2.0 * d1 - 0.5 * d2, 2.0 * f1 - 0.5 * f2)
    for name in GRADS.values():
        want = 2.0 * a[name] - 0.5 * b[name]
        err = np.max(np.abs(c[name] - want))
        assert err <= tol * max(1.0, np.max(np.abs(want))), f"{name}: {err:.3e}"


PINS = [pin_finite_differences, pin_linear_attention, pin_linearity_in_cotangents]
