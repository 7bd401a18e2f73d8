"""Pins of the FP64 oracle against facts the pages and the mathematics fix.

Each ``pin_*`` takes an oracle callable with the signature of
``oracle.recurrence.gdn2_recurrence`` and raises AssertionError when the
callable disagrees with the fact. The facts are independent of the oracle's
own code: a hand-worked example, a second algebraic form from another page,
closed forms of special cases, an independently derived chunk solve, and
invariants.
"""

from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-11


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_case(seed, T=23, H=2, HV=2, K=5, V=4, g_max=0.3, beta_max=1.0, with_state=True, N=1):
    r = _rng(seed)
    q = _unit(r.standard_normal((T, H, K)))
    k = _unit(r.standard_normal((T, H, K)))
    v = r.standard_normal((T, HV, V))
    g = -g_max * r.random((T, HV, K))
    beta = beta_max * r.random((T, HV, K))
    w = r.random((T, HV, V))
    S0 = 0.3 * r.standard_normal((N, HV, K, V)) if with_state else None
    return q, k, v, g, beta, w, S0


def _close(a, b, tol=TOL, what=""):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(1.0, np.max(np.abs(b)) if b.size else 1.0)
    assert err <= tol * scale, f"{what}: max abs diff {err:.3e}"


# --------------------------------------------------------------------------- #
# 1. Hand-worked example (tests/golden/hand_worked_t2_k2v2.txt)
# --------------------------------------------------------------------------- #
def load_hand_worked():
    vals = {}
    with open(os.path.join(GOLDEN, "hand_worked_t2_k2v2.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, *nums = line.split()
            vals[name] = np.array([float(x) for x in nums])
    return vals


def pin_hand_worked(fn):
    d = load_hand_worked()
    sh = lambda x: x.reshape(2, 1, 2)
    for s in (1.0, 0.5):
        o, S = fn(sh(d["q"]), sh(d["k"]), sh(d["v"]), sh(d["g"]), sh(d["beta"]), sh(d["w"]), s)
        _close(o.reshape(-1), s * d["out"], 1e-14, "hand-worked output")
        _close(S.reshape(-1), d["final"], 1e-14, "hand-worked state")


# --------------------------------------------------------------------------- #
# 2. The matrix form printed in the burn-gdn2 README ("Architecture"):
#    S_t = (I - k_t (b_t*k_t)^T) diag(alpha_t) S_{t-1} + k_t (w_t*v_t)^T,
#    o_t = q_t^T S_t  (no scale there, so compare at scale 1)
# --------------------------------------------------------------------------- #
def pin_matrix_form(fn):
    q, k, v, g, beta, w, S0 = _rand_case(11, T=17, H=1, HV=1, K=4, V=3)
    T, K, V = q.shape[0], q.shape[2], v.shape[2]
    S = S0[0, 0].copy()
    o_ref = np.zeros((T, 1, V))
    for t in range(T):
        kt, bt, at = k[t, 0], beta[t, 0], np.exp(g[t, 0])
        M = np.eye(K) - np.outer(kt, bt * kt)
        S = M @ np.diag(at) @ S + np.outer(kt, w[t, 0] * v[t, 0])
        o_ref[t, 0] = q[t, 0] @ S
    o, Sf = fn(q, k, v, g, beta, w, 1.0, S0)
    _close(o, o_ref, TOL, "matrix-form output")
    _close(Sf[0, 0], S, TOL, "matrix-form state")


# --------------------------------------------------------------------------- #
# 3. Retrieval identities (closed form): with the decayed state read through
#    beta*k and the output reading the written state, a query equal to the
#    erase direction returns exactly scale*w*v, for any g and any S0.
# --------------------------------------------------------------------------- #
def pin_retrieval(fn):
    q, k, v, g, beta, w, S0 = _rand_case(12, T=19, H=1, HV=1, K=6, V=5, g_max=2.0)
    # scalar version: beta = 1, unit k, q = k
    ones = np.ones_like(beta)
    o, _ = fn(k, k, v, g, ones, w, 0.7, S0)
    _close(o, 0.7 * w * v, TOL, "retrieval (beta=1, q=k)")
    # channel-wise version: q = beta*k with sum_c beta_c k_c^2 = 1
    b = beta + 0.1
    kk = k / np.sqrt(np.sum(b * k * k, axis=-1, keepdims=True))
    o, _ = fn(b * kk, kk, v, g, b, w, 1.3, S0)
    _close(o, 1.3 * w * v, TOL, "retrieval (channel-wise)")


# --------------------------------------------------------------------------- #
# 4. g = 0, beta = 0, w = 1: ungated linear attention in closed form
#    o = scale*(tril(Q K^T) V + Q S0),   S_T = S0 + K^T V
# --------------------------------------------------------------------------- #
def pin_linear_attention(fn):
    q, k, v, g, beta, w, S0 = _rand_case(13, T=21, H=1, HV=1, K=5, V=4)
    Q, Kk, Vv = q[:, 0], k[:, 0], v[:, 0]
    o_ref = 0.4 * (np.tril(Q @ Kk.T) @ Vv + Q @ S0[0, 0])
    S_ref = S0[0, 0] + Kk.T @ Vv
    o, S = fn(q, k, v, np.zeros_like(g), np.zeros_like(beta), np.ones_like(w), 0.4, S0)
    _close(o[:, 0], o_ref, TOL, "linear attention output")
    _close(S[0, 0], S_ref, TOL, "linear attention state")


# --------------------------------------------------------------------------- #
# 5. beta = 0: channel-wise gated linear attention, brute force O(T^2 K)
#    o_t = scale*[sum_{s<=t} ((q_t*exp(G_t-G_s)).k_s)(w_s*v_s) + (q_t*exp(G_t))^T S0]
#    S_T = diag(exp(G_T)) S0 + sum_s (k_s*exp(G_T-G_s)) (w_s*v_s)^T
# --------------------------------------------------------------------------- #
def pin_gated_linear_attention(fn):
    q, k, v, g, beta, w, S0 = _rand_case(14, T=15, H=1, HV=1, K=4, V=3, g_max=3.0)
    T = q.shape[0]
    G = np.cumsum(g[:, 0], axis=0)
    WV = w[:, 0] * v[:, 0]
    o_ref = np.zeros((T, v.shape[2]))
    for t in range(T):
        acc = (q[t, 0] * np.exp(G[t])) @ S0[0, 0]
        for s in range(t + 1):
            acc = acc + np.dot(q[t, 0] * np.exp(G[t] - G[s]), k[s, 0]) * WV[s]
        o_ref[t] = 0.9 * acc
    S_ref = np.diag(np.exp(G[-1])) @ S0[0, 0]
    for s in range(T):
        S_ref = S_ref + np.outer(k[s, 0] * np.exp(G[-1] - G[s]), WV[s])
    o, S = fn(q, k, v, g, np.zeros_like(beta), w, 0.9, S0)
    _close(o[:, 0], o_ref, TOL, "GLA output")
    _close(S[0, 0], S_ref, TOL, "GLA state")


# --------------------------------------------------------------------------- #
# 6. Channel-constant g = a_t and w = beta = b_t (FlashInfer docs: recovers
#    GDN) -> the scalar gated delta rule, written in its textbook form
#    S_t = exp(a_t) (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T
# --------------------------------------------------------------------------- #
def pin_scalar_gdn(fn):
    r = _rng(15)
    T, K, V = 18, 5, 4
    q = _unit(r.standard_normal((T, 1, K)))
    k = _unit(r.standard_normal((T, 1, K)))
    v = r.standard_normal((T, 1, V))
    a = -0.5 * r.random(T)
    b = r.random(T)
    S0 = 0.2 * r.standard_normal((1, 1, K, V))
    S = S0[0, 0].copy()
    o_ref = np.zeros((T, V))
    for t in range(T):
        kt = k[t, 0]
        S = np.exp(a[t]) * (np.eye(K) - b[t] * np.outer(kt, kt)) @ S + b[t] * np.outer(kt, v[t, 0])
        o_ref[t] = 0.6 * q[t, 0] @ S
    g = np.repeat(a[:, None, None], K, axis=2)
    beta = np.repeat(b[:, None, None], K, axis=2)
    w = np.repeat(b[:, None, None], V, axis=2)
    o, Sf = fn(q, k, v, g, beta, w, 0.6, S0)
    _close(o[:, 0], o_ref, TOL, "scalar GDN output")
    _close(Sf[0, 0], S, TOL, "scalar GDN state")


# --------------------------------------------------------------------------- #
# 7. Whole-sequence WY solve (independent chunk algebra, one chunk of T <= 64):
#    A_rs = sum_c beta_r k_r exp(G_r - G_s) k_s (s < r),  U = (I + A)^{-1}
#    (W*V - (beta*k*exp(G)) S0),  O = scale[(q*exp(G)) S0 + P U] with
#    P_rs = sum_c q_r exp(G_r - G_s) k_s (s <= r),
#    S_T = diag(exp(G_T)) S0 + sum_s (k_s*exp(G_T - G_s)) u_s^T
# --------------------------------------------------------------------------- #
def pin_wy_solve(fn):
    q, k, v, g, beta, w, S0 = _rand_case(16, T=40, H=1, HV=1, K=6, V=5, g_max=0.5, beta_max=2.0)
    Q, Kk, Vv, B, W = q[:, 0], k[:, 0], v[:, 0], beta[:, 0], w[:, 0]
    T = Q.shape[0]
    G = np.cumsum(g[:, 0], axis=0)
    E = np.exp(G[:, None, :] - G[None, :, :])          # [r, s, c], used for s <= r only
    A = np.einsum("rc,rsc,sc->rs", B * Kk, E, Kk) * np.tril(np.ones((T, T)), -1)
    P = np.einsum("rc,rsc,sc->rs", Q, E, Kk) * np.tril(np.ones((T, T)), 0)
    R = W * Vv - (B * Kk * np.exp(G)) @ S0[0, 0]
    U = np.linalg.solve(np.eye(T) + A, R)
    o_ref = 0.8 * ((Q * np.exp(G)) @ S0[0, 0] + P @ U)
    S_ref = np.diag(np.exp(G[-1])) @ S0[0, 0] + (Kk * np.exp(G[-1] - G)).T @ U
    o, S = fn(q, k, v, g, beta, w, 0.8, S0)
    _close(o[:, 0], o_ref, 1e-9, "WY output")
    _close(S[0, 0], S_ref, 1e-9, "WY state")


# --------------------------------------------------------------------------- #
# 8. Split and carry: [0, t1) then [t1, T) from the carried state == one pass
# --------------------------------------------------------------------------- #
def pin_split_carry(fn):
    q, k, v, g, beta, w, S0 = _rand_case(17, T=30)
    o, S = fn(q, k, v, g, beta, w, 0.5, S0)
    t1 = 13
    o1, S1 = fn(q[:t1], k[:t1], v[:t1], g[:t1], beta[:t1], w[:t1], 0.5, S0)
    o2, S2 = fn(q[t1:], k[t1:], v[t1:], g[t1:], beta[t1:], w[t1:], 0.5, S1)
    _close(np.concatenate([o1, o2]), o, 1e-13, "split/carry output")
    _close(S2, S, 1e-13, "split/carry state")


# --------------------------------------------------------------------------- #
# 9. Invariants
# --------------------------------------------------------------------------- #
def pin_linearity(fn):
    """Jointly linear in (v, S0): scaling and superposition."""
    q, k, v, g, beta, w, S0 = _rand_case(18)
    _, _, v2, _, _, _, S02 = _rand_case(19)
    o1, s1 = fn(q, k, v, g, beta, w, 0.5, S0)
    o2, s2 = fn(q, k, v2, g, beta, w, 0.5, S02)
    o3, s3 = fn(q, k, 2.0 * v - 3.0 * v2, g, beta, w, 0.5, 2.0 * S0 - 3.0 * S02)
    _close(o3, 2.0 * o1 - 3.0 * o2, 1e-12, "linearity output")
    _close(s3, 2.0 * s1 - 3.0 * s2, 1e-12, "linearity state")


def pin_key_permutation(fn):
    """Permuting key channels of q, k, g, beta and rows of S0 leaves o unchanged
    and permutes the rows of the final state."""
    q, k, v, g, beta, w, S0 = _rand_case(20, K=6)
    p = _rng(21).permutation(6)
    o, S = fn(q, k, v, g, beta, w, 0.5, S0)
    op, Sp = fn(q[..., p], k[..., p], v, g[..., p], beta[..., p], w, 0.5, S0[:, :, p, :])
    _close(op, o, 1e-12, "key permutation output")
    _close(Sp, S[:, :, p, :], 1e-12, "key permutation state")


def pin_value_permutation(fn):
    """Permuting value channels of v, w and columns of S0 permutes o and the
    columns of the state."""
    q, k, v, g, beta, w, S0 = _rand_case(22, V=5)
    p = _rng(23).permutation(5)
    o, S = fn(q, k, v, g, beta, w, 0.5, S0)
    op, Sp = fn(q, k, v[..., p], g, beta, w[..., p], 0.5, S0[..., p])
    _close(op, o[..., p], 1e-12, "value permutation output")
    _close(Sp, S[..., p], 1e-12, "value permutation state")


def pin_heads_and_gva(fn):
    """Heads are independent; grouped value heads equal the plain H = HV case
    with q/k repeated in contiguous groups (value head hv reads head hv // m)."""
    q, k, v, g, beta, w, S0 = _rand_case(24, H=2, HV=6)
    o, S = fn(q, k, v, g, beta, w, 0.5, S0)
    qr, kr = np.repeat(q, 3, axis=1), np.repeat(k, 3, axis=1)
    o2, S2 = fn(qr, kr, v, g, beta, w, 0.5, S0)
    _close(o2, o, 1e-13, "GVA == repeated q/k (output)")
    _close(S2, S, 1e-13, "GVA == repeated q/k (state)")
    for hv in range(6):
        oh, Sh = fn(q[:, hv // 3:hv // 3 + 1], k[:, hv // 3:hv // 3 + 1], v[:, hv:hv + 1],
                    g[:, hv:hv + 1], beta[:, hv:hv + 1], w[:, hv:hv + 1], 0.5, S0[:, hv:hv + 1])
        _close(oh[:, 0], o[:, hv], 1e-13, f"head {hv} alone (output)")
        _close(Sh[:, 0], S[:, hv], 1e-13, f"head {hv} alone (state)")


def pin_single_token(fn):
    """T = 1 closed form: Sd = diag(e^g) S0, vnew = w v - (beta k)^T Sd,
    S1 = Sd + k vnew^T, o = scale q^T S1."""
    q, k, v, g, beta, w, S0 = _rand_case(25, T=1, H=1, HV=1)
    Sd = np.exp(g[0, 0])[:, None] * S0[0, 0]
    vn = w[0, 0] * v[0, 0] - (beta[0, 0] * k[0, 0]) @ Sd
    S1 = Sd + np.outer(k[0, 0], vn)
    o, S = fn(q, k, v, g, beta, w, 0.25, S0)
    _close(o[0, 0], 0.25 * q[0, 0] @ S1, TOL, "single token output")
    _close(S[0, 0], S1, TOL, "single token state")


def pin_defaults(fn):
    """g None -> 0, beta None -> 1, w None -> 1, initial state None -> 0,
    scale None or 0 -> 1/sqrt(K) (FlashInfer docs, parameter list)."""
    q, k, v, g, beta, w, S0 = _rand_case(26, K=9)
    K = q.shape[2]
    base = fn(q, k, v, np.zeros_like(g), np.ones_like(beta), np.ones_like(w), 1 / math.sqrt(K), np.zeros_like(S0))
    for got in (fn(q, k, v, None, None, None, None, None), fn(q, k, v, None, None, None, 0.0, None)):
        _close(got[0], base[0], 1e-14, "defaults output")
        _close(got[1], base[1], 1e-14, "defaults state")


def pin_default_scale_key_dim(fn):
    """The default scale is 1/sqrt(K), K the q/k head dimension, also when
    the value dimension differs (FlashInfer docs, ``scale``: one over the
    square root of the head size of the q.k product). Pinned through the
    retrieval identity, not the formula: with beta = 1, unit k and q = k
    the delta rule returns exactly scale * w * v, so the output's magnitude
    shows the scale used: 1/4 at (K, V) = (16, 4), 1/2 at (4, 16)."""
    for K, V, want in ((16, 4, 0.25), (4, 16, 0.5)):
        q, k, v, g, beta, w, S0 = _rand_case(28, T=11, H=1, HV=1, K=K, V=V, g_max=1.0)
        ones = np.ones_like(beta)
        for sc in (None, 0.0):
            o, S = fn(k, k, v, g, ones, w, sc, S0)
            assert S.shape == (1, 1, K, V), f"state shape {S.shape} at (K, V) = ({K}, {V})"
            _close(o, want * w * v, TOL, f"default scale at (K, V) = ({K}, {V})")


def pin_varlen(fn):
    """Packed sequences == separate calls, each from its own initial state; an
    empty sequence returns its initial state."""
    lens = [9, 0, 14, 1]
    T = sum(lens)
    q, k, v, g, beta, w, S0 = _rand_case(27, T=T, N=len(lens))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, S = fn(q, k, v, g, beta, w, 0.5, S0, cu)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        on, Sn = fn(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], w[a:b], 0.5, S0[n:n + 1])
        _close(o[a:b], on, 1e-14, f"varlen seq {n} output")
        _close(S[n], Sn[0], 1e-14, f"varlen seq {n} state")
    _close(S[1], S0[1], 0.0, "empty sequence keeps its state")


# --------------------------------------------------------------------------- #
# In-kernel q/k L2 normalisation (FlashInfer docs, use_qk_l2norm_in_kernel).
# Facts that hold for any correct normalisation of each (token, head) row
# over the head dimension, whatever the raw norms:
#  * retrieval: q_t = c_t k_t, beta = 1 returns sign(c_t) scale w v exactly;
#  * invariance: positive per-row rescaling of q or k changes nothing;
#  * unit rows: the option is the identity;
#  * a zero row of q gives a zero output row (no division by zero).
# --------------------------------------------------------------------------- #
def pin_qk_l2norm(fn):
    r = _rng(31)
    T, H, K, V = 16, 2, 6, 5
    q, k, v, g, beta, w, S0 = _rand_case(31, T=T, H=H, HV=2 * H, K=K, V=V, g_max=1.0)
    raw_k = k * r.uniform(0.3, 4.0, size=(T, H, 1))
    c = r.uniform(0.2, 3.0, size=(T, H, 1)) * np.where(r.random((T, H, 1)) < 0.3, -1.0, 1.0)
    ones = np.ones_like(beta)
    o, _ = fn(c * raw_k, raw_k, v, g, ones, w, 0.7, S0, qk_l2norm=True)
    sgn = np.repeat(np.sign(c), 2, axis=1)  # value heads 2h, 2h + 1 read q/k head h
    _close(o, 0.7 * sgn * w * v, TOL, "l2norm retrieval")
    o1, s1 = fn(q, k, v, g, beta, w, 0.9, S0, qk_l2norm=True)
    a = r.uniform(0.1, 5.0, size=(T, H, 1))
    b = r.uniform(0.1, 5.0, size=(T, H, 1))
    o2, s2 = fn(a * q, b * k, v, g, beta, w, 0.9, S0, qk_l2norm=True)
    _close(o2, o1, TOL, "l2norm invariance (output)")
    _close(s2, s1, TOL, "l2norm invariance (state)")
    o3, s3 = fn(q, k, v, g, beta, w, 0.9, S0)
    _close(o1, o3, TOL, "l2norm on unit rows (output)")
    _close(s1, s3, TOL, "l2norm on unit rows (state)")
    qz = q.copy()
    qz[5] = 0.0
    o4, _ = fn(qz, k, v, g, beta, w, 0.9, S0, qk_l2norm=True)
    assert np.all(np.isfinite(o4)) and np.all(o4[5] == 0.0), "l2norm zero row"


ALL_PINS = [pin_hand_worked, pin_matrix_form, pin_retrieval, pin_default_scale_key_dim, pin_linear_attention,
            pin_gated_linear_attention, pin_scalar_gdn, pin_wy_solve, pin_split_carry,
            pin_linearity, pin_key_permutation, pin_value_permutation, pin_heads_and_gva,
            pin_single_token, pin_defaults, pin_varlen, pin_qk_l2norm]
