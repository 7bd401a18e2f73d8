"""Plain token-by-token FP64 oracle for the GDN-2 forward pass (numpy).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``). Parity of every function
here is pinned by ``tests/test_oracle_pins.py``.

Definition followed -- FlashInfer ``chunk_gated_delta_rule2`` docs, recurrence
display equation. Per value head, with key dimension K and value dimension V
and a K x V state S:

    S_t      = diag(exp(g_t)) S_{t-1}                    (forget gate, key axis)
    vnew_t   = w_t * v_t - (beta_t * k_t)^T S_t          (erase reads the decayed S)
    S_t     += k_t vnew_t^T                              (rank-one write)
    o_t      = scale * q_t^T S_t                         (reads the updated S)

Readings taken where the pages leave a step open:

* ``scale`` None or 0 means 1/sqrt(K) (same docs, ``scale`` parameter; K is
  the q.k contraction length).
* g None -> 0, beta None -> 1, w None -> 1, initial state None -> zeros (same
  docs, parameter list).
* Grouped value heads: value head ``hv`` reads q/k head ``hv // (HV // H)``
  (contiguous groups). The Flash-GDN-2 README ("Quick start") and the FlashRT
  card ("Usage", H32 producer profile) allow HV a multiple of H but do not state
  the mapping; contiguous groups is the plain reading.
* State layout [N, HV, K, V] (K-major), as in the Flash-GDN-2 README quick start.
* Varlen packing: tokens of all sequences end to end, sequence n spans
  ``cu_seqlens[n] .. cu_seqlens[n+1]`` (FlashInfer docs, description and
  ``cu_seqlens`` parameter). Each sequence starts from its own initial state.
* ``qk_l2norm`` (FlashInfer docs, ``use_qk_l2norm_in_kernel``: the q/k L2
  normalisation moved into the kernel instead of pre-normalised inputs): the
  pages do not spell the normalisation out; the one they use to make the
  pre-normalised inputs is the Flash-GDN-2 README quick start's torch
  ``normalize`` over the head dimension, x / max(||x||_2, 1e-12), applied
  here to every (token, head) row of q and of k before the recurrence.
"""

from __future__ import annotations

import math

import numpy as np


def resolve_scale(scale, K: int) -> float:
    """Query scale: 1/sqrt(K) when None or 0 (FlashInfer docs, ``scale``)."""
    if scale is None or scale == 0.0:
        return 1.0 / math.sqrt(K)
    return float(scale)


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor (e.g. bf16, which numpy lacks)
        import torch
        return x.detach().cpu().to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def l2_normalize_rows(x, eps: float = 1e-12):
    """Each row along the last (head) axis divided by max(its L2 norm, eps),
    in float64: the reading of the in-kernel q/k normalisation (module
    docstring)."""
    x = _f64(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def gdn2_sequence(q, k, v, g, beta, w, scale, S0):
    """Run the recurrence over ONE sequence, all value heads at once.

    Shapes (float64 arrays, already gathered per value head):
      q, k, g, beta : [L, HV, K]     v, w : [L, HV, V]     S0 : [HV, K, V]
    Returns (o [L, HV, V], S_L [HV, K, V]).

    Follows the FlashInfer ``chunk_gated_delta_rule2`` recurrence equation
    line for line, one token at a time.
    """
    S = S0.copy()
    L = q.shape[0]
    o = np.zeros((L, S.shape[0], S.shape[2]), dtype=np.float64)
    for t in range(L):
        # forget gate: scale row c of each head's state by exp(g_t[c])
        S *= np.exp(g[t])[:, :, None]
        # erase: read the decayed state through beta_t * k_t (key axis)
        erase = np.einsum("hk,hkv->hv", beta[t] * k[t], S)
        # write gate acts on the value axis
        vnew = w[t] * v[t] - erase
        S += k[t][:, :, None] * vnew[:, None, :]
        # output reads the state that already holds token t's write
        o[t] = scale * np.einsum("hk,hkv->hv", q[t], S)
    return o, S


def gdn2_recurrence(q, k, v, g=None, beta=None, w=None, scale=None,
                    initial_state=None, cu_seqlens=None, heads=None, qk_l2norm=False):
    """FP64 oracle of the GDN-2 forward over packed (varlen) sequences.

    Arguments follow the boundary's layout (any float dtype; upcast to float64
    exactly):
      q, k   [T, H, K]      v, w [T, HV, V]      g, beta [T, HV, K]
      initial_state [N, HV, K, V] or None, cu_seqlens [N+1] ints or None (one
      sequence of T tokens).
    ``heads``: optional list of value-head indices to evaluate (each head is an
    independent recurrence); outputs then carry only those heads, in order.
    ``qk_l2norm``: normalise every (token, head) row of q and k first.

    Returns (out [T, nH, V] float64, final_state [N, nH, K, V] float64).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if qk_l2norm:
        q, k = l2_normalize_rows(q), l2_normalize_rows(k)
    T, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    if HV % H != 0:
        raise ValueError("HV must be a multiple of H")
    m = HV // H
    g = np.zeros((T, HV, K)) if g is None else _f64(g)
    beta = np.ones((T, HV, K)) if beta is None else _f64(beta)
    w = np.ones((T, HV, V)) if w is None else _f64(w)
    scale = resolve_scale(scale, K)
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    hv_idx = np.arange(HV) if heads is None else np.asarray(heads, dtype=np.int64)
    hk_idx = hv_idx // m
    nh = len(hv_idx)
    if initial_state is None:
        S0_all = np.zeros((N, nh, K, V))
    else:
        S0_all = _f64(initial_state)[:, hv_idx]
    out = np.zeros((T, nh, V))
    final = np.zeros((N, nh, K, V))
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        o, S = gdn2_sequence(q[a:b][:, hk_idx], k[a:b][:, hk_idx],
                             v[a:b][:, hv_idx], g[a:b][:, hv_idx],
                             beta[a:b][:, hv_idx], w[a:b][:, hv_idx],
                             scale, S0_all[n])
        out[a:b] = o
        final[n] = S
    return out, final
