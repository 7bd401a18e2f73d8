"""CPU tests: the FP64 oracles against their pins, and planted mistakes.

Both oracle implementations (numpy and plain C) must satisfy every pin in
``oracle_pins.py``. Each planted mistake -- a plausible slip in writing the
recurrence, planted in a copy of the numpy oracle on the CPU -- must be caught
by at least one pin.
"""

import numpy as np
import pytest

import oracle.recurrence as rec
from oracle.recurrence import gdn2_recurrence
from tests import oracle_pins as pins


@pytest.fixture(scope="session")
def c_oracle():
    import os
    from oracle.build import LIB, build_c_oracle
    if not os.path.exists(LIB):
        build_c_oracle()
    from oracle.c_oracle import gdn2_recurrence_c
    return gdn2_recurrence_c


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_numpy_oracle_pin(pin):
    pin(gdn2_recurrence)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_c_oracle_pin(pin, c_oracle):
    pin(c_oracle)


def test_c_oracle_reads_bf16_exactly(c_oracle):
    """bf16 inputs passed as raw bit patterns give the same result as their
    exact float64 upcast."""
    import torch
    from linear_attention_rnn_gdn2_amd.workloads import synth
    d = synth([37, 64, 5], 2, 4, 16, 8, seed=3, init_std=0.02)
    args = [d[n] for n in ("q", "k", "v", "g", "beta", "w")]
    o1, s1 = c_oracle(*args, 0.3, d["initial_state"], d["cu_seqlens"])
    o2, s2 = c_oracle(*[a.to(torch.float64) for a in args], 0.3,
                      d["initial_state"].to(torch.float64), d["cu_seqlens"])
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_numpy_and_c_oracles_agree(c_oracle):
    import torch
    from linear_attention_rnn_gdn2_amd.workloads import synth
    d = synth([100, 3, 64], 2, 6, 16, 12, seed=4, init_std=0.02, g_max=1.0,
              g_extreme_max=8.0, extreme_frac=0.2, beta_max=2.0)
    args = [d[n] for n in ("q", "k", "v", "g", "beta", "w")]
    o1, s1 = c_oracle(*args, None, d["initial_state"], d["cu_seqlens"])
    o2, s2 = gdn2_recurrence(*[a.to(torch.float64).numpy() for a in args], None,
                             d["initial_state"].numpy(), d["cu_seqlens"].numpy())
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(s1 - s2)) < 1e-12
    # a head subset equals the same heads of the full evaluation
    o3, s3 = c_oracle(*args, None, d["initial_state"], d["cu_seqlens"], heads=[5, 1])
    assert np.array_equal(o3, o1[:, [5, 1]]) and np.array_equal(s3, s1[:, [5, 1]])


# --------------------------------------------------------------------------- #
# Planted mistakes (mutants of the per-sequence step), CPU only
# --------------------------------------------------------------------------- #
def _mutant_sequence(kind):
    def seq(q, k, v, g, beta, w, scale, S0):
        S = S0.copy()
        L = q.shape[0]
        o = np.zeros((L, S.shape[0], S.shape[2]))
        for t in range(L):
            if kind != "erase_before_decay":
                S *= np.exp(g[t] if kind != "decay_sign" else -g[t])[:, :, None]
            bk = k[t] if kind == "drop_beta" else beta[t] * k[t]
            erase = np.einsum("hk,hkv->hv", bk, S)
            if kind == "erase_before_decay":
                S *= np.exp(g[t])[:, :, None]
            wv = v[t] if kind == "drop_w" else w[t] * v[t]
            vnew = wv + erase if kind == "erase_sign" else wv - erase
            S_prev = S.copy()
            if kind == "transposed_write":
                S += np.einsum("hv,hk->hvk", vnew, k[t])
            else:
                S += k[t][:, :, None] * vnew[:, None, :]
            src = S_prev if kind == "exclusive_output" else S
            qq = k[t] if kind == "k_for_q" else q[t]
            o[t] = (1.0 if kind == "drop_scale" else scale) * np.einsum("hk,hkv->hv", qq, src)
        return o, S
    return seq


MUTANTS = ["erase_before_decay", "decay_sign", "drop_beta", "drop_w", "erase_sign",
           "transposed_write", "exclusive_output", "k_for_q", "drop_scale"]


def _pins_fail(fn):
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(fn)
        except (AssertionError, ValueError) as e:  # shape errors count as caught
            failed.append((pin.__name__, str(e)[:60]))
    return failed


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind, monkeypatch):
    monkeypatch.setattr(rec, "gdn2_sequence", _mutant_sequence(kind))
    assert _pins_fail(rec.gdn2_recurrence), f"mutant {kind} passed every pin"


def test_unmutated_copy_passes(monkeypatch):
    """The mutant harness itself, with no mutation, passes every pin."""
    monkeypatch.setattr(rec, "gdn2_sequence", _mutant_sequence("none"))
    assert _pins_fail(rec.gdn2_recurrence) == []


def test_wrong_gva_mapping_is_caught():
    """Value head hv must read q/k head hv // m; the interleaved reading
    hv % H is caught by the GVA pin."""
    def wrong(q, k, v, g=None, beta=None, w=None, scale=None, initial_state=None,
              cu_seqlens=None, heads=None):
        H, HV = q.shape[1], v.shape[1]
        idx = np.arange(HV) % H
        return gdn2_recurrence(q[:, idx], k[:, idx], v, g, beta, w, scale,
                               initial_state, cu_seqlens, heads)
    with pytest.raises(AssertionError):
        pins.pin_heads_and_gva(wrong)


def test_default_scale_from_value_dim_is_caught(monkeypatch):
    """A default scale taken from the value dimension (1/sqrt(V)) fails the
    default-scale pin."""
    real = rec.resolve_scale

    def wrong(q, k, v, g=None, beta=None, w=None, scale=None, initial_state=None,
              cu_seqlens=None, heads=None):
        sc = real(scale, v.shape[2])
        return gdn2_recurrence(q, k, v, g, beta, w, sc, initial_state, cu_seqlens, heads)
    with pytest.raises(AssertionError):
        pins.pin_default_scale_key_dim(wrong)


def _wrong_norm(kind):
    def norm(x, eps=1e-12):
        x = rec._f64(x)
        if kind == "none":
            return x
        if kind == "head_axis":  # over the heads instead of the head dimension
            return x / np.maximum(np.sqrt(np.sum(x * x, axis=-2, keepdims=True)), eps)
        if kind == "squared":  # divided by the squared norm
            return x / np.maximum(np.sum(x * x, axis=-1, keepdims=True), eps)
        if kind == "abs":  # sign dropped
            return np.abs(x) / np.maximum(np.sqrt(np.sum(x * x, axis=-1, keepdims=True)), eps)
        raise ValueError(kind)
    return norm


@pytest.mark.parametrize("kind", ["none", "head_axis", "squared", "abs"])
def test_planted_l2norm_mistake_is_caught(kind, monkeypatch):
    """A wrong in-kernel normalisation in the oracle fails the l2norm pin."""
    monkeypatch.setattr(rec, "l2_normalize_rows", _wrong_norm(kind))
    with pytest.raises(AssertionError):
        pins.pin_qk_l2norm(rec.gdn2_recurrence)
