"""CPU tests: the FP64 backward oracles against their pins, and planted mistakes.

The pins (``oracle_bwd_pins.py``) compare the numpy backward oracle with
finite differences of the pinned forward oracle and with closed forms. Each
planted mistake -- a plausible slip in the reverse sweep, planted in a copy of
the numpy backward oracle on the CPU -- must be caught by at least one pin.
The plain-C backward oracle is checked against the same pins and against the
numpy one.
"""

from __future__ import annotations

import inspect

import numpy as np
import pytest

import oracle.recurrence_bwd as rb
from tests.oracle_bwd_pins import PINS, rand_case


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_numpy_bwd_oracle_pin(pin):
    pin(rb.gdn2_recurrence_bwd)


MUTATIONS = {
    "dropped_beta_term_of_dk": ("dk[t] += dbk * beta[t]", "pass"),
    "adjoint_without_decay": ("dS = dSd * a[:, :, None]", "dS = dSd"),
    "dropped_erase_adjoint": ("dSd = dS + bk[:, :, None] * de[:, None, :]", "dSd = dS"),
    "erase_sign": ("        de = -dvnew\n", "        de = dvnew\n"),
    "dg_from_undecayed_gradient": ("dg[t] = np.sum(dSd * Sd, axis=2)", "dg[t] = np.sum(dS * Sd, axis=2)"),
    "dq_from_decayed_state": ('dq[t] = scale * np.einsum("hkv,hv->hk", St, do[t])',
                              'dq[t] = scale * np.einsum("hkv,hv->hk", Sd, do[t])'),
    "output_gradient_after_erase": ("dS = dS + scale * q[t][:, :, None] * do[t][:, None, :]\n",
                                    "dS = dS\n"),
    "gva_first_head_only": ("dq[:, h * m:(h + 1) * m].sum(axis=1)", "dq[:, h * m]"),
}


def _mutant(kind):
    old, new = MUTATIONS[kind]
    src = inspect.getsource(rb)
    assert src.count(old) == 1, kind
    src = src.replace(old, new).replace("from .recurrence import", "from oracle.recurrence import")
    ns = {"__name__": "mutant_" + kind}
    exec(compile(src, "mutant_" + kind, "exec"), ns)
    return ns["gdn2_recurrence_bwd"]


def _caught(fn):
    for pin in PINS:
        try:
            pin(fn)
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("kind", sorted(MUTATIONS))
def test_planted_bwd_mistake_is_caught(kind):
    assert _caught(_mutant(kind)), f"planted mistake {kind} passed every pin"


def test_unmutated_copy_passes():
    src = inspect.getsource(rb).replace("from .recurrence import", "from oracle.recurrence import")
    ns = {"__name__": "copy"}
    exec(compile(src, "copy", "exec"), ns)
    assert not _caught(ns["gdn2_recurrence_bwd"])


@pytest.fixture(scope="module")
def c_oracle():
    from oracle import c_oracle as co
    co.load()
    return co


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_c_bwd_oracle_pin(pin, c_oracle):
    pin(c_oracle.gdn2_recurrence_bwd_c)


@pytest.mark.parametrize("block", [1, 3, 64])
def test_numpy_and_c_bwd_oracles_agree(c_oracle, block):
    """Varlen, grouped heads, lengths straddling the C oracle's recompute
    blocks (the block length only changes where states are recomputed)."""
    x, cu, d_out, d_final = rand_case(11, lengths=(7, 1, 0, 12), H=2, HV=6, K=4, V=3)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["w"], 0.5, x["initial_state"], cu, d_out, d_final)
    a = rb.gdn2_recurrence_bwd(*args)
    b = c_oracle.gdn2_recurrence_bwd_c(*args, block=block)
    for name in a:
        np.testing.assert_allclose(b[name], a[name], rtol=1e-12, atol=1e-12, err_msg=name)
