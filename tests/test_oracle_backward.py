"""The backward oracle against its pins, and planted mistakes that some pin catches (CPU)."""
import numpy as np
import pytest

import _bwd_pins
from oracle import backward as G


@pytest.mark.parametrize("pin", _bwd_pins.BWD_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def _user_factory(kind):
    def f(q, k, v, do, mask, sc):
        s = np.where(mask, sc * (q @ k.T), -np.inf)
        has = mask.any(axis=1)
        p = np.zeros_like(s)
        if has.any():
            m = s[has].max(axis=1, keepdims=True)
            e = np.where(mask[has], np.exp(s[has] - m), 0.0)
            p[has] = e / e.sum(axis=1, keepdims=True)
        dv = (p @ do) if kind == "dv_not_transposed" else p.T @ do
        dp = do @ v.T
        if kind == "no_rowsum":
            ds = p * dp
        else:
            ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
        dq = (ds @ k) if kind == "dq_unscaled" else sc * (ds @ k)
        dk = sc * (ds @ q) if kind == "dk_not_transposed" else sc * (ds.T @ q)
        if kind == "dv_from_values":
            dv = p.T @ v
        return dq, dk, dv
    return f


MUTATIONS = ["no_rowsum", "dv_not_transposed", "dq_unscaled", "dk_not_transposed", "dv_from_values"]


@pytest.mark.parametrize("name", MUTATIONS)
def test_some_pin_catches(name, monkeypatch):
    monkeypatch.setattr(G, "_user_head_backward", _user_factory(name))
    caught = []
    for pin in _bwd_pins.BWD_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"


def _cand_scale_factory(kind, real):
    """Plausible mistakes in the candidate-only error scale: history key and value scales
    exchanged, the candidates' own key and value scales exchanged, or the history and
    candidate row maps of the fallback layout exchanged."""
    def f(*args, **kw):
        if kind == "rows_swapped":
            orig = G._cand_only_as_full

            def swapped(*a):
                q, k, v, g, off, cs, hr, cr = orig(*a)
                return q, k, v, g, off, cs, cr, hr
            G._cand_only_as_full = swapped
            try:
                return real(*args, **kw)
            finally:
                G._cand_only_as_full = orig
        eq, ekh, evh, ekc, evc = real(*args, **kw)
        if kind == "hist_k_v_swapped":
            return eq, evh, ekh, ekc, evc
        return eq, ekh, evh, evc, ekc
    return f


CAND_SCALE_MUTATIONS = ["hist_k_v_swapped", "cand_k_v_swapped", "rows_swapped"]


@pytest.mark.parametrize("name", CAND_SCALE_MUTATIONS)
def test_some_pin_catches_cand_only_scale(name, monkeypatch):
    monkeypatch.setattr(G, "cand_only_gradient_error_scale",
                        _cand_scale_factory(name, G.cand_only_gradient_error_scale))
    caught = []
    for pin in _bwd_pins.BWD_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"
