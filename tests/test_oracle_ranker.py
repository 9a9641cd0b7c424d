"""The layer-stack oracle against its pins, and planted mistakes that some pin catches (CPU)."""
import numpy as np
import pytest

import _ranker_pins
from oracle import ranker as RK


@pytest.mark.parametrize("pin", _ranker_pins.RANKER_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def _mut_no_gain(x, gain, eps=RK.RMS_EPS):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _mut_no_residual(x, o, layer):
    return o.reshape(o.shape[0], -1) @ np.asarray(layer.w_o, np.float64).T


def _mut_wo_untransposed(x, o, layer):
    return np.asarray(x, np.float64) + o.reshape(o.shape[0], -1) @ np.asarray(layer.w_o, np.float64)


def _mut_qkv_order(x, layer, H, d):
    q, k, v = _ORIG_QKV(x, layer, H, d)
    return k, q, v


def _mut_causal_positions(offsets, cand_start, pos_base=None):
    offsets = np.asarray(offsets, np.int64)
    pos = np.zeros(int(offsets[-1]), np.int64)
    for b in range(len(offsets) - 1):
        pos[offsets[b]:offsets[b + 1]] = np.arange(offsets[b + 1] - offsets[b]) + (
            0 if pos_base is None else int(pos_base[b]))
    return pos


_ORIG_QKV = RK._qkv
MUTATIONS = {"no_gain": ("rms_norm", _mut_no_gain), "no_residual": ("_out", _mut_no_residual),
             "wo_untransposed": ("_out", _mut_wo_untransposed), "qkv_order": ("_qkv", _mut_qkv_order),
             "causal_positions": ("right_anchored_positions", _mut_causal_positions)}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(RK, attr, fn)
    caught = []
    for pin in _ranker_pins.RANKER_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"
