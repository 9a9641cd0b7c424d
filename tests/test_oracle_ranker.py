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


def _sigma_mutation(kind):
    real = RK.full_layer_rounding_sigma
    real_layer = RK._perturbed_full_layer

    def sigma(x, layer, offsets, cand_start, H, d, base=RK.DEFAULT_BASE, scale=None, points=RK.ROUNDING_POINTS,
              samples=128, seed=0):
        if kind == "rotary_point_dropped":
            points = tuple(p for p in points if p != "rotary")
        return real(x, layer, offsets, cand_start, H, d, base, scale, points, samples, seed)

    def layer(x, L, offsets, cand_start, H, d, base, scale, jitter):
        return real_layer(x, L, offsets, np.asarray(cand_start) + 1, H, d, base, scale, jitter)
    return {"rotary_point_dropped": ("full_layer_rounding_sigma", sigma),
            "late_candidate_start": ("_perturbed_full_layer", layer)}[kind]


@pytest.mark.parametrize("name", ["u_halved", "u_doubled", "rotary_point_dropped", "late_candidate_start"])
def test_rounding_sigma_mutations_caught(name, monkeypatch):
    """Plausible mistakes in the layer's rounding spread: the unit roundoff off by a factor
    2 either way, a rounding point left out, the layer's candidate start off by one."""
    if name == "u_halved":
        monkeypatch.setattr(RK, "U_BF16", 2.0 ** -9)
    elif name == "u_doubled":
        monkeypatch.setattr(RK, "U_BF16", 2.0 ** -7)
    else:
        attr, fn = _sigma_mutation(name)
        monkeypatch.setattr(RK, attr, fn)
    with pytest.raises(AssertionError):
        _ranker_pins.pin_layer_rounding_sigma()


def _slack_mutation(kind):
    """``f32_slack`` with one of its terms mistaken: the float32 unit roundoff a quarter of
    its value, or the update-relative, the W_o-accumulation or the residual-add term left
    out."""
    def slack(x, layer, offsets, cand_start, H, d, base=RK.DEFAULT_BASE, scale=None):
        upd, o = RK._perturbed_full_layer(x, layer, offsets, cand_start, H, d, base, scale, lambda p, a: a)
        D = H * d
        u = RK.U_F32 / 4 if kind == "u_quarter" else RK.U_F32
        terms = {"accum": (D + 2) * u * (np.abs(o.reshape(len(upd), D)) @ np.abs(np.asarray(layer.w_o)).T),
                 "resid": 4 * u * np.abs(np.asarray(x, np.float64)),
                 "upd": (2.0 ** -18 if kind != "u_quarter" else 2.0 ** -20) * np.abs(upd)}
        dropped = {"no_upd_term": "upd", "no_accum_term": "accum", "no_resid_term": "resid"}.get(kind)
        return sum(v for k, v in terms.items() if k != dropped) + 1e-300
    return slack


@pytest.mark.parametrize("name", ["u_quarter", "no_upd_term", "no_accum_term", "no_resid_term"])
def test_f32_slack_mutations_caught(name, monkeypatch):
    monkeypatch.setattr(RK, "f32_slack", _slack_mutation(name))
    with pytest.raises(AssertionError):
        _ranker_pins.pin_f32_slack()
