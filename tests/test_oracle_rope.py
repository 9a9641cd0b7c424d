"""The rotary-position oracle against its pins, and planted mistakes that some pin catches (CPU)."""
import numpy as np
import pytest

import _rope_pins
from oracle import rotary as R


@pytest.mark.parametrize("pin", _rope_pins.ROPE_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


_orig_positions = R.right_anchored_positions
_orig_angles = R.rotary_angles
_orig_rope = R.rope


def _positions_not_anchored(offsets, cand_start, pos_base=None):
    offsets = np.asarray(offsets, dtype=np.int64)
    pos = np.zeros(int(offsets[-1]), dtype=np.int64)
    base = np.zeros(len(offsets) - 1, np.int64) if pos_base is None else np.asarray(pos_base)
    for b in range(len(offsets) - 1):
        pos[offsets[b]:offsets[b + 1]] = base[b] + np.arange(offsets[b + 1] - offsets[b])
    return pos


def _positions_shifted(offsets, cand_start, pos_base=None):
    return _orig_positions(offsets, cand_start, pos_base) + 1


def _positions_no_base(offsets, cand_start, pos_base=None):
    return _orig_positions(offsets, cand_start, None)


def _angles_wrong_exponent(pos, d, base=R.DEFAULT_BASE):
    base = R.DEFAULT_BASE if (base is None or base <= 0) else float(base)
    return np.asarray(pos, np.float64)[:, None] * (base ** (-np.arange(0, d, 2) / (2 * d)))[None, :]


def _rope_factory(kind):
    def f(x, pos, base=R.DEFAULT_BASE):
        x = np.asarray(x, dtype=np.float64)
        ang = R.rotary_angles(pos, x.shape[-1], base)[:, None, :]
        c, s = np.cos(ang), np.sin(ang)
        if kind == "reverse_rotation":
            s = -s
        if kind == "split_halves":
            h = x.shape[-1] // 2
            x0, x1 = x[..., :h], x[..., h:]
            out = np.empty_like(x)
            out[..., :h] = x0 * c - x1 * s
            out[..., h:] = x0 * s + x1 * c
            return out
        x0, x1 = x[..., 0::2], x[..., 1::2]
        out = np.empty_like(x)
        out[..., 0::2] = x0 * c - x1 * s
        out[..., 1::2] = x0 * s + x1 * c
        return out
    return f


def _full_rotates_values(q, k, v, offsets, cand_start, valid=None, attend_padded_history=False,
                         scale=None, base=R.DEFAULT_BASE):
    from oracle.attention import full_attention
    pos = R.right_anchored_positions(offsets, cand_start)
    return full_attention(R.rope(q, pos, base), R.rope(k, pos, base), R.rope(v, pos, base), offsets,
                          cand_start, valid, attend_padded_history, scale)


MUTATIONS = {
    "candidates_not_anchored": ("right_anchored_positions", _positions_not_anchored),
    "positions_off_by_one": ("right_anchored_positions", _positions_shifted),
    "cand_only_base_dropped": ("right_anchored_positions", _positions_no_base),
    "frequency_exponent_wrong": ("rotary_angles", _angles_wrong_exponent),
    "rotation_reversed": ("rope", _rope_factory("reverse_rotation")),
    "pairs_split_in_halves": ("rope", _rope_factory("split_halves")),
    "values_rotated": ("full_attention_rope", _full_rotates_values),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(R, attr, fn)
    caught = []
    for pin in _rope_pins.ROPE_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"
