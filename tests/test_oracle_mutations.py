"""Plant plausible mistakes in the oracle (on the CPU) and check that some pin fails.

This shows the pins are strong enough: a dropped term, a wrong sign or index, a
transposed operand or a mis-read flag anywhere in the oracle is caught."""
import math

import numpy as np
import pytest

import _pins
from oracle import attention as A
from oracle import jagged as J


def _mask_rows_factory(kind):
    """Mistakes planted on top of the oracle's own mask rows."""
    orig = A.isolation_mask_rows

    def f(seg, rows):
        seg = np.asarray(seg)
        rows = np.asarray(rows, dtype=np.int64)
        role = seg[rows]
        out = orig(seg, rows).copy()
        own = np.nonzero(role == -1)[0]
        if kind == "no_self":
            out[own, rows[own]] = False
        elif kind == "cands_see_cands":
            out[np.ix_(role == -1, seg == -1)] = True
        elif kind == "history_sees_cands":
            out[np.ix_(role == 1, seg == -1)] = True
        elif kind == "pad_query_attends":
            out[np.ix_(role == 0, seg == 1)] = True
        elif kind == "self_shifted":
            out[own, rows[own]] = False
            nxt = rows[own] + 1
            keep = (nxt < len(seg))
            keep[keep] = seg[nxt[keep]] == -1
            out[own[keep], nxt[keep]] = True
        return out
    return f


def _softmax_factory(kind):
    def f(q, k, v, mask, scale):
        q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
        out = np.zeros((q.shape[0], v.shape[1]))
        has = mask.any(axis=1)
        if not has.any():
            return out
        if kind == "transposed_scores" and q.shape[0] == k.shape[0]:
            s = scale * (k @ q.T)[has]
        else:
            s = scale * (q[has] @ k.T)
        s = np.where(mask[has], s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(m - s) if kind == "wrong_sign" else np.exp(s - m)
        e = np.where(mask[has], e, 0.0)
        p = e if kind == "no_normalise" else e / e.sum(axis=1, keepdims=True)
        if kind == "values_are_keys":
            out[has] = p @ k
        else:
            out[has] = p @ v
        return out
    return f


def _seg_factory(kind):
    """Mistakes planted on top of the oracle's own segment rule."""
    orig = J.segment_ids

    def f(offsets, cand_start, valid=None, attend_padded_history=False):
        if kind == "strict_start":       # the candidate block starts one row late
            return orig(offsets, np.asarray(cand_start, np.int64) + 1, valid, attend_padded_history)
        if kind == "flag_ignored":
            return orig(offsets, cand_start, valid, False)
        # flag_on_candidates: the flag revives padded candidates instead of padded history
        seg = orig(offsets, cand_start, valid, False)
        if attend_padded_history:
            block = orig(offsets, cand_start, None, False) == -1
            seg = np.where(block, np.int8(-1), seg).astype(np.int8)
        return seg
    return f


def _bounds_off_by_one(offsets, seg):
    out = J.__dict__["_orig_bounds"](offsets, seg)
    out[1] -= 1
    return out


MUTATIONS = {
    "no_self_term": [("A", "isolation_mask_rows", _mask_rows_factory("no_self"))],
    "candidates_see_candidates": [("A", "isolation_mask_rows", _mask_rows_factory("cands_see_cands"))],
    "history_sees_candidates": [("A", "isolation_mask_rows", _mask_rows_factory("history_sees_cands"))],
    "pad_query_attends": [("A", "isolation_mask_rows", _mask_rows_factory("pad_query_attends"))],
    "self_term_wrong_index": [("A", "isolation_mask_rows", _mask_rows_factory("self_shifted"))],
    "transposed_scores": [("A", "masked_softmax_attention", _softmax_factory("transposed_scores"))],
    "softmax_wrong_sign": [("A", "masked_softmax_attention", _softmax_factory("wrong_sign"))],
    "softmax_not_normalised": [("A", "masked_softmax_attention", _softmax_factory("no_normalise"))],
    "values_are_keys": [("A", "masked_softmax_attention", _softmax_factory("values_are_keys"))],
    "scale_dropped": [("A", "_scale", lambda scale, d: 1.0)],
    "scale_not_sqrt": [("A", "_scale", lambda scale, d: 1.0 / d)],
    "candidate_start_strict": [("J", "segment_ids", _seg_factory("strict_start")),
                               ("A", "segment_ids", _seg_factory("strict_start"))],
    "flag_ignored": [("J", "segment_ids", _seg_factory("flag_ignored")),
                     ("A", "segment_ids", _seg_factory("flag_ignored"))],
    "flag_widens_candidates": [("J", "segment_ids", _seg_factory("flag_on_candidates")),
                               ("A", "segment_ids", _seg_factory("flag_on_candidates"))],
    "bounds_off_by_one": [("J", "bounds", _bounds_off_by_one)],
    "offsets_inclusive": [("J", "offsets_from_lengths",
                           lambda lengths: np.cumsum([int(n) for n in lengths]))],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name, monkeypatch):
    monkeypatch.setitem(J.__dict__, "_orig_bounds", J.bounds)
    for mod, attr, fn in MUTATIONS[name]:
        monkeypatch.setattr(A if mod == "A" else J, attr, fn)
    caught = []
    for pin in _pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError) as e:   # noqa: PERF203
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"
