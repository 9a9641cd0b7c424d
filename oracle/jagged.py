"""Oracle: jagged offsets, segment IDs and bounds (test infrastructure only).

Plain loops over users; no blocking.  Citations name the page and section the
step follows.
"""
from __future__ import annotations

import numpy as np


def offsets_from_lengths(lengths) -> np.ndarray:
    """Offsets of a jagged values array: 0 followed by the running total of the lengths.

    HSTU scaling notes, section "手算 padding 的浪费与 offset": sequence i occupies
    ``values[offsets[i]:offsets[i+1]]``."""
    offsets = [0]
    for n in lengths:
        n = int(n)
        if n < 0:
            raise ValueError("negative length")
        offsets.append(offsets[-1] + n)
    return np.array(offsets, dtype=np.int64)


def segment_ids(offsets, cand_start, valid=None, attend_padded_history=False) -> np.ndarray:
    """Per-row segment ID: 1 = valid prefix/history, -1 = valid candidate, 0 = padding.

    Candidate isolation attention mask page, section "段 ID：掩码的表达方式".  Each row
    belongs to one user; the user's candidate block is every row from its candidate
    start onward.  A row's role is "candidate" (-1) inside that block and "history" (1)
    before it.  A row keeps its role when the padding mask marks it valid -- and, with
    ``attend_padded_history``, every row before the candidate block keeps it too --
    otherwise it is padding (0).

    ``offsets`` int [B+1]; ``cand_start`` int [B], absolute row of user b's first
    candidate; ``valid`` [T] truthy mask or None (= every row valid)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    cand_start = np.asarray(cand_start, dtype=np.int64)
    n_users = len(offsets) - 1
    n_rows = int(offsets[-1]) if n_users >= 0 else 0
    owner = np.repeat(np.arange(n_users), np.diff(offsets))       # user of every row
    row = np.arange(n_rows)
    in_candidate_block = row >= cand_start[owner]
    role = np.where(in_candidate_block, -1, 1)
    kept = np.ones(n_rows, dtype=bool) if valid is None else np.asarray(valid).astype(bool)
    if attend_padded_history:
        kept = kept | ~in_candidate_block
    return np.where(kept, role, 0).astype(np.int8)


def bounds(offsets, seg) -> np.ndarray:
    """Per-user ``[history_lower, history_upper)`` and ``[candidate_lower, candidate_upper)``.

    Candidate isolation attention mask page, section "段 ID：掩码的表达方式" (the
    attention operator derives history and candidate intervals from the segment
    IDs).  Reading: one interval pair per user, the tight hull of its segment-1
    rows and of its segment -1 rows, as absolute rows.  An empty history hull is
    ``[offsets[b], offsets[b])``; an empty candidate hull is
    ``[offsets[b+1], offsets[b+1])``.  Returns int64 [4, B]: hist_lo, hist_hi,
    cand_lo, cand_hi."""
    offsets = np.asarray(offsets, dtype=np.int64)
    seg = np.asarray(seg)
    B = len(offsets) - 1
    out = np.zeros((4, B), dtype=np.int64)
    for b in range(B):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        hist_rows = [r for r in range(lo, hi) if seg[r] == 1]
        cand_rows = [r for r in range(lo, hi) if seg[r] == -1]
        out[0, b], out[1, b] = (min(hist_rows), max(hist_rows) + 1) if hist_rows else (lo, lo)
        out[2, b], out[3, b] = (min(cand_rows), max(cand_rows) + 1) if cand_rows else (hi, hi)
    return out
