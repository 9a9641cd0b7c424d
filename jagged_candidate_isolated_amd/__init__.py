"""Jagged candidate-isolated attention for MI355X (gfx950).

* ``jagged_candidate_isolated_amd.rr`` -- Python binding of librr's C ABI
  (``rr_segment_ids``, ``rr_bounds``, ``rr_attn_fwd``, ``rr_cand_only_attn_fwd``);
  importing it loads the HIP library and fails if it is not built.
* ``jagged_candidate_isolated_amd.accounting`` -- pair, FLOP and byte accounting.
* ``jagged_candidate_isolated_amd.build`` -- builds librr.so with hipcc.
"""
