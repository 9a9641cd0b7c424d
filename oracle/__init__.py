"""Oracle: a plain, slow, float64 CPU implementation of jagged candidate-isolated attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run anything in this package; the product path
(the HIP library and its Python binding) never does, and shares no code with it.

What it computes (Candidate isolation attention mask page, sections
"段 ID：掩码的表达方式", "掩码长什么样" and "只更新候选的末尾层"):

  1. per-row segment IDs from the candidate start and the padding mask;
  2. per-user history / candidate bounds;
  3. for every user and head, the explicit [L, L] boolean mask built from the
     segment IDs, then dense softmax attention in float64;
  4. candidate-only layers as the page's fallback: the full layer over the
     concatenation [frozen history | candidates], keeping the candidate rows;
  5. right-anchored rotary positions and the rotary encoding of q and k (section
     "位置编码：候选共用一个位置"; ``rotary.py``);
  6. the gradients of the attention w.r.t. q, k, v and each row's log-sum-exp
     (``backward.py``), from the forward's definition and the softmax derivative, for
     full-sequence and candidate-only layers;
  7. the ranker's layer stack (``ranker.py``): full layers, the split into frozen
     history and candidates, candidate-only layers, and the cached request that reuses
     the history's keys and values (section "只更新候选的末尾层"), each layer read as a
     pre-norm attention block with random projections.

Readings of the pages where they are silent (each listed in the design notes):
softmax attention with scale 1/sqrt(d); bidirectional history; rows with no
admitted key (segment 0) output 0; bounds are tight hulls, empty hulls sit at
the user's start (history) or end (candidates); the frozen history of a
candidate-only layer includes the prefix.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against the
pages' worked examples, brute force with exactly rounded sums, a library
routine (torch's CPU scaled_dot_product_attention in float64), closed forms
and the invariants the page states.  No function is "parity unpinned".
"""
from .jagged import offsets_from_lengths, segment_ids, bounds  # noqa: F401
from .attention import (  # noqa: F401
    isolation_mask_rows, isolation_mask, masked_softmax_attention, full_attention,
    full_attention_rows, cand_only_attention, cand_only_attention_rows, DEFAULT_SCALE,
)
from .rotary import (  # noqa: F401
    right_anchored_positions, rotary_angles, rope, full_attention_rope, cand_only_attention_rope,
)
from .backward import (  # noqa: F401
    full_attention_backward, attention_lse, gradient_error_scale, cand_only_attention_backward,
    cand_only_gradient_error_scale,
)
from .ranker import (  # noqa: F401
    Layer, rms_norm, block_full, block_cand_only, block_user_token_layer, history_kv,
    split_history_and_candidates,
    ranker_forward, ranker_forward_cached,
)
