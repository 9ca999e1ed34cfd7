"""Float64 CPU oracle for the exact attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library and never
imports it.

Sources (cited by title and section throughout):

* [GS]  "How Does FlashAttention Preserve Global Softmax Across Tiles?"
        (youchengli.com) -- operator (section 1), mergeable state (sections 3-4),
        tile recurrence (section 5), global-position masks and empty rows
        (section 6), log-sum-exp (section 7), split-KV decode (section 8),
        CPU checks (section 9).
* [VW]  "Flash attention and efficient attention: Visual walkthrough"
        (brentwoodlivery.com) -- safe softmax (Step 3), per-tile state
        (Step 4), merge (Step 5), worked example (Step 6), edge cases (Step 7).
* [OA]  "Reducing Memory Traffic with Output Accumulation in FlashAttention"
        (llm-systems-engineering.pages.dev) -- weighted sum first (Figure 1),
        chunked update (Figure 2), Q/K/V tiles (Figure 3).

Modules:

* ``dense``  -- the plain definition: materialise S and P row by row.
* ``online`` -- the pages' tile recurrence with arbitrary key partitions and
  visiting orders, plus the two-block merge; used to pin the recurrence
  itself (tile-size and order invariance, the printed chunk states).
* ``backward`` -- gradients by recomputation from the saved output and
  log-sum-exp ([GS] section 7; [VW] Step 8).
* ``dropout`` -- the counter-based dropout mask (Philox4x32-10 from its
  published definition) that forward and backward both replay ([GS]
  section 6).

Parity pins: every function here is pinned by ``-m "not gpu"`` tests against
the pages' printed worked examples, closed forms, invariants and an
independent library routine; no function is "parity unpinned".
"""

from .backward import attention_bwd_head, attention_bwd_ref
from .dropout import dropout_bytes, keep_mask, keep_scale, philox4x32_10
from .dense import allowed_mask, attention_head, attention_ref
from .online import block_state, even_tiles, merge_states, online_ref

__all__ = [
    "allowed_mask",
    "attention_bwd_head",
    "attention_bwd_ref",
    "attention_head",
    "attention_ref",
    "block_state",
    "dropout_bytes",
    "even_tiles",
    "keep_mask",
    "keep_scale",
    "merge_states",
    "online_ref",
    "philox4x32_10",
]
