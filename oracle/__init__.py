"""Plain fp64 CPU oracle for SpecKV / SpecPC importance scoring (test infrastructure).

This package is TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The HIP library and
its Python binding never import, link or call anything in here, and this
package imports nothing from the library: the two share no code.

Every function follows the text of the paper notes "Draft-based Approximate
Inference for LLMs" (ICLR 2026 notes page, section "Background": attention
and KV cache cost; section "Key designs": the SpecKV, SpecPC and SpecKV-PC
paragraphs; section "Loss / training strategy": local pooling).
Where the pages leave a step open, the reading taken is stated in the
function's docstring under "Reading".

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(closed forms, library special cases, brute force, invariants); none is
"parity unpinned".
"""
from .speckv import (  # noqa: F401
    default_scale,
    row_logits,
    row_probabilities,
    head_scores,
    speckv_scores,
    pool1d,
    select_kept,
    speckv_select,
    compact_rows,
    speckv_compact,
    n_keep,
)
from .specpc import (  # noqa: F401
    default_query_weights,
    causal_window_probabilities,
    specpc_attention_mean,
    specpc_token_scores,
    specpc_select,
)
from .theorem1 import pre_softmax_scores, theorem1_bound  # noqa: F401
from .cascade import gather_tokens, speckv_pc_cascade  # noqa: F401
from .decode import decode_attention, error_scale, head_attention  # noqa: F401
