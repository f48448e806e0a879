"""CPU oracle for exact scaled-dot-product attention (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Nothing in the product imports this package: it
is used by ``tests/``, by ``__graft_entry__.smoke()`` and by the
``cpu_baseline`` leg of ``bench.py``.  It shares no code with the GPU
library and imports nothing from it.

Modules
-------
attention_ref
    The plain definition of attention, materialising S and P in fp64
    (forward, LSE, and the exact backward).
tiled_model
    A CPU model of the tiled double loop with an online softmax, following
    the steps the pages describe; used only to show that the recurrence
    reaches the plain definition.
fp8_ref
    FP8 (E4M3FN) codes, 64-row block quantisation with per-block scales, and
    attention on the dequantised inputs.
"""
from .attention_ref import (  # noqa: F401
    resolve_scale,
    ref_scores,
    ref_probs,
    ref_fwd,
    ref_fwd_rows,
    ref_bwd,
    ref_bwd_group,
    query_positions,
    local_visible,
    softcap_logits,
)
from .tiled_model import tiled_fwd  # noqa: F401
