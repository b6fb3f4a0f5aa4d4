"""CPU oracle for the exact attention forward pass (float64, numpy).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import it; the HIP library and
its Python binding never do, and the oracle never imports them.

  * ``ref``   - the plain definition, score matrix materialised.
  * ``tiled`` - the Q-outer online-softmax recurrence with tile sizes as
                arguments, used to pin the recurrence to the definition.
  * ``backward`` - the gradients dQ, dK, dV of the forward, from the plain
                definition and in the recomputation form (P from the saved
                LSE, D = O . dO).
  * ``variants`` - grouped K/V heads, queries at an offset into a longer
                key sequence, a sliding window, and split-KV partials with
                their merge.
  * ``native`` - the tiled recurrence in plain C (``tiled_ref.c``, fp64),
                loaded through ctypes; imported on its own (``from oracle
                import native``), not from here.
"""

from .ref import as_f64, scores_ref, probabilities_ref, attention_ref, attention_rows_ref
from .tiled import tiled_ref
from .variants import (attention_ex_ref, attention_ex_rows_ref, attention_split_ref, merge_mla_ref,
                       merge_partials_ref, visible_mask)
from .backward import (attention_bwd_ref, attention_bwd_from_lse_ref, attention_bwd_rows_ref,
                       attention_bwd_cols_ref)

__all__ = [
    "as_f64", "scores_ref", "probabilities_ref", "attention_ref",
    "attention_rows_ref", "tiled_ref", "attention_bwd_ref", "attention_bwd_from_lse_ref",
    "attention_bwd_rows_ref", "attention_bwd_cols_ref", "attention_ex_ref", "attention_ex_rows_ref",
    "visible_mask", "attention_split_ref", "merge_partials_ref", "merge_mla_ref",
]
