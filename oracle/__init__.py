"""Plain float64 CPU oracle for structured-mask softmax attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library; its inputs
come from the seeded generators in ``block_sparse_softmax_amd.inputs`` (which
draw data and hold none of the method's arithmetic).

Contents
--------
attention.py  the definition: explicit token mask from index predicates,
              dense scores, masked softmax with an optional per-head sink in
              the denominator, then P @ V (float64).
tiles.py      the per-query-tile KV tile lists in canonical CSR form, derived
              from the dense mask (and, for block matrices, by index arithmetic).
counts.py     unmasked-pair counts by enumeration of the explicit mask.
rr_search.py  RRAttention's block-pattern search (Eq. 6-12): sampled queries,
              stride-summed keys, stride softmax, block scores, top-tau, the
              last-row protection.
backward.py   the gradients dQ, dK, dV and of the sink logit, and the row
              log-sum-exp, by the chain rule through the masked softmax.
serialize.py  token positions under raster and 2x2-block serialisation orders.
decode.py     one-query decode over a key/value cache: the new token's row of
              the causal window (+ prefix) mask, gathered keys, the same softmax.

Every function is pinned by ``tests/test_oracle*.py`` against brute force,
closed forms, invariants and the worked numbers printed on the pages; see the
module docstrings for the passage each function follows.
"""

from .attention import attention, allowed_rows, bf16_to_f64, dense_mask  # noqa: F401
from .tiles import tile_lists  # noqa: F401
from .counts import pair_count  # noqa: F401
from .rr_search import rr_search  # noqa: F401
from .backward import attention_backward  # noqa: F401
from .decode import decode_attention  # noqa: F401
