"""Float64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library in ``exact_tiled_attention_10_amd`` and imports nothing from it.

Two independent CPU implementations live here:

* ``attention`` -- the plain definition (materialise the score matrix, softmax,
  multiply) and its backward through the softmax Jacobian.  This is the oracle
  the GPU path is compared against.
* ``tiled`` -- the tiled online-softmax algorithm with running max / running
  sum, one deferred division, causal tile skipping and analytic counters, plus
  the recomputing backward.  It exists to pin the oracle: the two must agree to
  float64 rounding, and its counters must reproduce the tile, FLOP and traffic
  tables the source pages print.
"""

from .attention import (
    softmax_rows,
    naive_probs,
    naive_fwd,
    naive_fwd_rows,
    naive_bwd_rows,
    naive_bwd,
    visible_mask,
    kv_head_of,
    naive_fwd_gqa,
    naive_bwd_gqa,
    visible_mask_kv,
    naive_fwd_kv,
    naive_bwd_kv,
    e4m3_decode,
    naive_fwd_fp8,
)
from .tiled import (
    online_normaliser,
    tiled_fwd,
    tiled_bwd,
    causal_tile_counts,
)

__all__ = [
    "softmax_rows",
    "naive_probs",
    "naive_fwd",
    "naive_fwd_rows",
    "naive_bwd_rows",
    "naive_bwd",
    "visible_mask",
    "kv_head_of",
    "naive_fwd_gqa",
    "naive_bwd_gqa",
    "visible_mask_kv",
    "naive_fwd_kv",
    "naive_bwd_kv",
    "e4m3_decode",
    "naive_fwd_fp8",
    "online_normaliser",
    "tiled_fwd",
    "tiled_bwd",
    "causal_tile_counts",
]
