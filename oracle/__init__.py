"""CPU oracle for the MoE token-reordering hot path (test infrastructure only).

This package is a plain, slow, deliberately unoptimised NumPy restatement of
what the two operations compute, written from the method's pages:

* ``ffn_worker_batching`` -- the forward FFN-side batching (aclnnFfnWorkerBatching
  API page, "Function description" steps 2-4 and the calculation formula);
* ``moe_token_unpermute_with_routing_map`` -- the reverse unpermute with optional
  prob-weighted accumulation (MoeTokenUnpermuteWithRoutingMap article, section
  "Function description and formulas", branches 1-4);
* ``moe_token_permute_with_routing_map`` -- the forward permute the same article
  names in "Operator positioning", defined as the arrangement the unpermute's
  formulas invert.

It exists to check the HIP library against.  Only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may import it;
the product package never does, and shares no code with it.

Parity status per function (see each module header for the pins):

* ``numerics``  -- pinned (torch CPU conversions, IEEE special cases).
* ``batching``  -- pinned (API-page worked example, brute force, invariants).
* ``unpermute`` -- pinned for all four branches under the W2 weight reading;
  the W1 switch and the non-padded ``out_index``/``permute_token_id`` outputs
  are pinned only by properties (ranges, permutation, stability) --
  "parity unpinned" beyond those.
* ``permute``   -- pinned (round trips through the unpermute oracle, a torch
  nonzero / cumsum construction, brute force of the capacity blocks).
"""

from .numerics import (  # noqa: F401
    DT_FP16, DT_BF16, DT_FP32, DT_INT8,
    to_f32, from_f32, f32_to_bf16_bits, bf16_bits_to_f32,
)
from .batching import ffn_worker_batching  # noqa: F401
from .unpermute import moe_token_unpermute_with_routing_map  # noqa: F401
from .permute import moe_token_permute_with_routing_map  # noqa: F401
from .schedule import ffn_worker_batching_from_context, decode_schedule_context  # noqa: F401
from .update_expert import moe_update_expert  # noqa: F401
