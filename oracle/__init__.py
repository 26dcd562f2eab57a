"""CPU fp64 oracle for shared-prefix GQA attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or
links this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
path (``gqa_attention_agentic_amd``); both take their seeded inputs from
``workload/``, which holds no attention arithmetic.

What it computes is plain softmax attention, in float64, materialising the
full score row of every query over its branch's whole context (shared
prefix followed by the branch's paged private suffix). ADR-0060 GQA fused
attention (Algorithm lineage paragraph) states that the tiled online
softmax, the split-KV log-sum-exp merge and the ring fold introduce no new
mathematics, so their exact result is this definition.

Pins: every function here is checked in ``tests/test_oracle_pins.py``
against brute force, a library routine (torch's scaled_dot_product_attention
on tiny inputs), closed forms, hand-derived golden cases in
``tests/golden/`` and the invariants the pages state. No function is
parity-unpinned.
"""

from .fp64 import (  # noqa: F401
    kv_head_of, default_scale, lse_of, query_positions, key_visible, private_location, append_kv,
    branch_context, attention, sample_slots, heads_of_kv, partial_state, merge_states, finalize,
    EMPTY_LSE,
)
