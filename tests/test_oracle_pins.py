"""The fp64 oracle against its pins, and planted mistakes against the pins.

Every pin must pass on the oracle as written. Then each plausible mistake
(a wrong index, a dropped term, a swapped operand) is planted in the oracle
on the CPU, and at least one pin must catch it -- otherwise the pins would
not be able to tell a wrong oracle from a right one.
"""

import math

import pytest
import torch

import oracle
from oracle import fp64 as OA

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()


def _merge_drop_b_scale(a, b):
    ma, la, oa = a
    mb, lb, ob = b
    m = torch.maximum(ma, mb)
    sa = torch.exp(ma - m)
    return m, la * sa + lb, oa * sa.unsqueeze(-1) + ob


def _branch_context_swapped(inp, b, page_size):
    k, v = ORIGINAL_BRANCH_CONTEXT(inp, b, page_size)
    return v, k


ORIGINAL_BRANCH_CONTEXT = OA.branch_context
ORIGINAL_APPEND = OA.append_kv


def _append_from_front(k_pages, v_pages, table, private_len, n_new, k_new, v_new, ps):
    return ORIGINAL_APPEND(k_pages, v_pages, table, [0] * len(n_new), n_new, k_new, v_new, ps)

def _slots_in_sorted_order(items):
    # right for a full call or an in-order sample, wrong for any other order
    return {x: i for i, x in enumerate(sorted(items))}


def _slots_first_only(items):
    # every requested id after the first lands on the slot of the one before it
    return {x: max(0, i - 1) for i, x in enumerate(items)}


MUTATIONS = {
    "gqa_interleaved_heads": ("kv_head_of", lambda h, hq, hkv: h % hkv),
    "queries_at_first_positions": ("query_positions", lambda C, T: torch.arange(0, T)),
    "causal_strict_diagonal": ("key_visible",
                               lambda kp, qp, c: (kp.view(1, -1) < qp.view(-1, 1)) if c
                               else torch.ones(qp.numel(), kp.numel(), dtype=torch.bool)),
    "causal_ignored": ("key_visible",
                       lambda kp, qp, c: torch.ones(qp.numel(), kp.numel(), dtype=torch.bool)),
    "page_and_slot_swapped": ("private_location", lambda i, ps: (i % ps, i // ps)),
    "slot_off_by_one": ("private_location", lambda i, ps: (i // ps, (i + 1) % ps)),
    "scale_dropped": ("default_scale", lambda d: 1.0),
    "scale_one_over_d": ("default_scale", lambda d: 1.0 / d),
    "lse_without_max": ("lse_of", lambda m, l: torch.log(l)),
    "lse_log2": ("lse_of", lambda m, l: m + torch.log2(l)),
    "merge_drops_rescale": ("merge_states", _merge_drop_b_scale),
    "k_and_v_swapped": ("branch_context", _branch_context_swapped),
    "append_from_slot_zero": ("append_kv", _append_from_front),
    "sample_slots_sorted": ("sample_slots", _slots_in_sorted_order),
    "sample_slots_shifted": ("sample_slots", _slots_first_only),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(OA, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    failing = P.failing_pins()
    assert failing, f"planted mistake {name!r} passed every pin"
