"""The step-planner oracle against its pins, and the pins against planted mistakes."""
import pytest

import oracle.planner_oracle as PL
from tests import planner_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def _prefill_first(prompt_len, num_computed, budget):
    n = len(prompt_len)
    q, left = [0] * n, budget
    for r in range(n):
        if num_computed[r] < prompt_len[r] and left:
            q[r] = min(prompt_len[r] - num_computed[r], left)
            left -= q[r]
    for r in range(n):
        if prompt_len[r] > 0 and num_computed[r] >= prompt_len[r] and left:
            q[r], left = 1, left - 1
    return q


def _budget_excludes_decodes(prompt_len, num_computed, budget):
    n = len(prompt_len)
    q = [1 if prompt_len[r] > 0 and num_computed[r] >= prompt_len[r] else 0 for r in range(n)]
    left = budget
    for r in range(n):
        if num_computed[r] < prompt_len[r] and left:
            q[r] = min(prompt_len[r] - num_computed[r], left)
            left -= q[r]
    return q


def _largest_prompt_first(prompt_len, num_computed, budget):
    n = len(prompt_len)
    q, left = [0] * n, budget
    for r in range(n):
        if prompt_len[r] > 0 and num_computed[r] >= prompt_len[r] and left:
            q[r], left = 1, left - 1
    for r in sorted(range(n), key=lambda r: -(prompt_len[r] - num_computed[r])):
        if num_computed[r] < prompt_len[r] and left:
            q[r] = min(prompt_len[r] - num_computed[r], left)
            left -= q[r]
    return q


def _fixed_chunk(prompt_len, num_computed, budget):
    """Slices of at most budget - 1 tokens even when nothing else is scheduled."""
    q = PL.__dict__["_orig_plan"](prompt_len, num_computed, budget)
    return [min(k, max(budget - 1, 1)) for k in q]


@pytest.mark.parametrize("wrong", [_prefill_first, _budget_excludes_decodes,
                                   _largest_prompt_first, _fixed_chunk])
def test_pins_catch_planted_planner_mistake(wrong, monkeypatch):
    monkeypatch.setitem(PL.__dict__, "_orig_plan", PL.plan_step)
    monkeypatch.setattr(PL, "plan_step", wrong)
    caught = 0
    for pin in P.ALL_PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin catches {wrong.__name__}"
