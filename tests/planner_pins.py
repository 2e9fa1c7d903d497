"""Pins of the step-planner oracle (oracle/planner_oracle.py) to facts that do not come
from the oracle itself: the chunk slices the inference-engine page prints for an 8K
prompt under a 2K budget (tests/golden/pages_facts.json), the mixed-step workload's
own composition (2,048 = 31 decode tokens + a 2,017-token chunk at positions
1,483..3,499), and brute-force properties of decode-first filling over random request
mixes."""
from __future__ import annotations

import json
import os

import numpy as np

import oracle.planner_oracle as PL

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pages_facts.json")


def run_until_done(prompt_len, budget, num_computed=None, steps=1000):
    """Steps of the planner until every prompt is cached; returns per step the list of
    (request, first position, count)."""
    nc = list(num_computed or [0] * len(prompt_len))
    hist = []
    for _ in range(steps):
        if all(c >= p for c, p in zip(nc, prompt_len)):
            break
        q = PL.plan_step(prompt_len, nc, budget)
        hist.append([(r, nc[r], q[r]) for r in range(len(q)) if q[r] > 0])
        for r, k in enumerate(q):
            nc[r] += k
    return hist


def pin_pages_8k_prompt_2k_budget():
    """The page's example: an 8K prompt alone under a 2K budget runs as the four
    printed slices, one per pass."""
    with open(GOLDEN) as f:
        ex = json.load(f)["chunked_prefill_8k_prompt_2k_budget"]
    hist = run_until_done([ex["prompt_len"]], ex["budget"])
    got = [[first, first + k - 1] for step in hist for (_, first, k) in step]
    assert got == ex["chunks_inclusive"]


def pin_decoders_never_stall():
    """The page's point: while the long prompt is sliced, every active user still gets
    its one decode token in every step (decode tokens fill the step first)."""
    prompts = [300, 300, 300, 8192]        # three users already decoding, one long prompt
    nc = [300, 300, 300, 0]
    hist = run_until_done([p + 100 for p in prompts[:3]] + [8192], 2048,
                          num_computed=nc)
    for step in hist:
        sched = {r: k for r, _, k in step}
        for r in range(3):
            assert sched.get(r) is not None
    chunks = [k for step in hist for (r, _, k) in step if r == 3]
    assert sum(chunks) == 8192 and all(k <= 2048 for k in chunks)


def pin_mixed_step_workload_composition():
    """The mixed-step workload: a 3,500-token prompt with 1,483 positions cached and 31
    decoding requests under a 2,048-token budget give exactly the 2,017-token chunk at
    positions 1,483..3,499 plus 31 single decode tokens."""
    prompt = [3500] + [1000] * 31
    nc = [1483] + [1000 + k for k in range(31)]      # decoders: prompt fully cached
    q = PL.plan_step(prompt, nc, 2048)
    assert q[0] == 2017 and q[1:] == [1] * 31
    seqs, qsl, ctx = PL.batch_of(nc, q)
    assert seqs == list(range(32)) and qsl[1] == 2017 and qsl[-1] == 2048
    assert ctx[0] == 3500 and ctx[1:] == [1001 + k for k in range(31)]


def pin_budget_properties_random_mixes():
    """Brute force over random mixes: never over budget; work-conserving (uses
    min(budget, demand)); a decoder is left out only if decoders alone filled the
    budget; prompt slices go in request order (after a request gets less than it still
    needs, no later prompt gets anything); chunks continue the cached positions."""
    rng = np.random.Generator(np.random.PCG64(21))
    for _ in range(3000):
        n = int(rng.integers(1, 12))
        prompt = [int(x) for x in rng.integers(0, 5000, n)]
        nc = [int(min(p, x)) if rng.random() < 0.5 else p for p, x in
              zip(prompt, rng.integers(0, 5000, n))]
        budget = int(rng.integers(1, 4096))
        q = PL.plan_step(prompt, nc, budget)
        decoding = [r for r in range(n) if prompt[r] > 0 and nc[r] >= prompt[r]]
        filling = [r for r in range(n) if nc[r] < prompt[r]]
        demand = len(decoding) + sum(prompt[r] - nc[r] for r in filling)
        assert sum(q) <= budget and sum(q) == min(budget, demand)
        if any(q[r] == 0 for r in decoding):
            assert sum(q[r] for r in decoding) == budget
            assert all(q[r] == 0 for r in filling)
        for r in decoding:
            assert q[r] in (0, 1)
        short = False
        for r in filling:
            assert 0 <= q[r] <= prompt[r] - nc[r]
            if short:
                assert q[r] == 0
            if q[r] < prompt[r] - nc[r]:
                short = True
        for r in range(n):
            if prompt[r] == 0:
                assert q[r] == 0


def pin_slices_cover_prompts_once():
    """Over many steps every prompt is covered by contiguous slices, each position once
    (a request whose prompt is done decodes one token per step meanwhile)."""
    rng = np.random.Generator(np.random.PCG64(4))
    for _ in range(50):
        prompt = [int(x) for x in rng.integers(1, 6000, int(rng.integers(1, 8)))]
        hist = run_until_done(prompt, int(rng.integers(64, 3000)))
        nxt = [0] * len(prompt)
        for step in hist:
            for r, first, k in step:
                assert first == nxt[r]
                assert first < prompt[r] or k == 1
                nxt[r] += k
        assert all(n >= p for n, p in zip(nxt, prompt))


ALL_PINS = [pin_pages_8k_prompt_2k_budget, pin_decoders_never_stall,
            pin_mixed_step_workload_composition, pin_budget_properties_random_mixes,
            pin_slices_cover_prompts_once]
