"""CPU oracle for the chunked-prefill step planner: which tokens of which requests run
in one engine step under a token budget, and the varlen batch that step hands to the
paged-attention path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute
this module: only the tests use it.  It shares no code with the library's planner.

What it computes, and where that is defined (pages cited by title and section):

* "How inference engines actually work" page (xiaohu-jiedu), Chunked Prefill
  subsection: each step has a compute budget in tokens (2K in the page's example); a
  long prompt is not prefilled at once but cut into consecutive slices that fit the
  budget (an 8K prompt: 0-2047, 2048-4095, 4096-6143, 6144-8191, over four passes),
  and in every such step the active users' single decode tokens are packed in too,
  so decoding never stalls.
* Serving-engine KV page (ttlab), section 3, "the new problem": chunked prefill
  combined with filling the step with decode tokens first ("decode-first fill").
  Read with the page's own measurement (the per-step input-token limit,
  --max-num-batched-tokens, counts every token of the step), the budget covers
  decode tokens and chunk tokens together.

So one step: every request in its decode phase (its prompt fully cached) gets its one
next token, in request order, while the budget lasts; the budget left over goes to
requests still prefilling, in request order, each taking the next
min(remaining prompt, remaining budget) prompt tokens as one chunk.  A chunk always
continues where the request's cached positions end.

Readings where the pages are silent (also listed in the design notes):
* "Request order" is the order the caller lists the requests in (arrival order).
* A request whose prompt has length 0 is not scheduled.
* The step's varlen batch lists the scheduled requests in request order; each
  sequence's context_len counts its cached tokens plus this step's tokens.
"""
from __future__ import annotations


def plan_step(prompt_len: list[int], num_computed: list[int], budget: int) -> list[int]:
    """Tokens each request runs this step (0 = not scheduled).  num_computed[r] is how
    many of request r's tokens already have their K/V in the cache; a request with
    num_computed >= prompt_len is decoding (one new token per step)."""
    n = len(prompt_len)
    q = [0] * n
    left = budget
    for r in range(n):                       # decode tokens first
        if prompt_len[r] > 0 and num_computed[r] >= prompt_len[r] and left > 0:
            q[r] = 1
            left -= 1
    for r in range(n):                       # then prompt slices with what is left
        if left == 0:
            break
        if num_computed[r] < prompt_len[r]:
            take = min(prompt_len[r] - num_computed[r], left)
            q[r] = take
            left -= take
    return q


def batch_of(num_computed: list[int], q: list[int]):
    """The varlen batch of one step: (request index per sequence, query_start_loc,
    context_lens).  Sequence s is the s-th scheduled request in request order; its
    rows are positions num_computed .. num_computed + q - 1."""
    seqs = [r for r in range(len(q)) if q[r] > 0]
    qsl = [0]
    for r in seqs:
        qsl.append(qsl[-1] + q[r])
    ctx = [num_computed[r] + q[r] for r in seqs]
    return seqs, qsl, ctx
