"""CPU oracle for KV swap: moving a request's blocks out of the GPU pools into host
memory and back into (possibly different) blocks.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute
this module: only the tests use it.  It shares no code with the library's swap
kernels.

What it computes, and where that is defined (pages cited by title and section):

* "How inference engines actually work" page (xiaohu-jiedu), agent-traffic section
  (long idle during tool execution): a request's KV cache is moved out of GPU memory
  into larger, cheaper CPU memory while the request waits, and moved back when its
  next turn arrives.
* Serving-engine KV page (ttlab), section 5 ("when KV capacity runs short"): the
  alternative is preemption, where a running request gives up its KV and is prefilled
  again from the start later (the same KV computed twice).

So a swap-out copies every row of the listed blocks (all kv heads, all 16 offsets,
both pools) to host memory, bit for bit, after which the blocks can be freed; a
swap-in copies them back into whatever blocks are free then, and the request's table
names those.  Readings (also in the design notes): the host image holds the K rows
of block 0..n-1 followed by the V rows of block 0..n-1, each block as it lies in the
pool; a swap moves whole blocks, stale rows past the context included.
"""
from __future__ import annotations

import numpy as np


def swap_out(k_pool: np.ndarray, v_pool: np.ndarray, blocks) -> np.ndarray:
    """Host image of `blocks`: [2, n, num_kv_heads, 16, head_dim] (K then V)."""
    idx = np.asarray(blocks, dtype=np.int64)
    return np.stack([k_pool[idx], v_pool[idx]])


def swap_in(k_pool: np.ndarray, v_pool: np.ndarray, blocks, image: np.ndarray):
    """Pools with `image` (from swap_out) written into `blocks`, in order."""
    kp, vp = k_pool.copy(), v_pool.copy()
    for i, b in enumerate(blocks):
        kp[b] = image[0, i]
        vp[b] = image[1, i]
    return kp, vp
