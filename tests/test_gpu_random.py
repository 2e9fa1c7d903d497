"""GPU parity over seeded random batches.

Each case draws a batch shape at random — element type, head layout, head size,
number of sequences, and per sequence a query count (none, one decode row, or a
chunk) over a context at least that long — plus a scale (sometimes negative or far
from 1/sqrt(d)) and a pool with NaN in every unused slot.  The step runs through the
plain two-call path or the fused call (alternating) and is compared element by
element with the fp64 oracle, and the pools bit for bit.  The draws are fixed by
the seed, so a failure names a reproducible case.
"""
import numpy as np
import pytest

import oracle.pagedkv_oracle as O
from tests.gpu_util import DeviceBatch, out_f64, to_raw, tolerance
from workloads import make_batch

pytestmark = pytest.mark.gpu

HEADS = [(4, 4), (8, 2), (16, 8), (32, 8), (16, 2), (6, 3)]


def _draw(seed):
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    dtype = "f32" if rng.random() < 0.3 else "bf16"
    hq, hkv = HEADS[rng.integers(len(HEADS))]
    d = int(rng.choice([64, 128]))
    n = int(rng.integers(1, 13))
    qlens, ctxs = [], []
    for _ in range(n):
        kind = rng.random()
        q = 0 if kind < 0.1 else (1 if kind < 0.65 else int(rng.integers(2, 201)))
        c = int(rng.integers(max(q, 1), 1501))
        qlens.append(q)
        ctxs.append(c)
    scale = float(rng.choice([1.0, -1.0])) * float(rng.uniform(0.02, 0.3))
    nb = sum((c + 15) // 16 for c in ctxs) + int(rng.integers(0, 64))
    return rng, dict(dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                     num_blocks=nb, context_lens=ctxs, query_lens=qlens, scale=scale)


@pytest.mark.parametrize("seed", range(24))
def test_random_batch_matches_oracle(seed):
    rng, kw = _draw(seed)
    print(f"[case] random seed={seed} {kw}", flush=True)
    b = make_batch(rng, name=f"random{seed}", stale="nan", **kw)
    kp, vp, ref = O.step(b)
    db = DeviceBatch(b)
    out = db.step_fused() if seed % 2 else db.step()
    assert to_raw(db.k_pool).tobytes() == kp.tobytes(), "K pool after the write"
    assert to_raw(db.v_pool).tobytes() == vp.tobytes(), "V pool after the write"
    got = out_f64(out)
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), "non-finite output"
    assert (err <= tolerance(b, ref)).all(), f"max err {err.max():.3g}"
