"""Pins of the swap oracle (oracle/swap_oracle.py): a swap round trip leaves every
token's K/V as it was when read through the request's new table (the inference-engine
page: the KV is restored when the next turn arrives), and the blocks freed in between
can be reused by other requests without harm.  Checked against the attention oracle
(the attention result after the round trip equals the one before) and against planted
mistakes."""
import numpy as np
import pytest

import oracle.blocks_oracle as B
import oracle.pagedkv_oracle as O
import oracle.swap_oracle as S


def _pools(rng, nb, hkv=2, d=8):
    return (rng.standard_normal((nb, hkv, 16, d)).astype(np.float32),
            rng.standard_normal((nb, hkv, 16, d)).astype(np.float32))


def _round_trip(swap_out, swap_in):
    """A request with 50 tokens is swapped out, another request takes the freed blocks
    and writes into them, the first is swapped back into fresh blocks.  Returns the
    request's K/V (through its table) before and after, and its attention output."""
    rng = np.random.Generator(np.random.PCG64(1))
    nb = 8
    kp, vp = _pools(rng, nb)
    a = B.RefcountAllocator(nb)
    t = []
    a.append(t, 0, 50)                                  # blocks 0..3
    k_before = O.gather(kp, t, 50)
    v_before = O.gather(vp, t, 50)
    q = rng.standard_normal((1, 4, 8)).astype(np.float32)
    out_before = O.attention_contiguous(q.astype(np.float64), k_before.astype(np.float64),
                                        v_before.astype(np.float64), 0.3, [49])
    image = swap_out(kp, vp, t)
    a.release(t)
    u = []
    a.append(u, 0, 64)                                  # another request reuses them
    kp[u] = rng.standard_normal(kp[u].shape)
    vp[u] = rng.standard_normal(vp[u].shape)
    t2 = []
    a.append(t2, 0, 50)                                 # fresh blocks: 4..7
    assert set(t2).isdisjoint(u)
    kp, vp = swap_in(kp, vp, t2, image)
    k_after, v_after = O.gather(kp, t2, 50), O.gather(vp, t2, 50)
    out_after = O.attention_contiguous(q.astype(np.float64), k_after.astype(np.float64),
                                       v_after.astype(np.float64), 0.3, [49])
    return k_before, v_before, k_after, v_after, out_before, out_after, kp, u


def test_round_trip_restores_the_request():
    kb, vb, ka, va, ob, oa, _, _ = _round_trip(S.swap_out, S.swap_in)
    assert np.array_equal(kb, ka) and np.array_equal(vb, va)
    assert np.array_equal(ob, oa)


def test_swap_in_touches_only_its_blocks():
    rng = np.random.Generator(np.random.PCG64(2))
    kp, vp = _pools(rng, 10)
    image = S.swap_out(kp, vp, [7, 2])
    assert image.shape == (2, 2, 2, 16, 8)
    assert np.array_equal(image[0, 0], kp[7]) and np.array_equal(image[1, 1], vp[2])
    kp2, vp2 = S.swap_in(kp, vp, [4, 5], image)
    for b in range(10):
        if b not in (4, 5):
            assert np.array_equal(kp2[b], kp[b]) and np.array_equal(vp2[b], vp[b])
    assert np.array_equal(kp2[4], kp[7]) and np.array_equal(vp2[5], vp[2])


def _mutant_k_twice(k_pool, v_pool, blocks):
    idx = np.asarray(blocks, dtype=np.int64)
    return np.stack([k_pool[idx], k_pool[idx]])


def _mutant_reversed(k_pool, v_pool, blocks, image):
    return S.swap_in(k_pool, v_pool, list(blocks)[::-1], image)


@pytest.mark.parametrize("out_fn,in_fn", [(_mutant_k_twice, S.swap_in),
                                          (S.swap_out, _mutant_reversed)])
def test_pins_catch_planted_mistakes(out_fn, in_fn):
    kb, vb, ka, va, ob, oa, _, _ = _round_trip(out_fn, in_fn)
    assert not (np.array_equal(kb, ka) and np.array_equal(vb, va))
