"""The seeded input generator: determinism and the workload shapes taken from the pages."""
import json
import os

import numpy as np
import pytest

from workloads import BLOCK_SIZE, make_batch, make_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


def _facts():
    with open(GOLDEN) as f:
        return json.load(f)


def _same(a, b):
    for f in ("k_pool", "v_pool", "block_tables", "context_lens", "query_start_loc", "q",
              "k_new", "v_new", "slot_mapping"):
        if getattr(a, f).tobytes() != getattr(b, f).tobytes():
            return False
    return True


@pytest.mark.parametrize("name", ["tiny_f32_decode", "qwen3_1p7b_decode_640",
                                  "shared_prefix_decode"])
def test_seed_determinism(name):
    assert _same(make_config(name, 3), make_config(name, 3))
    assert not _same(make_config(name, 3), make_config(name, 4))


def test_tiny_config():
    b = make_config("tiny_f32_decode", 0)
    assert b.dtype == "f32" and b.k_pool.shape == (64, 2, 16, 64)
    assert b.context_lens.tolist() == [5, 17, 33, 64]
    assert b.num_q_heads == 4 and b.num_kv_heads == 2
    assert abs(b.scale - 0.125) < 1e-15


def test_capacity_config_matches_pages():
    """22,048 KV tokens in 16-token blocks, 640-token requests: 34 fit."""
    f = _facts()["kv_capacity_tokens"]
    b = make_config("qwen3_1p7b_decode_640", 0)
    assert b.num_blocks * BLOCK_SIZE == f["value"]
    assert b.num_seqs == f["requests_that_fit"] == f["value"] // f["request_tokens"]
    assert b.context_lens.min() >= 512 and b.context_lens.max() <= f["request_tokens"]
    used = b.block_tables[b.block_tables >= 0]
    assert len(np.unique(used)) == len(used) <= b.num_blocks


def test_shared_prefix_config_matches_pages():
    """Only full blocks of the 3,000-token prefix are shareable: 187 blocks, 2,992 tokens."""
    f = _facts()["shared_prefix_tokens"]
    b = make_config("shared_prefix_decode", 0)
    nshared = f["value"] // BLOCK_SIZE
    assert nshared == 187
    assert (b.block_tables[:, :nshared] == b.block_tables[0, :nshared]).all()
    priv = b.block_tables[:, nshared:]
    priv = priv[priv >= 0]
    assert len(np.unique(priv)) == len(priv)
    assert not set(priv.tolist()) & set(b.block_tables[0, :nshared].tolist())
    extra = b.context_lens - nshared * BLOCK_SIZE
    assert extra.min() >= 40 and extra.max() <= 40 + 128


def test_slot_mapping_points_at_last_positions():
    rng = np.random.Generator(np.random.PCG64(1))
    b = make_batch(rng, name="t", dtype="bf16", num_q_heads=2, num_kv_heads=1, head_dim=8,
                   num_blocks=20, context_lens=[3, 16, 40], query_lens=[1, 16, 5])
    slots = b.slot_mapping.tolist()
    assert len(slots) == 22 and len(set(slots)) == 22
    # the chunk of sequence 2 covers positions 35..39: block 2 offsets 3..7
    blk = int(b.block_tables[2, 2])
    assert slots[17:] == [blk * 16 + o for o in range(3, 8)]


def test_stale_nan_only_outside_contexts():
    rng = np.random.Generator(np.random.PCG64(2))
    b = make_batch(rng, name="t", dtype="f32", num_q_heads=2, num_kv_heads=1, head_dim=8,
                   num_blocks=8, context_lens=[3, 20], query_lens=[1, 1], stale="nan")
    assert np.isnan(b.k_pool[b.block_tables[0, 0], 0, 3:]).all()
    assert not np.isnan(b.k_pool[b.block_tables[0, 0], 0, :3]).any()
    assert not np.isnan(b.k_pool[b.block_tables[1, 0]]).any()
