"""The CPU oracle against its pins, and the pins against planted oracle mistakes."""
import numpy as np
import pytest

import oracle.pagedkv_oracle as O
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ---------------------------------------------------------------------------
# Mutation checks: each plausible mistake planted in the oracle (on the CPU) must be
# caught by at least one pin.  This is what shows the pins are tight.
# ---------------------------------------------------------------------------

def _m_gqa_interleaved(h, group):           # wrong KV head: h mod (number of groups)
    return h % group


def _m_positions_top_left(ctx, q_len):      # chunk rows aligned at position 0
    return np.arange(0, q_len, dtype=np.int64)


def _m_positions_off_by_one(ctx, q_len):    # each row sees one key too few
    return np.arange(ctx - q_len - 1, ctx - 1, dtype=np.int64)


def _m_table_swapped(table_row, pos):       # block index and offset exchanged
    return int(table_row[pos % 16]), pos // 16


def _m_table_offset(table_row, pos):        # off by one inside the block
    return int(table_row[pos // 16]), (pos + 1) % 16


def _m_locate_swapped(slot):
    return slot % 16, slot // 16


def _m_softmax_unnormalised(scores):
    m = scores.max(axis=1, keepdims=True)
    return np.exp(scores - m)


def _m_softmax_no_mask_zero(scores):        # masked entries leak as weight 1
    m = scores.max(axis=1, keepdims=True)
    w = np.exp(np.where(np.isinf(scores), 0.0, scores - m))
    return w / w.sum(axis=1, keepdims=True)


def _m_to_f64_bad_bf16(raw, dtype):
    if dtype == "bf16":
        bits = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(raw, dtype=np.float32).astype(np.float64)


_ORIG_ATT = O.attention_contiguous


def _m_scale_dropped(q, K, V, scale, positions):
    return _ORIG_ATT(q, K, V, 1.0, positions)


def _m_scale_squared(q, K, V, scale, positions):
    return _ORIG_ATT(q, K, V, scale * scale, positions)


_ORIG_WRITE = O.kv_write


def _m_write_skips_zero(k_pool, v_pool, k_new, v_new, slot_mapping):
    sm = np.asarray(slot_mapping).copy()
    sm[sm == 0] = -1
    return _ORIG_WRITE(k_pool, v_pool, k_new, v_new, sm)


def _m_write_k_only(k_pool, v_pool, k_new, v_new, slot_mapping):
    k2, _ = _ORIG_WRITE(k_pool, v_pool, k_new, v_new, slot_mapping)
    return k2, np.array(v_pool, copy=True)


MUTANTS = {
    "kv_head_of": [_m_gqa_interleaved],
    "query_positions": [_m_positions_top_left, _m_positions_off_by_one],
    "table_lookup": [_m_table_swapped, _m_table_offset],
    "locate": [_m_locate_swapped],
    "softmax_rows": [_m_softmax_unnormalised, _m_softmax_no_mask_zero],
    "to_f64": [_m_to_f64_bad_bf16],
    "attention_contiguous": [_m_scale_dropped, _m_scale_squared],
    "kv_write": [_m_write_skips_zero, _m_write_k_only],
}

CASES = [(name, m) for name, ms in MUTANTS.items() for m in ms]


@pytest.mark.parametrize("target,mutant", CASES, ids=[m.__name__ for _, m in CASES])
def test_pins_catch_planted_mistake(monkeypatch, target, mutant):
    monkeypatch.setattr(O, target, mutant)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {mutant.__name__}"
