"""The block-bookkeeping oracle against its pins, and the pins against planted
oracle mistakes (each must be caught by at least one pin)."""
import pytest

import oracle.blocks_oracle as B
from tests import blocks_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


class _NoDecrementOnCopy(B.RefcountAllocator):
    """Copy-on-write that forgets to drop the appender's reference to the original."""

    def append(self, table, context_len, num_new):
        ref_before = list(self.ref)
        slots, copies = super().append(table, context_len, num_new)
        for src, _ in copies:
            self.ref[src] = ref_before[src]
        return slots, copies


class _CopyAlways(B.RefcountAllocator):
    """Copies the last block even when the appender is its only holder."""

    def append(self, table, context_len, num_new):
        if num_new and context_len % 16 and self.ref[table[context_len // 16]] == 1:
            self.ref[table[context_len // 16]] += 1
        return super().append(table, context_len, num_new)


class _ForkNoRef(B.RefcountAllocator):
    def fork(self, table):
        return list(table)


class _FreeEarly(B.RefcountAllocator):
    def _drop(self, b):
        self.ref[b] -= 1
        if self.ref[b] <= 1 and b not in self._free:
            import heapq
            self.ref[b] = 0
            heapq.heappush(self._free, b)


class _BoundaryOffByOne(B.RefcountAllocator):
    """Takes the new block one position late (at pos % 16 == 1)."""

    def append(self, table, context_len, num_new):
        slots, copies = [], []
        for i in range(num_new):
            pos = context_len + i
            lb, off = divmod(pos, 16)
            if off == 1 or (off == 0 and lb >= len(table)):
                if lb >= len(table):
                    table.append(self._take())
            slots.append(table[lb] * 16 + off)
        return slots, copies


def _copy_first_head_only(k_pool, v_pool, copies):
    kp, vp = k_pool.copy(), v_pool.copy()
    for src, dst in copies:
        kp[dst, 0] = kp[src, 0]
        vp[dst, 0] = vp[src, 0]
    return kp, vp


@pytest.mark.parametrize("cls", [_NoDecrementOnCopy, _CopyAlways, _ForkNoRef, _FreeEarly,
                                 _BoundaryOffByOne])
def test_pins_catch_planted_allocator_mistake(cls, monkeypatch):
    monkeypatch.setattr(B, "RefcountAllocator", cls)
    caught = 0
    for pin in P.ALL_PINS:
        try:
            pin()
        except (AssertionError, IndexError, KeyError, ValueError, B.OutOfBlocks):
            caught += 1
    assert caught > 0, f"no pin catches {cls.__name__}"


def test_pins_catch_partial_copy(monkeypatch):
    monkeypatch.setattr(B, "copy_blocks", _copy_first_head_only)
    with pytest.raises(AssertionError):
        P.pin_copy_makes_private_equal_to_shared()
