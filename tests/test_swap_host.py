"""Host-side checks of the swap entry points through the C ABI: the image size, and
argument errors returned before any launch (no GPU needed)."""
from paged_kv_cache_290_amd import _lib


def test_swap_bytes():
    lib = _lib.load()
    assert lib.paged_kv_swap_bytes(3, 8, 128, 16, _lib.PKV_BF16) == 2 * 3 * 8 * 16 * 128 * 2
    assert lib.paged_kv_swap_bytes(5, 2, 64, 16, _lib.PKV_F32) == 2 * 5 * 2 * 16 * 64 * 4
    assert lib.paged_kv_swap_bytes(0, 8, 128, 16, _lib.PKV_BF16) == 0
    assert lib.paged_kv_swap_bytes(3, 8, 128, 32, _lib.PKV_BF16) == 0


def test_swap_argument_errors():
    lib = _lib.load()
    for fn in (lib.paged_kv_swap_out, lib.paged_kv_swap_in):
        # unsupported shapes and types
        assert fn(None, None, None, 1, None, None, 8, 2, 96, 16, _lib.PKV_BF16, None) == \
            _lib.PKV_ERR_UNSUPPORTED
        assert fn(None, None, None, 1, None, None, 8, 2, 64, 8, _lib.PKV_BF16, None) == \
            _lib.PKV_ERR_UNSUPPORTED
        assert fn(None, None, None, 1, None, None, 8, 2, 64, 16, 7, None) == \
            _lib.PKV_ERR_UNSUPPORTED
        # bad sizes and missing buffers
        assert fn(None, None, None, -1, None, None, 8, 2, 64, 16, _lib.PKV_BF16, None) == \
            _lib.PKV_ERR_INVALID_ARG
        assert fn(None, None, None, 2, None, None, 8, 2, 64, 16, _lib.PKV_BF16, None) == \
            _lib.PKV_ERR_INVALID_ARG
        assert fn(None, None, None, 0, None, None, 0, 2, 64, 16, _lib.PKV_BF16, None) == \
            _lib.PKV_ERR_INVALID_ARG
        # nothing to move: a no-op
        assert fn(None, None, None, 0, None, None, 8, 2, 64, 16, _lib.PKV_BF16, None) == \
            _lib.PKV_OK
