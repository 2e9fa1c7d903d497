"""The read-only probe (pkv_read_probe) reads exactly the tiles it is given.

The probe's rate is what the decode kernel is compared against, so its bytes must be
real: each wave folds the words its lane 0 loads into one XOR, and the test rebuilds
those XORs on the CPU from the same buffer and tile list (in-range and clamped
indices, tiles of 1, 2 and 4 KiB, shares that are not a multiple of the unroll).
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_290_amd as pkv

pytestmark = pytest.mark.gpu


def _expected(base_u32, tiles, tile_bytes, waves):
    """XOR per wave of the words lane 0 loads (the kernel's loop, replayed)."""
    n = len(tiles)
    base_tiles = len(base_u32) * 4 // tile_bytes
    per_tile = tile_bytes // 1024
    per_wave = (n + waves - 1) // waves
    out = np.zeros(waves, dtype=np.uint32)
    for w in range(waves):
        t_begin, acc = min(n, w * per_wave), np.uint32(0)
        t_end = min(n, t_begin + per_wave)
        for c0 in range(t_begin, t_end, 64):
            nc = min(64, t_end - c0)
            idx = np.clip(tiles[c0:c0 + nc].astype(np.int64), 0, base_tiles - 1)
            nl = nc * per_tile
            for l in range(0, nl, 4):
                for u in range(4):
                    ll = min(l + u, nl - 1)
                    k, j = divmod(ll, per_tile)
                    word0 = (int(idx[k]) * tile_bytes + j * 1024) // 4  # lane 0's 16 bytes
                    for q in range(4):
                        acc ^= base_u32[word0 + q]
        out[w] = acc  # lane 0 folds in lane index 0
    return out


@pytest.mark.parametrize("tile_bytes,ntiles,grid", [(2048, 1000, 3), (4096, 257, 2),
                                                    (1024, 130, 1)])
def test_probe_reads_the_named_tiles(tile_bytes, ntiles, grid):
    rng = np.random.Generator(np.random.PCG64(tile_bytes + ntiles))
    nbytes = 64 * tile_bytes
    base = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    tiles = rng.integers(-3, 64 + 3, ntiles).astype(np.int32)  # some out of range
    print(f"[case] probe tile_bytes={tile_bytes} tiles={ntiles} grid={grid}", flush=True)
    dev_base = torch.from_numpy(base.view(np.int32)).cuda()
    dev_tiles = torch.from_numpy(tiles).cuda()
    sink = torch.zeros(grid * 4, dtype=torch.int32, device="cuda")
    pkv.read_probe(dev_base, dev_tiles, tile_bytes, sink, grid)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    want = _expected(base, tiles, tile_bytes, grid * 4)
    assert (got == want).all(), f"{np.flatnonzero(got != want)[:8]}"
