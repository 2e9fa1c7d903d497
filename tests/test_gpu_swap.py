"""GPU parity of the KV swap (paged_kv_swap_out / paged_kv_swap_in) against the swap
oracle, bit for bit, and a tool-call idle round trip: a request's blocks go to pinned
host memory, other requests overwrite the freed blocks, the request comes back into
fresh blocks and its attention output is what it was before, bit for bit."""
import numpy as np
import pytest
import torch

import oracle.swap_oracle as S
import paged_kv_cache_290_amd as pkv
from tests.gpu_util import DeviceBatch, to_raw, to_torch
from workloads import make_batch

pytestmark = pytest.mark.gpu


def _pools(rng, nb, hkv, d, dtype):
    shape = (nb, hkv, 16, d)
    if dtype == "bf16":
        return (rng.integers(0, 1 << 16, size=shape, dtype=np.uint16),
                rng.integers(0, 1 << 16, size=shape, dtype=np.uint16))
    return (rng.standard_normal(shape).astype(np.float32),
            rng.standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("dtype,hkv,d", [("bf16", 8, 128), ("bf16", 8, 64), ("f32", 2, 64)])
def test_swap_matches_oracle(dtype, hkv, d):
    print(f"[case] swap {dtype} hkv={hkv} d={d}", flush=True)
    rng = np.random.Generator(np.random.PCG64(3))
    nb = 200
    kp, vp = _pools(rng, nb, hkv, d, dtype)
    blocks = [int(b) for b in rng.permutation(nb)[:37]]
    k_t, v_t = to_torch(kp, dtype), to_torch(vp, dtype)
    nbytes = pkv.swap_bytes(k_t, len(blocks))
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    staging = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    bl = torch.tensor(blocks + [-1, nb], dtype=torch.int32, device="cuda")
    pkv.swap_out(k_t, v_t, bl[:len(blocks)], staging, host)
    torch.cuda.synchronize()
    want = S.swap_out(kp, vp, blocks)
    assert host.numpy().tobytes() == want.tobytes()
    # Back into other blocks; two extra image blocks with out-of-range ids are skipped.
    dst = [int(b) for b in rng.permutation(nb)[:37]]
    junk = _pools(rng, 2, hkv, d, dtype)
    image = np.concatenate([want[0], junk[0], want[1], junk[1]])
    host2 = torch.from_numpy(np.frombuffer(image.tobytes(), dtype=np.uint8).copy()).pin_memory()
    staging2 = torch.empty(host2.numel(), dtype=torch.uint8, device="cuda")
    kp2, vp2 = S.swap_in(kp, vp, dst, want)
    pkv.swap_in(k_t, v_t, torch.tensor(dst + [-1, nb], dtype=torch.int32, device="cuda"),
                staging2, host2)
    torch.cuda.synchronize()
    assert to_raw(k_t).tobytes() == kp2.tobytes()
    assert to_raw(v_t).tobytes() == vp2.tobytes()


def test_idle_request_round_trip_is_exact():
    """Request 1 of a decode batch goes idle: its blocks are swapped out and freed,
    another request fills them with new K/V, request 1 comes back into fresh blocks,
    and the next decode step gives the same output as before, bit for bit."""
    print("[case] swap round trip, decode batch", flush=True)
    rng = np.random.Generator(np.random.PCG64(8))
    hq, hkv, d, nb = 16, 8, 128, 400
    b = make_batch(rng, name="swap", dtype="bf16", num_q_heads=hq, num_kv_heads=hkv,
                   head_dim=d, num_blocks=nb, context_lens=[300, 640, 77],
                   query_lens=[1, 1, 1], stale="random")
    db = DeviceBatch(b)
    db.write()
    out_before = db.attend().clone()
    torch.cuda.synchronize()
    used = (640 + 15) // 16
    t1 = [int(x) for x in b.block_tables[1, :used]]
    n = len(t1)
    nbytes = pkv.swap_bytes(db.k_pool, n)
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    staging = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    pkv.swap_out(db.k_pool, db.v_pool, torch.tensor(t1, dtype=torch.int32, device="cuda"),
                 staging, host)
    # Another request takes the freed blocks and writes its own K/V into them.
    filler = torch.empty((n, hkv, 16, d), dtype=torch.bfloat16, device="cuda").normal_()
    db.k_pool[t1] = filler
    db.v_pool[t1] = filler
    # Fresh blocks for the returning request: any blocks no table of the batch uses.
    in_use = set(int(x) for x in b.block_tables[b.block_tables >= 0])
    fresh = [x for x in range(nb) if x not in in_use][:n]
    assert len(fresh) == n
    pkv.swap_in(db.k_pool, db.v_pool, torch.tensor(fresh, dtype=torch.int32, device="cuda"),
                staging, host)
    bt = b.block_tables.copy()
    bt[1, :n] = fresh
    db.block_tables = torch.from_numpy(bt.astype(np.int32)).cuda()
    out_after = db.attend()
    torch.cuda.synchronize()
    assert torch.equal(out_before.view(torch.int16), out_after.view(torch.int16))
