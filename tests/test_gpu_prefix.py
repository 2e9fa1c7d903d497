"""End-to-end prefix caching on the GPU: requests with a common 3,000-token prefix and
their own 32-token tails.  The first request prefills everything and registers its
full blocks; each later one finds 187 blocks (2,992 tokens) through the prefix cache,
prefills only its last 40 tokens over the shared blocks, and then all of them decode a
token.  Every output equals contiguous-cache attention over the request's own K/V
history (the attention oracle), and the shared blocks are never written after the
first request filled them."""
import numpy as np
import pytest
import torch

import oracle.pagedkv_oracle as O
import paged_kv_cache_290_amd as pkv
from tests.gpu_util import BF16_TOL, out_f64, to_raw, to_torch
from workloads.synth import bf16_round_bits

pytestmark = pytest.mark.gpu


def _draw(rng, shape):
    return bf16_round_bits(rng.standard_normal(size=shape, dtype=np.float32))


def test_shared_prefix_through_the_prefix_cache():
    print("[case] prefix cache: 4 requests, 3,000-token common prefix", flush=True)
    rng = np.random.Generator(np.random.PCG64(77))
    hq, hkv, d, nb, mb = 16, 8, 128, 512, 200
    scale = 1.0 / np.sqrt(d)
    alloc = pkv.BlockAllocator(nb)
    alloc.enable_prefix_cache()
    kp = to_torch(_draw(rng, (nb, hkv, 16, d)), "bf16")
    vp = to_torch(_draw(rng, (nb, hkv, 16, d)), "bf16")
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()  # noqa
    prefix = [int(x) for x in rng.integers(0, 151_936, 3000)]
    kpre, vpre = _draw(rng, (3000, hkv, d)), _draw(rng, (3000, hkv, d))
    reqs = []
    for r in range(4):
        tail = [int(x) for x in rng.integers(0, 151_936, 32)]
        toks = prefix + tail
        khist = np.concatenate([kpre, _draw(rng, (32, hkv, d))])
        vhist = np.concatenate([vpre, _draw(rng, (32, hkv, d))])
        keys = pkv.block_keys(toks)
        table = alloc.prefix_match(keys)
        cached = 16 * len(table)
        assert cached == (0 if r == 0 else 2992)
        slots, copies = alloc.append(table, cached, len(toks) - cached)
        assert copies == []
        n = len(toks) - cached
        q = _draw(rng, (n, hq, d))
        bt = np.full((1, mb), -1, np.int32)
        bt[0, :len(table)] = table
        before = (to_raw(kp)[table[:187]].copy(), to_raw(vp)[table[:187]].copy()) if r else None
        out = pkv.attention_with_write(
            to_torch(q, "bf16"), to_torch(khist[cached:], "bf16"),
            to_torch(vhist[cached:], "bf16"), kp, vp, i32(slots), i32(bt), i32([len(toks)]),
            i32([0, n]), scale=scale, max_context_len=len(toks), max_query_len=n)
        torch.cuda.synchronize()
        ref = O.attention_contiguous(O.to_f64(q, "bf16"), O.to_f64(khist, "bf16"),
                                     O.to_f64(vhist, "bf16"), scale,
                                     O.query_positions(len(toks), n))
        got = out_f64(out)
        tol = np.maximum(BF16_TOL, np.abs(ref) * 2.0 ** -8 + 2e-3)
        assert np.isfinite(got).all() and (np.abs(got - ref) <= tol).all(), f"request {r}"
        if r:
            assert to_raw(kp)[table[:187]].tobytes() == before[0].tobytes()
            assert to_raw(vp)[table[:187]].tobytes() == before[1].tobytes()
        alloc.prefix_register(table, keys)
        reqs.append((table, toks, khist, vhist))
    shared = reqs[0][0][:187]
    assert all(t[:187] == shared for t, _, _, _ in reqs)
    assert all(alloc.refcount(b) == 4 for b in shared)

    # One decode token for every request.
    q = _draw(rng, (4, hq, d))
    kn, vn = _draw(rng, (4, hkv, d)), _draw(rng, (4, hkv, d))
    slots, bt, ctx = [], np.full((4, mb), -1, np.int32), []
    for r, (table, toks, khist, vhist) in enumerate(reqs):
        s, c = alloc.append(table, len(toks), 1)
        assert c == []
        slots += s
        bt[r, :len(table)] = table
        ctx.append(len(toks) + 1)
    out = pkv.attention_with_write(
        to_torch(q, "bf16"), to_torch(kn, "bf16"), to_torch(vn, "bf16"), kp, vp, i32(slots),
        i32(bt), i32(ctx), i32([0, 1, 2, 3, 4]), scale=scale, max_context_len=max(ctx),
        max_query_len=1)
    torch.cuda.synchronize()
    got = out_f64(out)
    for r, (table, toks, khist, vhist) in enumerate(reqs):
        kh = np.concatenate([khist, kn[r:r + 1]])
        vh = np.concatenate([vhist, vn[r:r + 1]])
        ref = O.attention_contiguous(O.to_f64(q[r:r + 1], "bf16"), O.to_f64(kh, "bf16"),
                                     O.to_f64(vh, "bf16"), scale, [len(toks)])
        tol = np.maximum(BF16_TOL, np.abs(ref) * 2.0 ** -8 + 2e-3)
        assert (np.abs(got[r:r + 1] - ref) <= tol).all(), f"decode request {r}"


@pytest.mark.parametrize("hq,hkv,d,qlens,ctxs", [
    (16, 8, 128, [40], [3032]),           # a prefix-cache hit: 12 key splits
    (32, 8, 64, [7, 1, 1], [2100, 900, 1500]),
    (8, 2, 64, [129, 3], [1500, 777]),
    (16, 8, 128, [2], [600]),
    (4, 4, 128, [17, 1, 33], [4096, 200, 2049]),
])
def test_split_chunks_match_oracle(hq, hkv, d, qlens, ctxs):
    """Chunks with too few tiles to fill the GPU split their key range over several
    workgroups and merge; results equal the oracle (unused pool slots hold NaN)."""
    from tests.gpu_util import DeviceBatch, tolerance
    from workloads import make_batch
    print(f"[case] split chunks hq={hq} hkv={hkv} d={d} q={qlens} ctx={ctxs}", flush=True)
    rng = np.random.Generator(np.random.PCG64(sum(ctxs) + d))
    nb = sum((c + 15) // 16 for c in ctxs) + 64
    b = make_batch(rng, name="split", dtype="bf16", num_q_heads=hq, num_kv_heads=hkv,
                   head_dim=d, num_blocks=nb, context_lens=ctxs, query_lens=qlens,
                   stale="nan")
    kp, vp, ref = O.step(b)
    got = out_f64(DeviceBatch(b).step())
    tol = tolerance(b, ref)
    assert np.isfinite(got).all()
    assert (np.abs(got - ref) <= tol).all(), float(np.abs(got - ref).max())
