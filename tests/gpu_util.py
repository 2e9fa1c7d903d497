"""Helpers for the GPU parity tests: move a seeded `PagedBatch` to the device, run the
HIP path through the binding, and bring results back as raw numpy arrays."""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_290_amd as pkv
import oracle.pagedkv_oracle as O

BF16_TOL = 1e-2
F32_TOL = 1e-5


def to_torch(raw: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(raw, dtype=np.float32))
    return t.to(device)


def to_raw(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class DeviceBatch:
    """Device copies of one batch plus the call of one engine step on them."""

    def __init__(self, b, device="cuda"):
        self.b = b
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(device)  # noqa
        self.k_pool = to_torch(b.k_pool, b.dtype, device)
        self.v_pool = to_torch(b.v_pool, b.dtype, device)
        self.q = to_torch(b.q, b.dtype, device)
        self.k_new = to_torch(b.k_new, b.dtype, device)
        self.v_new = to_torch(b.v_new, b.dtype, device)
        self.block_tables = i32(b.block_tables)
        self.context_lens = i32(b.context_lens)
        self.query_start_loc = i32(b.query_start_loc)
        self.slot_mapping = i32(b.slot_mapping)

    def write(self):
        pkv.kv_write(self.k_new, self.v_new, self.k_pool, self.v_pool, self.slot_mapping)

    def attend(self, out=None):
        b = self.b
        return pkv.attention(self.q, self.k_pool, self.v_pool, self.block_tables,
                             self.context_lens, self.query_start_loc, scale=b.scale,
                             max_context_len=b.max_context_len,
                             max_query_len=b.max_query_len, out=out)

    def step(self):
        self.write()
        out = self.attend()
        torch.cuda.synchronize()
        return out

    def step_fused(self, out=None):
        """The same step through paged_attention_varlen_with_write (one call)."""
        b = self.b
        out = pkv.attention_with_write(self.q, self.k_new, self.v_new, self.k_pool,
                                       self.v_pool, self.slot_mapping, self.block_tables,
                                       self.context_lens, self.query_start_loc,
                                       scale=b.scale, max_context_len=b.max_context_len,
                                       max_query_len=b.max_query_len, out=out)
        torch.cuda.synchronize()
        return out


def out_f64(out: torch.Tensor) -> np.ndarray:
    return O.to_f64(to_raw(out), "bf16" if out.dtype == torch.bfloat16 else "f32")


def oracle_rows(b, k_pool, v_pool, rows) -> np.ndarray:
    """Oracle output for selected global query rows only: [len(rows), Hq, D] f64."""
    qsl = b.query_start_loc
    res = np.zeros((len(rows), b.num_q_heads, b.head_dim))
    for n, r in enumerate(rows):
        s = int(np.searchsorted(qsl, r, side="right") - 1)
        a, e = int(qsl[s]), int(qsl[s + 1])
        ctx = int(b.context_lens[s])
        pos = ctx - (e - a) + (r - a)
        K = O.to_f64(O.gather(k_pool, b.block_tables[s], pos + 1), b.dtype)
        V = O.to_f64(O.gather(v_pool, b.block_tables[s], pos + 1), b.dtype)
        res[n] = O.attention_contiguous(O.to_f64(b.q[r:r + 1], b.dtype), K, V, b.scale,
                                        [pos])[0]
    return res


def tolerance(b, ref: np.ndarray) -> np.ndarray:
    """Max-abs bound per element: 1e-5 for fp32; 1e-2 for bf16, widened by the bf16
    output rounding (half an ulp, at most 2^-8 |ref|) where that exceeds it."""
    if b.dtype == "f32":
        return np.full(ref.shape, F32_TOL)
    return np.maximum(BF16_TOL, np.abs(ref) * 2.0 ** -8 + 2e-3)
