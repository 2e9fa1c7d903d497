"""Torch-facing binding of libpagedkv: checks tensor shapes, dtypes and devices, then
passes raw device pointers and the current HIP stream to the C ABI.  Every step of the
computation runs in the library's HIP kernels; nothing here computes.
"""
from __future__ import annotations

import ctypes
from typing import NamedTuple

import torch

from . import _lib

BLOCK_SIZE = 16
_DTYPES = {torch.float32: _lib.PKV_F32, torch.bfloat16: _lib.PKV_BF16}


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported element type {t.dtype}; use float32 or bfloat16")


def _stream_handle(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _empty_on(stream, *args, **kw) -> torch.Tensor:
    """torch.empty allocated on the stream the library's kernels will use.  The
    caching allocator then hands the memory to no other stream's allocation before
    that stream's work is done (a temporary made on the current stream and dropped
    on return could be reused by the current stream while a side-stream kernel still
    writes it)."""
    if stream is None:
        return torch.empty(*args, **kw)
    with torch.cuda.stream(stream):
        return torch.empty(*args, **kw)


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _on_gpu(name: str, t: torch.Tensor, device) -> None:
    _require(t.is_cuda, f"{name} must be a GPU tensor")
    _require(t.device == device, f"{name} is on {t.device}, expected {device}")
    _require(t.is_contiguous(), f"{name} must be contiguous")


def kv_write(k_new: torch.Tensor, v_new: torch.Tensor, k_pool: torch.Tensor,
             v_pool: torch.Tensor, slot_mapping: torch.Tensor, stream=None) -> None:
    """Write new K/V rows [T, Hkv, D] into pools [num_blocks, Hkv, 16, D] at slots."""
    dev = k_pool.device
    for n, t in (("k_new", k_new), ("v_new", v_new), ("k_pool", k_pool), ("v_pool", v_pool),
                 ("slot_mapping", slot_mapping)):
        _on_gpu(n, t, dev)
    _require(k_pool.dim() == 4 and k_pool.shape == v_pool.shape, "pool shape mismatch")
    nb, hkv, bs, d = k_pool.shape
    _require(k_new.shape == v_new.shape and k_new.dim() == 3, "k_new/v_new shape mismatch")
    _require(tuple(k_new.shape[1:]) == (hkv, d), "new K/V heads or head_dim differ from pool")
    _require(k_new.dtype == k_pool.dtype == v_new.dtype == v_pool.dtype, "dtype mismatch")
    _require(slot_mapping.dtype == torch.int32 and slot_mapping.shape == (k_new.shape[0],),
             "slot_mapping must be int32 [num_tokens]")
    lib = _lib.load()
    st = lib.paged_kv_write(k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(),
                            v_pool.data_ptr(), slot_mapping.data_ptr(), k_new.shape[0], nb,
                            hkv, d, bs, _dtype_code(k_pool), _stream_handle(stream))
    _lib.check("paged_kv_write", st)


def workspace_size(num_seqs: int, total_q: int, num_q_heads: int, num_kv_heads: int,
                   head_dim: int, max_context_len: int, dtype: torch.dtype) -> int:
    return int(_lib.load().paged_attention_workspace_size(
        num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, max_context_len,
        _DTYPES[dtype]))


def attention(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
              block_tables: torch.Tensor, context_lens: torch.Tensor,
              query_start_loc: torch.Tensor, *, scale: float, max_context_len: int,
              max_query_len: int, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Varlen paged attention; returns `out` [total_q, Hq, D] (same dtype as q).

    `max_context_len` / `max_query_len` are host-side upper bounds of the device
    metadata.  `workspace` (uint8) must hold at least workspace_size(...) bytes; when
    omitted it is allocated here, like a default `out`, on `stream` (the current
    stream if None).
    """
    dev = q.device
    for n, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool),
                 ("block_tables", block_tables), ("context_lens", context_lens),
                 ("query_start_loc", query_start_loc)):
        _on_gpu(n, t, dev)
    _require(q.dim() == 3, "q must be [total_q, Hq, D]")
    total_q, hq, d = q.shape
    _require(k_pool.dim() == 4 and k_pool.shape == v_pool.shape, "pool shape mismatch")
    nb, hkv, bs, d2 = k_pool.shape
    _require(d2 == d, "head_dim of q and pools differ")
    _require(q.dtype == k_pool.dtype == v_pool.dtype, "dtype mismatch")
    _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2,
             "block_tables must be int32 [num_seqs, max_blocks_per_seq]")
    num_seqs, max_blocks = block_tables.shape
    _require(context_lens.dtype == torch.int32 and context_lens.shape == (num_seqs,),
             "context_lens must be int32 [num_seqs]")
    _require(query_start_loc.dtype == torch.int32 and
             query_start_loc.shape == (num_seqs + 1,),
             "query_start_loc must be int32 [num_seqs + 1]")
    if out is None:
        out = _empty_on(stream, q.shape, dtype=q.dtype, device=dev)
    else:
        _on_gpu("out", out, dev)
        _require(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    need = workspace_size(num_seqs, total_q, hq, hkv, d, max_context_len, q.dtype) \
        if num_seqs and total_q else 0
    if workspace is None:
        workspace = _empty_on(stream, max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _on_gpu("workspace", workspace, dev)
    lib = _lib.load()
    st = lib.paged_attention_varlen(
        out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), query_start_loc.data_ptr(),
        num_seqs, total_q, nb, max_blocks, max_context_len, max_query_len, hq, hkv, d, bs,
        float(scale), _dtype_code(q), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _lib.check("paged_attention_varlen", st)
    return out


def attention_with_write(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                         k_pool: torch.Tensor, v_pool: torch.Tensor,
                         slot_mapping: torch.Tensor, block_tables: torch.Tensor,
                         context_lens: torch.Tensor, query_start_loc: torch.Tensor, *,
                         scale: float, max_context_len: int, max_query_len: int,
                         out: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kv_write(k_new, v_new, pools, slot_mapping) then attention(...), in one call.

    Requires slot_mapping[t] to be the table slot of new row t's position (the usual
    scheduler layout); see paged_attention_varlen_with_write in include/pagedkv.h.
    """
    dev = q.device
    for n, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_pool", k_pool),
                 ("v_pool", v_pool), ("slot_mapping", slot_mapping),
                 ("block_tables", block_tables), ("context_lens", context_lens),
                 ("query_start_loc", query_start_loc)):
        _on_gpu(n, t, dev)
    _require(q.dim() == 3, "q must be [total_q, Hq, D]")
    total_q, hq, d = q.shape
    _require(k_pool.dim() == 4 and k_pool.shape == v_pool.shape, "pool shape mismatch")
    nb, hkv, bs, d2 = k_pool.shape
    _require(d2 == d, "head_dim of q and pools differ")
    _require(q.dtype == k_pool.dtype == v_pool.dtype == k_new.dtype == v_new.dtype,
             "dtype mismatch")
    _require(tuple(k_new.shape) == (total_q, hkv, d) and k_new.shape == v_new.shape,
             "k_new/v_new must be [total_q, Hkv, D]")
    _require(slot_mapping.dtype == torch.int32 and slot_mapping.shape == (total_q,),
             "slot_mapping must be int32 [total_q]")
    _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2,
             "block_tables must be int32 [num_seqs, max_blocks_per_seq]")
    num_seqs, max_blocks = block_tables.shape
    _require(context_lens.dtype == torch.int32 and context_lens.shape == (num_seqs,),
             "context_lens must be int32 [num_seqs]")
    _require(query_start_loc.dtype == torch.int32 and
             query_start_loc.shape == (num_seqs + 1,),
             "query_start_loc must be int32 [num_seqs + 1]")
    if out is None:
        out = _empty_on(stream, q.shape, dtype=q.dtype, device=dev)
    else:
        _on_gpu("out", out, dev)
        _require(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    need = workspace_size(num_seqs, total_q, hq, hkv, d, max_context_len, q.dtype) \
        if num_seqs and total_q else 0
    if workspace is None:
        workspace = _empty_on(stream, max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _on_gpu("workspace", workspace, dev)
    lib = _lib.load()
    st = lib.paged_attention_varlen_with_write(
        out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
        k_pool.data_ptr(), v_pool.data_ptr(), slot_mapping.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), query_start_loc.data_ptr(),
        num_seqs, total_q, nb, max_blocks, max_context_len, max_query_len, hq, hkv, d, bs,
        float(scale), _dtype_code(q), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _lib.check("paged_attention_varlen_with_write", st)
    return out


def shared_prefix_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                                 head_dim: int, max_context_len: int, shared_blocks: int,
                                 dtype: torch.dtype = torch.bfloat16) -> int:
    return int(_lib.load().paged_attention_shared_prefix_workspace_size(
        num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, shared_blocks,
        _DTYPES[dtype]))


def attention_shared_prefix(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                            block_tables: torch.Tensor, context_lens: torch.Tensor,
                            query_start_loc: torch.Tensor, *, shared_blocks: int,
                            scale: float, max_context_len: int,
                            k_new: torch.Tensor | None = None,
                            v_new: torch.Tensor | None = None,
                            slot_mapping: torch.Tensor | None = None,
                            out: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None,
                            stream=None) -> torch.Tensor:
    """Decode attention for a batch whose tables all start with the same
    `shared_blocks` blocks (paged_attention_varlen_shared_prefix): the shared keys are
    read once for all rows.  With k_new/v_new/slot_mapping it is the fused step (their
    slot write first, as in attention_with_write)."""
    dev = q.device
    for n, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool),
                 ("block_tables", block_tables), ("context_lens", context_lens),
                 ("query_start_loc", query_start_loc)):
        _on_gpu(n, t, dev)
    with_write = k_new is not None
    _require(with_write == (v_new is not None) == (slot_mapping is not None),
             "give k_new, v_new and slot_mapping together, or none of them")
    _require(q.dim() == 3, "q must be [total_q, Hq, D]")
    total_q, hq, d = q.shape
    _require(k_pool.dim() == 4 and k_pool.shape == v_pool.shape, "pool shape mismatch")
    nb, hkv, bs, d2 = k_pool.shape
    _require(d2 == d, "head_dim of q and pools differ")
    _require(q.dtype == k_pool.dtype == v_pool.dtype, "dtype mismatch")
    _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2,
             "block_tables must be int32 [num_seqs, max_blocks_per_seq]")
    num_seqs, max_blocks = block_tables.shape
    _require(context_lens.dtype == torch.int32 and context_lens.shape == (num_seqs,),
             "context_lens must be int32 [num_seqs]")
    _require(query_start_loc.dtype == torch.int32 and
             query_start_loc.shape == (num_seqs + 1,),
             "query_start_loc must be int32 [num_seqs + 1]")
    if with_write:
        for n, t in (("k_new", k_new), ("v_new", v_new), ("slot_mapping", slot_mapping)):
            _on_gpu(n, t, dev)
        _require(tuple(k_new.shape) == (total_q, hkv, d) and k_new.shape == v_new.shape and
                 k_new.dtype == v_new.dtype == q.dtype,
                 "k_new/v_new must be [total_q, Hkv, D] of q's dtype")
        _require(slot_mapping.dtype == torch.int32 and slot_mapping.shape == (total_q,),
                 "slot_mapping must be int32 [total_q]")
    if out is None:
        out = _empty_on(stream, q.shape, dtype=q.dtype, device=dev)
    else:
        _on_gpu("out", out, dev)
        _require(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    if workspace is None:
        need = shared_prefix_workspace_size(num_seqs, hq, hkv, d, max_context_len,
                                            shared_blocks, q.dtype) \
            if shared_blocks > 0 else \
            (workspace_size(num_seqs, total_q, hq, hkv, d, max_context_len, q.dtype)
             if num_seqs and total_q else 0)
        workspace = _empty_on(stream, max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _on_gpu("workspace", workspace, dev)
    ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    st = _lib.load().paged_attention_varlen_shared_prefix(
        out.data_ptr(), q.data_ptr(), ptr(k_new), ptr(v_new), k_pool.data_ptr(),
        v_pool.data_ptr(), ptr(slot_mapping), block_tables.data_ptr(), context_lens.data_ptr(),
        query_start_loc.data_ptr(), num_seqs, total_q, nb, max_blocks, max_context_len, 1,
        shared_blocks, hq, hkv, d, bs, float(scale), _dtype_code(q), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _lib.check("paged_attention_varlen_shared_prefix", st)
    return out


def validate_shared_prefix(block_tables, context_lens, query_start_loc,
                           shared_blocks: int) -> tuple[bool, int]:
    """Host check of the shared-prefix precondition (pkv_validate_shared_prefix)."""
    import numpy as np

    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    qsl = np.ascontiguousarray(np.asarray(query_start_loc, dtype=np.int32))
    bad = ctypes.c_int32(-1)
    st = _lib.load().pkv_validate_shared_prefix(
        bt.ctypes.data, cl.ctypes.data, qsl.ctypes.data, cl.shape[0],
        bt.shape[1] if bt.ndim == 2 else 0, shared_blocks, ctypes.byref(bad))
    return st == _lib.PKV_OK, bad.value


def attention_with_write_noalloc(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                 k_pool: torch.Tensor, v_pool: torch.Tensor,
                                 slot_mapping: torch.Tensor, block_tables: torch.Tensor,
                                 context_lens: torch.Tensor, query_start_loc: torch.Tensor,
                                 *, scale: float, max_context_len: int, max_query_len: int,
                                 out: torch.Tensor, stream=None) -> torch.Tensor:
    """attention_with_write without a workspace and with a caller-given `out`: nothing
    is allocated (paged_attention_varlen_with_write_noalloc; the library's per-GPU
    scratch holds the partials, so calls that overlap in time on one GPU race)."""
    dev = q.device
    for n, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_pool", k_pool),
                 ("v_pool", v_pool), ("slot_mapping", slot_mapping),
                 ("block_tables", block_tables), ("context_lens", context_lens),
                 ("query_start_loc", query_start_loc), ("out", out)):
        _on_gpu(n, t, dev)
    _require(q.dim() == 3, "q must be [total_q, Hq, D]")
    total_q, hq, d = q.shape
    _require(k_pool.dim() == 4 and k_pool.shape == v_pool.shape, "pool shape mismatch")
    nb, hkv, bs, d2 = k_pool.shape
    _require(d2 == d, "head_dim of q and pools differ")
    _require(q.dtype == k_pool.dtype == v_pool.dtype == k_new.dtype == v_new.dtype,
             "dtype mismatch")
    _require(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _require(tuple(k_new.shape) == (total_q, hkv, d) and k_new.shape == v_new.shape,
             "k_new/v_new must be [total_q, Hkv, D]")
    _require(slot_mapping.dtype == torch.int32 and slot_mapping.shape == (total_q,),
             "slot_mapping must be int32 [total_q]")
    _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2,
             "block_tables must be int32 [num_seqs, max_blocks_per_seq]")
    num_seqs, max_blocks = block_tables.shape
    _require(context_lens.dtype == torch.int32 and context_lens.shape == (num_seqs,),
             "context_lens must be int32 [num_seqs]")
    _require(query_start_loc.dtype == torch.int32 and
             query_start_loc.shape == (num_seqs + 1,),
             "query_start_loc must be int32 [num_seqs + 1]")
    st = _lib.load().paged_attention_varlen_with_write_noalloc(
        out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
        k_pool.data_ptr(), v_pool.data_ptr(), slot_mapping.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), query_start_loc.data_ptr(),
        num_seqs, total_q, nb, max_blocks, max_context_len, max_query_len, hq, hkv, d, bs,
        float(scale), _dtype_code(q), _stream_handle(stream))
    _lib.check("paged_attention_varlen_with_write_noalloc", st)
    return out


def validate_metadata(block_tables, context_lens, query_start_loc, slot_mapping,
                      num_blocks: int, fused: bool = False) -> tuple[bool, int]:
    """Host-side metadata check on CPU int32 arrays/tensors; (ok, bad_index).  With
    fused=True also the extra precondition of attention_with_write (each new row's
    slot is its position's table slot; pkv_validate_fused_metadata)."""
    import numpy as np

    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    qsl = np.ascontiguousarray(np.asarray(query_start_loc, dtype=np.int32))
    sm = None if slot_mapping is None else \
        np.ascontiguousarray(np.asarray(slot_mapping, dtype=np.int32))
    bad = ctypes.c_int32(-1)
    ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
    fn = _lib.load().pkv_validate_fused_metadata if fused else \
        _lib.load().pkv_validate_metadata
    st = fn(
        ptr(bt), ptr(cl), ptr(qsl), ptr(sm), cl.shape[0], int(qsl[-1]) if qsl.size else 0,
        num_blocks, bt.shape[1] if bt.ndim == 2 else 0, ctypes.byref(bad))
    return st == _lib.PKV_OK, bad.value


class BlockAllocator:
    """Host reference-counted allocator of physical blocks (pkv_allocator_* in the C
    ABI).  Tables are Python lists of block ids (a request's block_tables row)."""

    def __init__(self, num_blocks: int):
        self._lib = _lib.load()
        h = ctypes.c_void_p()
        _lib.check("pkv_allocator_create", self._lib.pkv_allocator_create(num_blocks,
                                                                          ctypes.byref(h)))
        self._h = h
        self.num_blocks = num_blocks

    def close(self) -> None:
        if self._h:
            self._lib.pkv_allocator_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown
            pass

    def num_free(self) -> int:
        return int(self._lib.pkv_allocator_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(self._lib.pkv_allocator_refcount(self._h, block))

    @staticmethod
    def _arr(table, extra: int = 0):
        import numpy as np

        a = np.zeros(len(table) + extra, dtype=np.int32)
        a[:len(table)] = table
        return a

    def fork(self, table) -> list:
        a = self._arr(table)
        _lib.check("pkv_allocator_fork",
                   self._lib.pkv_allocator_fork(self._h, a.ctypes.data, len(table)))
        return list(table)

    def release(self, table) -> None:
        a = self._arr(table)
        _lib.check("pkv_allocator_release",
                   self._lib.pkv_allocator_release(self._h, a.ctypes.data, len(table)))

    def append(self, table: list, context_len: int, num_new: int, max_blocks: int = 1 << 20):
        """Room for num_new tokens after context_len; `table` (list) is updated in
        place.  Returns (slots, copies) like the C call: slots of the new tokens and
        the (source, destination) pairs to copy first."""
        import numpy as np

        used = (context_len + 15) // 16
        end_blocks = (context_len + num_new + 15) // 16
        arr = self._arr(table[:used], max(end_blocks - used, 0))
        slots = np.zeros(max(num_new, 1), dtype=np.int32)
        copies = np.zeros(2, dtype=np.int32)
        ncopy = ctypes.c_int32(0)
        st = self._lib.pkv_allocator_append(self._h, arr.ctypes.data,
                                            min(max_blocks, len(arr)), context_len,
                                            num_new, slots.ctypes.data, copies.ctypes.data,
                                            1, ctypes.byref(ncopy))
        _lib.check("pkv_allocator_append", st)
        table[:] = [int(x) for x in arr[:end_blocks]]
        pairs = [(int(copies[0]), int(copies[1]))] if ncopy.value else []
        return [int(x) for x in slots[:num_new]], pairs


    def build_step(self, tables, num_computed, query_len, max_blocks: int):
        """The varlen batch of one planned step (pkv_build_step).  `tables` is either a
        list of per-request block lists or an int32 numpy array [num_requests,
        max_blocks] (the faster form: passed to the library as is); either is updated
        in place with the blocks the step needs.  Returns a StepBatch of host int32
        arrays; nothing changes on error."""
        import numpy as np

        as_array = isinstance(tables, np.ndarray)
        n = tables.shape[0] if as_array else len(tables)
        _require(len(num_computed) == n and len(query_len) == n, "one entry per request")
        if as_array:
            _require(tables.dtype == np.int32 and tables.ndim == 2 and
                     tables.shape[1] == max_blocks and tables.flags.c_contiguous,
                     "tables must be a C-contiguous int32 [num_requests, max_blocks] array")
            tab = tables
        else:
            tab = np.full((max(n, 1), max_blocks), -1, dtype=np.int32)
            for r, t in enumerate(tables):
                _require(len(t) <= max_blocks, f"table {r} longer than max_blocks")
                tab[r, :len(t)] = t
        nc = np.ascontiguousarray(num_computed, dtype=np.int32).reshape(-1)
        ql = np.ascontiguousarray(query_len, dtype=np.int32).reshape(-1)
        tokens = int(ql.sum()) if n else 0
        seq_request = np.empty(max(n, 1), dtype=np.int32)
        bt = np.empty((max(n, 1), max_blocks), dtype=np.int32)
        qsl = np.empty(n + 1, dtype=np.int32)
        ctx = np.empty(max(n, 1), dtype=np.int32)
        slots = np.empty(max(tokens, 1), dtype=np.int32)
        copies = np.empty((max(n, 1), 2), dtype=np.int32)
        ns, ncp = ctypes.c_int32(0), ctypes.c_int32(0)
        st = self._lib.pkv_build_step(self._h, n, tab.ctypes.data, max_blocks,
                                      nc.ctypes.data, ql.ctypes.data, seq_request.ctypes.data,
                                      bt.ctypes.data, qsl.ctypes.data, ctx.ctypes.data,
                                      slots.ctypes.data, tokens, copies.ctypes.data,
                                      ctypes.byref(ns), ctypes.byref(ncp))
        _lib.check("pkv_build_step", st)
        if not as_array:
            for r in range(n):
                if ql[r] > 0:
                    tables[r][:] = tab[r, :(int(nc[r]) + int(ql[r]) + 15) // 16].tolist()
        s = ns.value
        if n == 0:
            qsl[0] = 0
        return StepBatch(seq_request[:s], bt[:s], qsl[:s + 1], ctx[:s], slots[:tokens],
                         copies[:ncp.value])


    # ---- prefix cache ----
    def enable_prefix_cache(self) -> None:
        """Keep the contents of registered blocks after their last reference goes
        (pkv_allocator_enable_prefix_cache)."""
        _lib.check("pkv_allocator_enable_prefix_cache",
                   self._lib.pkv_allocator_enable_prefix_cache(self._h))

    def prefix_match(self, keys: list) -> list:
        """Blocks of the longest cached run of leading keys (each gains a reference)."""
        import numpy as np

        n = len(keys)
        kb = np.frombuffer(b"".join(keys), dtype=np.uint8) if n else np.zeros(1, np.uint8)
        table = np.zeros(max(n, 1), dtype=np.int32)
        hit = ctypes.c_int32(0)
        _lib.check("pkv_prefix_match", self._lib.pkv_prefix_match(
            self._h, kb.ctypes.data, n, table.ctypes.data, ctypes.byref(hit)))
        return [int(x) for x in table[:hit.value]]

    def prefix_register(self, table: list, keys: list) -> None:
        """Cache the full blocks table[i] under keys[i] (pkv_prefix_register)."""
        import numpy as np

        n = min(len(table), len(keys))
        if n == 0:
            return
        t = np.asarray(table[:n], dtype=np.int32)
        kb = np.frombuffer(b"".join(keys[:n]), dtype=np.uint8)
        _lib.check("pkv_prefix_register", self._lib.pkv_prefix_register(
            self._h, t.ctypes.data, kb.ctypes.data, n))

    def num_cached(self) -> int:
        return int(self._lib.pkv_prefix_num_cached(self._h))

    def num_evictable(self) -> int:
        return int(self._lib.pkv_prefix_num_evictable(self._h))

class StepBatch(NamedTuple):
    """Host int32 metadata of one engine step (pkv_build_step's outputs)."""
    seq_request: "np.ndarray"      # request index of each sequence
    block_tables: "np.ndarray"     # [num_seqs, max_blocks], -1 past the used blocks
    query_start_loc: "np.ndarray"  # [num_seqs + 1]
    context_lens: "np.ndarray"     # [num_seqs]
    slot_mapping: "np.ndarray"     # [total new tokens]
    copies: "np.ndarray"           # [num_copies, 2] (source, destination)


def swap_bytes(k_pool: torch.Tensor, n: int) -> int:
    """Bytes of the host image (and staging buffer) of n blocks of these pools."""
    nb, hkv, bs, d = k_pool.shape
    return int(_lib.load().paged_kv_swap_bytes(n, hkv, d, bs, _dtype_code(k_pool)))


def _swap_args(k_pool, v_pool, blocks, staging, host, n_bytes):
    dev = k_pool.device
    for nme, t in (("k_pool", k_pool), ("v_pool", v_pool), ("blocks", blocks),
                   ("staging", staging)):
        _on_gpu(nme, t, dev)
    _require(k_pool.dim() == 4 and k_pool.shape == v_pool.shape, "pool shape mismatch")
    _require(blocks.dtype == torch.int32 and blocks.dim() == 1, "blocks must be int32 [n]")
    _require(host.device.type == "cpu" and host.is_contiguous(), "host must be a CPU tensor")
    _require(staging.is_contiguous(), "staging must be contiguous")
    _require(host.numel() * host.element_size() >= n_bytes and
             staging.numel() * staging.element_size() >= n_bytes,
             "host and staging must hold swap_bytes(k_pool, n) bytes")


def swap_out(k_pool: torch.Tensor, v_pool: torch.Tensor, blocks: torch.Tensor,
             staging: torch.Tensor, host: torch.Tensor, stream=None) -> None:
    """Copy blocks (device int32 [n]) of both pools to `host` (pinned CPU tensor, K then
    V) through the device `staging` buffer (paged_kv_swap_out)."""
    n = blocks.shape[0]
    _swap_args(k_pool, v_pool, blocks, staging, host, swap_bytes(k_pool, n))
    nb, hkv, bs, d = k_pool.shape
    st = _lib.load().paged_kv_swap_out(k_pool.data_ptr(), v_pool.data_ptr(),
                                       blocks.data_ptr(), n, staging.data_ptr(),
                                       host.data_ptr(), nb, hkv, d, bs, _dtype_code(k_pool),
                                       _stream_handle(stream))
    _lib.check("paged_kv_swap_out", st)


def swap_in(k_pool: torch.Tensor, v_pool: torch.Tensor, blocks: torch.Tensor,
            staging: torch.Tensor, host: torch.Tensor, stream=None) -> None:
    """Write the host image back into blocks (device int32 [n]) of both pools
    (paged_kv_swap_in)."""
    n = blocks.shape[0]
    _swap_args(k_pool, v_pool, blocks, staging, host, swap_bytes(k_pool, n))
    nb, hkv, bs, d = k_pool.shape
    st = _lib.load().paged_kv_swap_in(k_pool.data_ptr(), v_pool.data_ptr(),
                                      blocks.data_ptr(), n, staging.data_ptr(),
                                      host.data_ptr(), nb, hkv, d, bs, _dtype_code(k_pool),
                                      _stream_handle(stream))
    _lib.check("paged_kv_swap_in", st)

def block_keys(tokens, extras: bytes = b"", parent: bytes | None = None) -> list:
    """32-byte keys of the full blocks of `tokens` (pkv_block_keys)."""
    import numpy as np

    t = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
    n = len(t) // BLOCK_SIZE
    out = np.zeros(max(n, 1) * 32, dtype=np.uint8)
    ex = np.frombuffer(extras, dtype=np.uint8) if extras else None
    pk = np.frombuffer(parent, dtype=np.uint8) if parent is not None else None
    _require(parent is None or len(parent) == 32, "parent key must be 32 bytes")
    got = ctypes.c_int32(0)
    _lib.check("pkv_block_keys", _lib.load().pkv_block_keys(
        t.ctypes.data if len(t) else None, len(t),
        ex.ctypes.data if ex is not None else None, len(extras),
        pk.ctypes.data if pk is not None else None, out.ctypes.data, n, ctypes.byref(got)))
    raw = out.tobytes()
    return [raw[32 * i:32 * i + 32] for i in range(got.value)]

def plan_step(prompt_len, num_computed, token_budget: int) -> list:
    """Tokens each request runs this step under `token_budget` (pkv_plan_step): decode
    tokens first, then prompt slices in request order."""
    import numpy as np

    pl = np.asarray(prompt_len, dtype=np.int32).reshape(-1)
    nc = np.asarray(num_computed, dtype=np.int32).reshape(-1)
    _require(pl.shape == nc.shape, "prompt_len and num_computed differ in length")
    ql = np.zeros(max(len(pl), 1), dtype=np.int32)
    st = _lib.load().pkv_plan_step(len(pl), pl.ctypes.data, nc.ctypes.data, token_budget,
                                   ql.ctypes.data)
    _lib.check("pkv_plan_step", st)
    return [int(x) for x in ql[:len(pl)]]


def copy_blocks(k_pool: torch.Tensor, v_pool: torch.Tensor, copies: torch.Tensor,
                stream=None) -> None:
    """Copy whole blocks in both pools: copies is an int32 [n, 2] (source, destination)
    device tensor (paged_kv_copy_blocks)."""
    dev = k_pool.device
    for n, t in (("k_pool", k_pool), ("v_pool", v_pool), ("copies", copies)):
        _on_gpu(n, t, dev)
    _require(k_pool.dim() == 4 and k_pool.shape == v_pool.shape, "pool shape mismatch")
    _require(copies.dtype == torch.int32 and copies.dim() == 2 and copies.shape[1] == 2,
             "copies must be int32 [n, 2]")
    nb, hkv, bs, d = k_pool.shape
    st = _lib.load().paged_kv_copy_blocks(k_pool.data_ptr(), v_pool.data_ptr(),
                                          copies.data_ptr(), copies.shape[0], nb, hkv, d,
                                          bs, _dtype_code(k_pool), _stream_handle(stream))
    _lib.check("paged_kv_copy_blocks", st)


def read_probe(base: torch.Tensor, tiles: torch.Tensor, tile_bytes: int, sink: torch.Tensor,
               grid: int, stream=None) -> None:
    """Measuring aid (pkv_read_probe): read the `tile_bytes`-byte tiles of `base` named
    by the int32 device tensor `tiles`; `sink` is a uint8/int32 device buffer of at
    least grid * 16 bytes (one word per wave)."""
    dev = base.device
    for n, t in (("base", base), ("tiles", tiles), ("sink", sink)):
        _on_gpu(n, t, dev)
    _require(tiles.dtype == torch.int32 and tiles.dim() == 1 and tiles.is_contiguous(),
             "tiles must be a contiguous int32 vector")
    _require(base.is_contiguous(), "base must be contiguous")
    _require(sink.numel() * sink.element_size() >= grid * 16, "sink too small")
    st = _lib.load().pkv_read_probe(base.data_ptr(), base.numel() * base.element_size(),
                                    tiles.data_ptr(), tiles.numel(), tile_bytes,
                                    sink.data_ptr(), grid, _stream_handle(stream))
    _lib.check("pkv_read_probe", st)
