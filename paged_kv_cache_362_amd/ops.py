"""Python binding of libpagedattn.so on torch tensors (argument marshalling only).

torch supplies device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels. There is no fallback: when the
library is missing or the tensors are not on a GPU, these functions raise.
"""

from __future__ import annotations

import ctypes

import torch

from ._lib import lib, status_str

DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

PA_OK = 0
STATUS = {0: "PA_OK", 1: "PA_ERR_NULL_POINTER", 2: "PA_ERR_BAD_SHAPE", 3: "PA_ERR_UNSUPPORTED",
          4: "PA_ERR_WORKSPACE_TOO_SMALL", 5: "PA_ERR_HIP", 6: "PA_ERR_BAD_INDEX",
          7: "PA_ERR_BAD_POINTER", 8: "PA_ERR_SCRATCH_TOO_SMALL"}


class PagedAttentionError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({status_str(code)})")
        self.code = code


def _check(fn: str, code: int) -> None:
    if code != PA_OK:
        raise PagedAttentionError(fn, code)


def _dev_ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _addressable(t: torch.Tensor) -> bool:
    """On the GPU, or pinned host memory the GPU can read and write."""
    return t.is_cuda or t.is_pinned()


def _on_gpu(*ts: torch.Tensor) -> None:
    dev = ts[0].device
    for t in ts:
        _require(t.is_cuda, "tensors must live on a GPU")
        _require(t.device == dev, "tensors must live on one GPU")
        _require(t.is_contiguous(), "tensors must be contiguous")


def dtype_code(dtype: torch.dtype) -> int:
    if dtype not in DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dtype}")
    return DTYPE_CODE[dtype]


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, slot_mapping: torch.Tensor) -> None:
    """Write key/value [T, Hkv, D] into the pools [N, Hkv, B, D] at slot_mapping [T]."""
    _on_gpu(key, value, k_cache, v_cache, slot_mapping)
    _require(key.dim() == 3 and value.shape == key.shape, "key/value must be [T, Hkv, D]")
    _require(k_cache.dim() == 4 and v_cache.shape == k_cache.shape, "pools must be [N, Hkv, B, D]")
    _require(key.dtype == value.dtype == k_cache.dtype == v_cache.dtype, "one dtype for all")
    _require(slot_mapping.dtype == torch.int32 and slot_mapping.shape == (key.shape[0],),
             "slot_mapping must be int32 [T]")
    n, hkv, bs, d = k_cache.shape
    _require(key.shape[1:] == (hkv, d), "key heads/dim must match the pools")
    code = lib().pa_reshape_and_cache(
        _dev_ptr(key), _dev_ptr(value), _dev_ptr(k_cache), _dev_ptr(v_cache),
        _dev_ptr(slot_mapping), key.shape[0], hkv, d, bs, n, dtype_code(key.dtype),
        _stream(key))
    _check("pa_reshape_and_cache", code)


def workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                   max_context_len: int, dtype: torch.dtype, partition: int = 0) -> int:
    """Bytes of decode scratch; ``partition`` 0 = balanced form, else fixed partitions."""
    size = lib().pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                          max_context_len, partition, dtype_code(dtype))
    _require(size != ctypes.c_size_t(-1).value, "invalid workspace request")
    return size


def new_workspace(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                  max_context_len: int, dtype: torch.dtype, device, partition: int = 0
                  ) -> torch.Tensor:
    """A zero-filled workspace (the library keeps its counters zero afterwards)."""
    size = workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                          dtype, partition)
    return torch.zeros(max(size, 16), dtype=torch.uint8, device=device)


def _decode_args(q, k_cache, v_cache, block_tables, context_lens, max_context_len, out,
                 workspace, partition):
    _on_gpu(q, k_cache, v_cache, block_tables, context_lens)
    _require(q.dim() == 3, "q must be [S, Hq, D]")
    _require(k_cache.dim() == 4 and v_cache.shape == k_cache.shape, "pools must be [N, Hkv, B, D]")
    _require(q.dtype == k_cache.dtype == v_cache.dtype, "q and the pools share one dtype")
    _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2,
             "block_tables must be int32 [S, M]")
    _require(context_lens.dtype == torch.int32 and context_lens.shape == (q.shape[0],),
             "context_lens must be int32 [S]")
    s, hq, d = q.shape
    _, hkv, _, d2 = k_cache.shape
    _require(d == d2 and block_tables.shape[0] == s, "inconsistent shapes")
    if out is None:
        out = torch.empty_like(q)
    else:
        _on_gpu(out)
        _require(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    if workspace is None:
        workspace = new_workspace(s, hq, hkv, d, max_context_len, q.dtype, q.device, partition)
    else:
        _on_gpu(workspace)
    return out, workspace


def _launch_decode(fn_name, q, k_cache, v_cache, block_tables, context_lens, scale,
                   max_context_len, out, workspace, partition):
    s, hq, d = q.shape
    n, hkv, bs, _ = k_cache.shape
    fn = getattr(lib(), fn_name)
    code = fn(_dev_ptr(out), _dev_ptr(q), _dev_ptr(k_cache), _dev_ptr(v_cache),
              _dev_ptr(block_tables), _dev_ptr(context_lens), float(scale), s, hq, hkv, d, bs, n,
              block_tables.shape[1], int(max_context_len), int(partition), dtype_code(q.dtype),
              _dev_ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q))
    _check(fn_name, code)


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
           max_context_len: int, out: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None, partition: int = 0) -> torch.Tensor:
    """Paged decode attention; returns out [S, Hq, D] in q's dtype.

    ``max_context_len`` is the host-side maximum of ``context_lens``.
    ``partition`` 0 is the balanced single-launch form; a positive multiple of
    16 selects fixed partitions of that many tokens. ``workspace`` (uint8, at
    least ``workspace_size(...)`` bytes, zero-filled before its first use) is
    allocated here when not given.
    """
    out, workspace = _decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                  max_context_len, out, workspace, partition)
    _launch_decode("pa_decode", q, k_cache, v_cache, block_tables, context_lens, scale,
                   max_context_len, out, workspace, partition)
    return out


def decode_step(q: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                k_cache: torch.Tensor, v_cache: torch.Tensor, slot_mapping: torch.Tensor,
                block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                max_context_len: int, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step in one launch: write key/value [S, Hkv, D] at slot_mapping
    [S] (each the last attended position of its sequence, or a slot no sequence
    attends), then paged attention."""
    out, workspace = _decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                  max_context_len, out, workspace, 0)
    _on_gpu(key, value, slot_mapping)
    _require(key.shape == value.shape == (q.shape[0], k_cache.shape[1], q.shape[2]),
             "key/value must be [S, Hkv, D]")
    _require(key.dtype == value.dtype == q.dtype, "key/value share q's dtype")
    _require(slot_mapping.dtype == torch.int32 and slot_mapping.shape == (q.shape[0],),
             "slot_mapping must be int32 [S]")
    s, hq, d = q.shape
    n, hkv, bs, _ = k_cache.shape
    code = lib().pa_decode_step(
        _dev_ptr(out), _dev_ptr(q), _dev_ptr(key), _dev_ptr(value), _dev_ptr(k_cache),
        _dev_ptr(v_cache), _dev_ptr(slot_mapping), _dev_ptr(block_tables),
        _dev_ptr(context_lens), float(scale), s, hq, hkv, d, bs, n, block_tables.shape[1],
        int(max_context_len), dtype_code(q.dtype), _dev_ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q))
    _check("pa_decode_step", code)
    return out


def decode_step_noalloc(q: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                        k_cache: torch.Tensor, v_cache: torch.Tensor,
                        slot_mapping: torch.Tensor, block_tables: torch.Tensor,
                        context_lens: torch.Tensor, scale: float, max_context_len: int,
                        out: torch.Tensor) -> torch.Tensor:
    """decode_step with the library's static scratch (``pa_decode_step_noalloc``):
    nothing is allocated, so ``out`` must be given. Calls that overlap on one
    GPU share that scratch and must be ordered on one stream."""
    _on_gpu(q, k_cache, v_cache, block_tables, context_lens, out, key, value, slot_mapping)
    _require(q.dim() == 3 and out.shape == q.shape and out.dtype == q.dtype,
             "q [S, Hq, D] and out of the same shape and dtype")
    _require(k_cache.dim() == 4 and v_cache.shape == k_cache.shape, "pools must be [N, Hkv, B, D]")
    _require(q.dtype == k_cache.dtype == v_cache.dtype == key.dtype == value.dtype,
             "one dtype for q, key, value and the pools")
    _require(key.shape == value.shape == (q.shape[0], k_cache.shape[1], q.shape[2]),
             "key/value must be [S, Hkv, D]")
    for t, name in ((slot_mapping, "slot_mapping"), (context_lens, "context_lens")):
        _require(t.dtype == torch.int32 and t.shape == (q.shape[0],), f"{name} must be int32 [S]")
    _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and
             block_tables.shape[0] == q.shape[0], "block_tables must be int32 [S, M]")
    s, hq, d = q.shape
    n, hkv, bs, _ = k_cache.shape
    code = lib().pa_decode_step_noalloc(
        _dev_ptr(out), _dev_ptr(q), _dev_ptr(key), _dev_ptr(value), _dev_ptr(k_cache),
        _dev_ptr(v_cache), _dev_ptr(slot_mapping), _dev_ptr(block_tables),
        _dev_ptr(context_lens), float(scale), s, hq, hkv, d, bs, n, block_tables.shape[1],
        int(max_context_len), dtype_code(q.dtype), _stream(q))
    _check("pa_decode_step_noalloc", code)
    return out


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor,
                block_mapping: torch.Tensor) -> None:
    """Copy-on-write: for each row (src, dst) of block_mapping int32 [P, 2],
    block dst of both pools becomes a copy of block src."""
    _on_gpu(k_cache, v_cache, block_mapping)
    _require(k_cache.dim() == 4 and v_cache.shape == k_cache.shape, "pools must be [N, Hkv, B, D]")
    _require(k_cache.dtype == v_cache.dtype, "one dtype for both pools")
    _require(block_mapping.dtype == torch.int32 and block_mapping.dim() == 2 and
             block_mapping.shape[1] == 2, "block_mapping must be int32 [P, 2]")
    n, hkv, bs, d = k_cache.shape
    code = lib().pa_copy_blocks(_dev_ptr(k_cache), _dev_ptr(v_cache), _dev_ptr(block_mapping),
                                block_mapping.shape[0], hkv, d, bs, n,
                                dtype_code(k_cache.dtype), _stream(k_cache))
    _check("pa_copy_blocks", code)


def swap_blocks(src_k: torch.Tensor, src_v: torch.Tensor, dst_k: torch.Tensor,
                dst_v: torch.Tensor, block_mapping: torch.Tensor) -> None:
    """Swap-out / swap-in: for each row (src, dst) of block_mapping int32 [P, 2]
    (on the GPU), block dst of (dst_k, dst_v) becomes a copy of block src of
    (src_k, src_v). Pools may live on the GPU or in pinned host memory; the
    copy runs on the current stream of the GPU holding block_mapping."""
    for t in (src_k, src_v, dst_k, dst_v):
        _require(_addressable(t), "pools must be on the GPU or in pinned host memory")
        _require(t.is_contiguous(), "pools must be contiguous")
    _require(block_mapping.is_cuda and block_mapping.dtype == torch.int32 and
             block_mapping.dim() == 2 and block_mapping.shape[1] == 2 and
             block_mapping.is_contiguous(), "block_mapping must be int32 [P, 2] on the GPU")
    _require(src_k.shape == src_v.shape and dst_k.shape == dst_v.shape and
             src_k.shape[1:] == dst_k.shape[1:] and src_k.dim() == 4,
             "pools must be [N, Hkv, B, D] with matching block shapes")
    _require(src_k.dtype == src_v.dtype == dst_k.dtype == dst_v.dtype, "one dtype")
    _, hkv, bs, d = src_k.shape
    code = lib().pa_swap_blocks(_dev_ptr(src_k), _dev_ptr(src_v), _dev_ptr(dst_k),
                                _dev_ptr(dst_v), _dev_ptr(block_mapping),
                                block_mapping.shape[0], hkv, d, bs, src_k.shape[0],
                                dst_k.shape[0], dtype_code(src_k.dtype), _stream(block_mapping))
    _check("pa_swap_blocks", code)


def prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
            block_tables: torch.Tensor, context_lens: torch.Tensor,
            query_start_loc: torch.Tensor, scale: float, max_query_len: int,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """Chunked-prefill paged attention (``pa_prefill``): q [T, Hq, D] packs the
    chunks of all sequences (sequence s owns tokens query_start_loc[s] ..
    query_start_loc[s+1]-1, the last tokens of its context_lens[s] cached
    ones); each token attends causally to its sequence's cache."""
    _on_gpu(q, k_cache, v_cache, block_tables, context_lens, query_start_loc)
    _require(q.dim() == 3 and k_cache.dim() == 4 and k_cache.shape == v_cache.shape,
             "q must be [T, Hq, D] and the pools [N, Hkv, B, D]")
    for t in (q, k_cache, v_cache, block_tables, context_lens, query_start_loc):
        _require(t.is_contiguous(), "all tensors must be contiguous")
    _require(q.dtype == k_cache.dtype == v_cache.dtype, "q and the pools share one dtype")
    for t in (block_tables, context_lens, query_start_loc):
        _require(t.dtype == torch.int32, "tables, lengths and query_start_loc are int32")
    s = context_lens.shape[0]
    _require(query_start_loc.shape == (s + 1,) and block_tables.dim() == 2 and
             block_tables.shape[0] == s, "query_start_loc [S+1], block_tables [S, M]")
    n, hkv, bs, d = k_cache.shape
    if out is None:
        out = torch.empty_like(q)
    _require(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous(),
             "out must match q")
    code = lib().pa_prefill(
        _dev_ptr(out), _dev_ptr(q), _dev_ptr(k_cache), _dev_ptr(v_cache),
        _dev_ptr(block_tables), _dev_ptr(context_lens), _dev_ptr(query_start_loc), float(scale),
        s, q.shape[0], q.shape[1], hkv, d, bs, n, block_tables.shape[1], int(max_query_len),
        dtype_code(q.dtype), _stream(q))
    _check("pa_prefill", code)
    return out
