"""Python binding of the paged GQA attention C ABI (include/paged_attn.h).

Argument marshalling only: every function here reads shapes and device
pointers off torch tensors and calls the function of the same name in
`libpaged_attn.so`.  All computation happens in the library's HIP kernels;
nothing here computes attention, and there is no CPU or PyTorch fallback --
a missing library raises.  PyTorch supplies device memory and streams.

Tensors: q / out bf16 [num_seqs, H_q, D] (decode) or [total_q, H_q, D]
(prefill); k_cache / v_cache bf16 [num_blocks, H_kv, block_size, D] (or uint8
E4M3 codes with fp32 scales [num_blocks, H_kv, block_size] for the FP8 cache);
block_tables int32 [num_seqs, max_blocks_per_seq]; seq_lens int32 [num_seqs];
cu_seqlens int32 [num_seqs + 1]; partials fp32.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import List, Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libpaged_attn.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "paged_attn.h")

PA_OK = 0
PA_ERR_NULL_POINTER = 1
PA_ERR_BAD_SHAPE = 2
PA_ERR_UNSUPPORTED = 3
PA_ERR_LAUNCH = 4
PA_ERR_ALIGNMENT = 5
PA_ERR_BAD_VALUE = 6
PA_ERR_SCRATCH_LIMIT = 7


class PagedAttnError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


_vp = ctypes.c_void_p
_i = ctypes.c_int
_lib: Optional[ctypes.CDLL] = None


def library() -> ctypes.CDLL:
    """Load libpaged_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is not built; run `python -m paged_kv_cache_34_amd.build`")
        lib = ctypes.CDLL(LIBRARY)
        lib.paged_attn_decode.argtypes = [_vp] * 5 + [_i] * 7 + [ctypes.c_float, _i] + [_vp] * 4 + [_i, _vp]
        lib.paged_attn_decode_fused.argtypes = [_vp] * 5 + [_i] * 7 + [ctypes.c_float, _i] + [_vp] * 4 + [_i, _vp, _vp]
        lib.paged_attn_decode_fused_noalloc.argtypes = [_vp] * 5 + [_i] * 7 + [ctypes.c_float, _i, _vp, _vp]
        lib.paged_attn_decode_reduce.argtypes = [_vp] * 4 + [_i] * 5 + [_vp, _vp]
        lib.paged_attn_decode_fp8.argtypes = [_vp] * 7 + [_i] * 7 + [ctypes.c_float, _i] + [_vp] * 4 + [_i, _vp]
        lib.paged_attn_kv_append.argtypes = [_vp] * 5 + [_i] * 8 + [_vp] * 3
        lib.paged_attn_kv_append_fp8.argtypes = [_vp] * 5 + [_i] * 8 + [_vp] * 5
        lib.paged_attn_decode_xpacked.argtypes = lib.paged_attn_decode.argtypes
        lib.paged_attn_kv_append_xpacked.argtypes = lib.paged_attn_kv_append.argtypes
        lib.paged_attn_decode_tokens.argtypes = [_vp] * 5 + [_i] * 6 + [ctypes.c_float, _i] + [_vp] * 4 + [_i, _vp]
        lib.paged_attn_decode_reduce_indptr.argtypes = lib.paged_attn_decode_reduce.argtypes
        lib.paged_attn_prefill_ragged.argtypes = [_vp] * 6 + [_i] * 9 + [ctypes.c_float, _vp, _vp]
        lib.paged_attn_prefill_ragged_split.argtypes = ([_vp] * 6 + [_i] * 9 + [ctypes.c_float, _i, _vp,
                                                          ctypes.c_longlong, _vp, _vp])
        lib.paged_attn_prefill_chunk_size.argtypes = [_i] * 6
        lib.paged_attn_prefill_workspace_size.argtypes = [_i] * 6
        lib.paged_attn_prefill_workspace_size.restype = ctypes.c_longlong
        lib.paged_attn_num_partitions.argtypes = [_i, _i, _i]
        lib.paged_attn_choose_partition_size.argtypes = [_i, _i, _i, ctypes.c_long]
        lib.paged_attn_prefill_tile_map.argtypes = [_vp, _i, _i, _vp, _vp, _i]
        lib.paged_attn_read_probe.argtypes = [_vp, ctypes.c_longlong, _vp, _i, _vp]
        lib.paged_attn_gather_probe.argtypes = [_vp] * 4 + [_i] * 6 + [_vp, _i, _vp]
        lib.paged_attn_status_string.argtypes = [_i]
        lib.paged_attn_status_string.restype = ctypes.c_char_p
        for fn in ("paged_attn_decode", "paged_attn_decode_fused", "paged_attn_decode_fused_noalloc",
                   "paged_attn_decode_reduce",
                   "paged_attn_decode_fp8", "paged_attn_kv_append", "paged_attn_kv_append_fp8",
                   "paged_attn_decode_xpacked", "paged_attn_kv_append_xpacked",
                   "paged_attn_decode_tokens", "paged_attn_decode_reduce_indptr",
                   "paged_attn_prefill_ragged", "paged_attn_prefill_ragged_split",
                   "paged_attn_prefill_chunk_size",
                   "paged_attn_num_partitions", "paged_attn_choose_partition_size",
                   "paged_attn_prefill_tile_map", "paged_attn_read_probe", "paged_attn_gather_probe"):
            getattr(lib, fn).restype = _i
        _lib = lib
    return _lib


def declared_functions() -> List[str]:
    """Names of the functions include/paged_attn.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(paged_attn_\w+)\s*\(", text)))


def status_string(status: int) -> str:
    return library().paged_attn_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != PA_OK:
        raise PagedAttnError(fn, status)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream) if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _want(t, dtype, name):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(t, shape, name, fn):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{fn}: {name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_decode_buffers(fn, q, seq_lens, rows, out, partition_size, max_logits, exp_sums,
                          tmp_out, max_num_partitions, counters=None, num_kv_heads=0):
    """The library trusts its buffers to be as large as its size arguments
    say; check every tensor against them before the call (a short buffer
    would be read or written out of bounds on the device)."""
    num_seqs, hq, d = q.shape
    if seq_lens is not None and seq_lens.numel() != num_seqs:
        raise ValueError(f"{fn}: seq_lens must have {num_seqs} entries, got {seq_lens.numel()}")
    if rows is not None and rows.shape[0] != num_seqs:
        raise ValueError(f"{fn}: block_tables must have {num_seqs} rows, got {rows.shape[0]}")
    _shape(out, (num_seqs, hq, d), "out", fn)
    if partition_size > 0:
        if max_logits is None or exp_sums is None or tmp_out is None:
            raise ValueError(f"{fn}: split-KV (partition_size > 0) needs max_logits, exp_sums and tmp_out")
        np_ = int(max_num_partitions)
        _shape(max_logits, (num_seqs, hq, np_), "max_logits", fn)
        _shape(exp_sums, (num_seqs, hq, np_), "exp_sums", fn)
        _shape(tmp_out, (num_seqs, hq, np_, d), "tmp_out", fn)
    if counters is not None and counters.numel() < num_seqs * num_kv_heads:
        raise ValueError(f"{fn}: counters must hold num_seqs * num_kv_heads = {num_seqs * num_kv_heads} "
                         f"entries, got {counters.numel()}")


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def paged_attn_decode(q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                      partition_size: int = 0, out=None, max_logits=None, exp_sums=None,
                      tmp_out=None, max_num_partitions: Optional[int] = None, stream=None) -> None:
    """Decode: writes `out` (partition_size == 0) or the fp32 partials (> 0)."""
    import torch
    _want(q, torch.bfloat16, "q")
    _want(k_cache, torch.bfloat16, "k_cache")
    _want(v_cache, torch.bfloat16, "v_cache")
    _want(block_tables, torch.int32, "block_tables")
    _want(seq_lens, torch.int32, "seq_lens")
    _want(out, torch.bfloat16, "out")
    for name, t in (("max_logits", max_logits), ("exp_sums", exp_sums), ("tmp_out", tmp_out)):
        _want(t, torch.float32, name)
    num_seqs, hq, d = q.shape
    num_blocks, hkv, bs, _ = k_cache.shape
    _shape(v_cache, k_cache.shape, "v_cache", "paged_attn_decode")
    if max_num_partitions is None:
        max_num_partitions = tmp_out.shape[2] if tmp_out is not None else 1
    _check_decode_buffers("paged_attn_decode", q, seq_lens, block_tables, out, partition_size,
                          max_logits, exp_sums, tmp_out, max_num_partitions)
    st = library().paged_attn_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens), num_seqs, hq,
        hkv, d, bs, num_blocks, block_tables.shape[1], float(scale), int(partition_size),
        _ptr(out), _ptr(max_logits), _ptr(exp_sums), _ptr(tmp_out), int(max_num_partitions),
        _stream(stream))
    _check("paged_attn_decode", st)


def paged_attn_decode_fused(q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                            partition_size: int, out, max_logits, exp_sums, tmp_out, counters,
                            stream=None) -> None:
    """Split-KV decode with the merge fused in: writes `out`; partials are workspace;
    `counters` int32 [num_seqs * num_kv_heads] must be zero and is left zero."""
    import torch
    _want(q, torch.bfloat16, "q")
    _want(k_cache, torch.bfloat16, "k_cache")
    _want(v_cache, torch.bfloat16, "v_cache")
    _want(block_tables, torch.int32, "block_tables")
    _want(seq_lens, torch.int32, "seq_lens")
    _want(out, torch.bfloat16, "out")
    _want(counters, torch.int32, "counters")
    for name, t in (("max_logits", max_logits), ("exp_sums", exp_sums), ("tmp_out", tmp_out)):
        _want(t, torch.float32, name)
    num_seqs, hq, d = q.shape
    num_blocks, hkv, bs, _ = k_cache.shape
    _shape(v_cache, k_cache.shape, "v_cache", "paged_attn_decode_fused")
    if tmp_out is None or tmp_out.dim() != 4:
        raise ValueError("paged_attn_decode_fused: tmp_out must be [num_seqs, H_q, max_num_partitions, D]")
    _check_decode_buffers("paged_attn_decode_fused", q, seq_lens, block_tables, out, partition_size,
                          max_logits, exp_sums, tmp_out, tmp_out.shape[2], counters, hkv)
    st = library().paged_attn_decode_fused(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens), num_seqs, hq,
        hkv, d, bs, num_blocks, block_tables.shape[1], float(scale), int(partition_size),
        _ptr(out), _ptr(max_logits), _ptr(exp_sums), _ptr(tmp_out), tmp_out.shape[2],
        _ptr(counters), _stream(stream))
    _check("paged_attn_decode_fused", st)


def paged_attn_decode_fused_noalloc(q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                                    partition_size: int, out, stream=None) -> None:
    """paged_attn_decode_fused with the library's fixed device scratch as its
    workspace: allocates nothing (calls that overlap on one GPU race)."""
    import torch
    _want(q, torch.bfloat16, "q")
    _want(k_cache, torch.bfloat16, "k_cache")
    _want(v_cache, torch.bfloat16, "v_cache")
    _want(block_tables, torch.int32, "block_tables")
    _want(seq_lens, torch.int32, "seq_lens")
    _want(out, torch.bfloat16, "out")
    num_seqs, hq, d = q.shape
    num_blocks, hkv, bs, _ = k_cache.shape
    _shape(v_cache, k_cache.shape, "v_cache", "paged_attn_decode_fused_noalloc")
    _check_decode_buffers("paged_attn_decode_fused_noalloc", q, seq_lens, block_tables, out, 0,
                          None, None, None, 1)
    st = library().paged_attn_decode_fused_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens), num_seqs, hq,
        hkv, d, bs, num_blocks, block_tables.shape[1], float(scale), int(partition_size), _ptr(out),
        _stream(stream))
    _check("paged_attn_decode_fused_noalloc", st)


def paged_attn_decode_reduce(max_logits, exp_sums, tmp_out, seq_lens, partition_size: int, out,
                             stream=None) -> None:
    """Merge fp32 partials [S, H_q, NP(, D)] into bf16 `out` [S, H_q, D]."""
    import torch
    for name, t in (("max_logits", max_logits), ("exp_sums", exp_sums), ("tmp_out", tmp_out)):
        _want(t, torch.float32, name)
    _want(seq_lens, torch.int32, "seq_lens")
    _want(out, torch.bfloat16, "out")
    s, hq, npart, d = tmp_out.shape
    _shape(max_logits, (s, hq, npart), "max_logits", "paged_attn_decode_reduce")
    _shape(exp_sums, (s, hq, npart), "exp_sums", "paged_attn_decode_reduce")
    _shape(out, (s, hq, d), "out", "paged_attn_decode_reduce")
    if seq_lens.numel() != s:
        raise ValueError(f"paged_attn_decode_reduce: seq_lens must have {s} entries")
    st = library().paged_attn_decode_reduce(
        _ptr(max_logits), _ptr(exp_sums), _ptr(tmp_out), _ptr(seq_lens), s, hq, d,
        int(partition_size), npart, _ptr(out), _stream(stream))
    _check("paged_attn_decode_reduce", st)


def paged_attn_decode_fp8(q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens,
                          scale: float, partition_size: int = 0, out=None, max_logits=None,
                          exp_sums=None, tmp_out=None, max_num_partitions: Optional[int] = None,
                          stream=None) -> None:
    """Decode over an FP8 cache: k_cache / v_cache uint8 E4M3 codes
    [num_blocks, H_kv, bs, D], k_scales / v_scales fp32 [num_blocks, H_kv, bs]."""
    import torch
    _want(q, torch.bfloat16, "q")
    _want(k_cache, torch.uint8, "k_cache")
    _want(v_cache, torch.uint8, "v_cache")
    _want(k_scales, torch.float32, "k_scales")
    _want(v_scales, torch.float32, "v_scales")
    _want(block_tables, torch.int32, "block_tables")
    _want(seq_lens, torch.int32, "seq_lens")
    _want(out, torch.bfloat16, "out")
    for name, t in (("max_logits", max_logits), ("exp_sums", exp_sums), ("tmp_out", tmp_out)):
        _want(t, torch.float32, name)
    num_seqs, hq, d = q.shape
    num_blocks, hkv, bs, _ = k_cache.shape
    _shape(v_cache, k_cache.shape, "v_cache", "paged_attn_decode_fp8")
    _shape(k_scales, (num_blocks, hkv, bs), "k_scales", "paged_attn_decode_fp8")
    _shape(v_scales, (num_blocks, hkv, bs), "v_scales", "paged_attn_decode_fp8")
    if max_num_partitions is None:
        max_num_partitions = tmp_out.shape[2] if tmp_out is not None else 1
    _check_decode_buffers("paged_attn_decode_fp8", q, seq_lens, block_tables, out, partition_size,
                          max_logits, exp_sums, tmp_out, max_num_partitions)
    st = library().paged_attn_decode_fp8(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales), _ptr(block_tables),
        _ptr(seq_lens), num_seqs, hq, hkv, d, bs, num_blocks, block_tables.shape[1], float(scale),
        int(partition_size), _ptr(out), _ptr(max_logits), _ptr(exp_sums), _ptr(tmp_out),
        int(max_num_partitions), _stream(stream))
    _check("paged_attn_decode_fp8", st)


def paged_attn_decode_xpacked(q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                              partition_size: int = 0, out=None, max_logits=None, exp_sums=None,
                              tmp_out=None, max_num_partitions: Optional[int] = None,
                              stream=None) -> None:
    """Decode over the x-packed K [num_blocks, H_kv, D/8, bs, 8] and transposed
    V [num_blocks, H_kv, D, bs] caches (bf16)."""
    import torch
    _want(q, torch.bfloat16, "q")
    _want(k_cache, torch.bfloat16, "k_cache")
    _want(v_cache, torch.bfloat16, "v_cache")
    _want(block_tables, torch.int32, "block_tables")
    _want(seq_lens, torch.int32, "seq_lens")
    _want(out, torch.bfloat16, "out")
    for name, t in (("max_logits", max_logits), ("exp_sums", exp_sums), ("tmp_out", tmp_out)):
        _want(t, torch.float32, name)
    if k_cache.dim() != 5 or v_cache.dim() != 4:
        raise ValueError("k_cache must be [num_blocks, H_kv, D/8, bs, 8] and v_cache [num_blocks, H_kv, D, bs]")
    num_seqs, hq, d = q.shape
    num_blocks, hkv, _, bs = v_cache.shape
    _shape(k_cache, (num_blocks, hkv, d // 8, bs, 8), "k_cache", "paged_attn_decode_xpacked")
    _shape(v_cache, (num_blocks, hkv, d, bs), "v_cache", "paged_attn_decode_xpacked")
    if max_num_partitions is None:
        max_num_partitions = tmp_out.shape[2] if tmp_out is not None else 1
    _check_decode_buffers("paged_attn_decode_xpacked", q, seq_lens, block_tables, out, partition_size,
                          max_logits, exp_sums, tmp_out, max_num_partitions)
    st = library().paged_attn_decode_xpacked(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens), num_seqs, hq,
        hkv, d, bs, num_blocks, block_tables.shape[1], float(scale), int(partition_size),
        _ptr(out), _ptr(max_logits), _ptr(exp_sums), _ptr(tmp_out), int(max_num_partitions),
        _stream(stream))
    _check("paged_attn_decode_xpacked", st)


def paged_attn_decode_tokens(q, k_cache, v_cache, kv_indptr, kv_indices, max_kv_len: int,
                             scale: float, partition_size: int = 0, out=None, max_logits=None,
                             exp_sums=None, tmp_out=None, max_num_partitions: Optional[int] = None,
                             stream=None) -> None:
    """Decode over a token-granular cache k/v [num_slots, H_kv, D]; sequence s's
    token t is slot kv_indices[kv_indptr[s] + t]."""
    import torch
    _want(q, torch.bfloat16, "q")
    _want(k_cache, torch.bfloat16, "k_cache")
    _want(v_cache, torch.bfloat16, "v_cache")
    _want(kv_indptr, torch.int32, "kv_indptr")
    _want(kv_indices, torch.int32, "kv_indices")
    _want(out, torch.bfloat16, "out")
    for name, t in (("max_logits", max_logits), ("exp_sums", exp_sums), ("tmp_out", tmp_out)):
        _want(t, torch.float32, name)
    num_seqs, hq, d = q.shape
    num_slots, hkv, _ = k_cache.shape
    _shape(v_cache, k_cache.shape, "v_cache", "paged_attn_decode_tokens")
    if kv_indptr.numel() != num_seqs + 1:
        raise ValueError(f"paged_attn_decode_tokens: kv_indptr must have {num_seqs + 1} entries")
    if max_num_partitions is None:
        max_num_partitions = tmp_out.shape[2] if tmp_out is not None else 1
    _check_decode_buffers("paged_attn_decode_tokens", q, None, None, out, partition_size,
                          max_logits, exp_sums, tmp_out, max_num_partitions)
    st = library().paged_attn_decode_tokens(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_indptr), _ptr(kv_indices), num_seqs, hq, hkv,
        d, num_slots, int(max_kv_len), float(scale), int(partition_size), _ptr(out), _ptr(max_logits),
        _ptr(exp_sums), _ptr(tmp_out), int(max_num_partitions), _stream(stream))
    _check("paged_attn_decode_tokens", st)


def paged_attn_decode_reduce_indptr(max_logits, exp_sums, tmp_out, kv_indptr, partition_size: int,
                                    out, stream=None) -> None:
    """Merge partials [S, H_q, NP(, D)] with lengths from adjacent kv_indptr entries."""
    import torch
    for name, t in (("max_logits", max_logits), ("exp_sums", exp_sums), ("tmp_out", tmp_out)):
        _want(t, torch.float32, name)
    _want(kv_indptr, torch.int32, "kv_indptr")
    _want(out, torch.bfloat16, "out")
    s, hq, npart, d = tmp_out.shape
    _shape(max_logits, (s, hq, npart), "max_logits", "paged_attn_decode_reduce_indptr")
    _shape(exp_sums, (s, hq, npart), "exp_sums", "paged_attn_decode_reduce_indptr")
    _shape(out, (s, hq, d), "out", "paged_attn_decode_reduce_indptr")
    if kv_indptr.numel() != s + 1:
        raise ValueError(f"paged_attn_decode_reduce_indptr: kv_indptr must have {s + 1} entries")
    st = library().paged_attn_decode_reduce_indptr(
        _ptr(max_logits), _ptr(exp_sums), _ptr(tmp_out), _ptr(kv_indptr), s, hq, d,
        int(partition_size), npart, _ptr(out), _stream(stream))
    _check("paged_attn_decode_reduce_indptr", st)


def paged_attn_kv_append_xpacked(k_new, v_new, block_tables, seq_lens, cu_seqlens,
                                 max_new_tokens: int, k_cache, v_cache, stream=None) -> None:
    """Write new rows (bf16 [num_tokens, H_kv, D]) into x-packed K / transposed V caches."""
    import torch
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _want(t, torch.bfloat16, name)
    _want(block_tables, torch.int32, "block_tables")
    _want(seq_lens, torch.int32, "seq_lens")
    _want(cu_seqlens, torch.int32, "cu_seqlens")
    num_tokens, hkv, d = k_new.shape
    num_blocks, _, _, bs = v_cache.shape
    st = library().paged_attn_kv_append_xpacked(
        _ptr(k_new), _ptr(v_new), _ptr(block_tables), _ptr(seq_lens), _ptr(cu_seqlens),
        seq_lens.shape[0], num_tokens, int(max_new_tokens), hkv, d, bs, num_blocks,
        block_tables.shape[1], _ptr(k_cache), _ptr(v_cache), _stream(stream))
    _check("paged_attn_kv_append_xpacked", st)


def paged_attn_kv_append(k_new, v_new, block_tables, seq_lens, cu_seqlens, max_new_tokens: int,
                         k_cache, v_cache, stream=None) -> None:
    """Write new rows (bf16 [num_tokens, H_kv, D]) into a bf16 cache in place."""
    import torch
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _want(t, torch.bfloat16, name)
    _want(block_tables, torch.int32, "block_tables")
    _want(seq_lens, torch.int32, "seq_lens")
    _want(cu_seqlens, torch.int32, "cu_seqlens")
    num_tokens, hkv, d = k_new.shape
    num_blocks, _, bs, _ = k_cache.shape
    st = library().paged_attn_kv_append(
        _ptr(k_new), _ptr(v_new), _ptr(block_tables), _ptr(seq_lens), _ptr(cu_seqlens),
        seq_lens.shape[0], num_tokens, int(max_new_tokens), hkv, d, bs, num_blocks,
        block_tables.shape[1], _ptr(k_cache), _ptr(v_cache), _stream(stream))
    _check("paged_attn_kv_append", st)


def paged_attn_kv_append_fp8(k_new, v_new, block_tables, seq_lens, cu_seqlens,
                             max_new_tokens: int, k_cache, v_cache, k_scales, v_scales,
                             stream=None) -> None:
    """Quantize new rows to E4M3 (one scale per row) and write them into an FP8 cache."""
    import torch
    _want(k_new, torch.bfloat16, "k_new")
    _want(v_new, torch.bfloat16, "v_new")
    _want(k_cache, torch.uint8, "k_cache")
    _want(v_cache, torch.uint8, "v_cache")
    _want(k_scales, torch.float32, "k_scales")
    _want(v_scales, torch.float32, "v_scales")
    _want(block_tables, torch.int32, "block_tables")
    _want(seq_lens, torch.int32, "seq_lens")
    _want(cu_seqlens, torch.int32, "cu_seqlens")
    num_tokens, hkv, d = k_new.shape
    num_blocks, _, bs, _ = k_cache.shape
    st = library().paged_attn_kv_append_fp8(
        _ptr(k_new), _ptr(v_new), _ptr(block_tables), _ptr(seq_lens), _ptr(cu_seqlens),
        seq_lens.shape[0], num_tokens, int(max_new_tokens), hkv, d, bs, num_blocks,
        block_tables.shape[1], _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales),
        _stream(stream))
    _check("paged_attn_kv_append_fp8", st)


def paged_attn_prefill_ragged(q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens,
                              max_q_len: int, scale: float, out, stream=None) -> None:
    """Ragged causal prefill over packed rows [total_q, H_q, D]."""
    import torch
    _want(q, torch.bfloat16, "q")
    _want(k_cache, torch.bfloat16, "k_cache")
    _want(v_cache, torch.bfloat16, "v_cache")
    _want(block_tables, torch.int32, "block_tables")
    _want(seq_lens, torch.int32, "seq_lens")
    _want(cu_seqlens, torch.int32, "cu_seqlens")
    _want(out, torch.bfloat16, "out")
    total_q, hq, d = q.shape
    num_blocks, hkv, bs, _ = k_cache.shape
    st = library().paged_attn_prefill_ragged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens),
        _ptr(cu_seqlens), seq_lens.shape[0], total_q, int(max_q_len), hq, hkv, d, bs, num_blocks,
        block_tables.shape[1], float(scale), _ptr(out), _stream(stream))
    _check("paged_attn_prefill_ragged", st)


def paged_attn_prefill_ragged_split(q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens,
                                    max_q_len: int, scale: float, out, workspace=None,
                                    kv_chunk: int = 0, stream=None) -> None:
    """Split-KV form of the ragged causal prefill.  `workspace` is a uint8 device
    tensor of at least paged_attn_prefill_workspace_size(...) bytes whose first
    8 bytes are zero before the first call (a PrefillWorkspace provides one)."""
    import torch
    _want(q, torch.bfloat16, "q")
    _want(k_cache, torch.bfloat16, "k_cache")
    _want(v_cache, torch.bfloat16, "v_cache")
    _want(block_tables, torch.int32, "block_tables")
    _want(seq_lens, torch.int32, "seq_lens")
    _want(cu_seqlens, torch.int32, "cu_seqlens")
    _want(out, torch.bfloat16, "out")
    _want(workspace, torch.uint8, "workspace")
    total_q, hq, d = q.shape
    num_blocks, hkv, bs, _ = k_cache.shape
    nbytes = 0 if workspace is None else workspace.numel()
    st = library().paged_attn_prefill_ragged_split(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens),
        _ptr(cu_seqlens), seq_lens.shape[0], total_q, int(max_q_len), hq, hkv, d, bs, num_blocks,
        block_tables.shape[1], float(scale), int(kv_chunk), _ptr(workspace), nbytes, _ptr(out),
        _stream(stream))
    _check("paged_attn_prefill_ragged_split", st)


def paged_attn_prefill_chunk_size(num_seqs: int, total_q: int, num_q_heads: int, num_kv_heads: int,
                                  max_blocks_per_seq: int, block_size: int) -> int:
    return int(library().paged_attn_prefill_chunk_size(num_seqs, total_q, num_q_heads, num_kv_heads,
                                                       max_blocks_per_seq, block_size))


def paged_attn_prefill_workspace_size(total_q: int, num_q_heads: int, head_dim: int,
                                      max_blocks_per_seq: int, block_size: int, kv_chunk: int) -> int:
    return int(library().paged_attn_prefill_workspace_size(total_q, num_q_heads, head_dim,
                                                           max_blocks_per_seq, block_size, kv_chunk))


class PrefillWorkspace:
    """Zero-filled device workspace for paged_attn_prefill_ragged_split, sized for
    the chunk the call will use (kv_chunk, or the automatic choice when 0)."""

    def __init__(self, num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                 block_size, device, kv_chunk: int = 0):
        import torch
        chunk = int(kv_chunk) or paged_attn_prefill_chunk_size(
            num_seqs, total_q, num_q_heads, num_kv_heads, max_blocks_per_seq, block_size)
        self.kv_chunk = chunk
        nbytes = 256
        if chunk > 0:
            nbytes = paged_attn_prefill_workspace_size(total_q, num_q_heads, head_dim,
                                                       max_blocks_per_seq, block_size, chunk)
        self.buffer = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


def paged_attn_num_partitions(max_blocks_per_seq: int, block_size: int, partition_size: int) -> int:
    return int(library().paged_attn_num_partitions(max_blocks_per_seq, block_size, partition_size))


def paged_attn_choose_partition_size(num_seqs: int, num_kv_heads: int, max_seq_len: int,
                                     total_kv_tokens: int = 0) -> int:
    return int(library().paged_attn_choose_partition_size(num_seqs, num_kv_heads, max_seq_len,
                                                          int(total_kv_tokens)))


def paged_attn_prefill_tile_map(cu_seqlens_host, tile_rows: int) -> Tuple[list, list]:
    """Q-tile work map from host cu_seqlens (any int sequence)."""
    vals = [int(x) for x in cu_seqlens_host]
    n = len(vals) - 1
    cu = (ctypes.c_int32 * len(vals))(*vals)
    count = library().paged_attn_prefill_tile_map(cu, n, int(tile_rows), None, None, 0)
    if count < 0:
        raise ValueError("bad cu_seqlens or tile_rows")
    tb = (ctypes.c_int32 * max(count, 1))()
    ti = (ctypes.c_int32 * max(count, 1))()
    library().paged_attn_prefill_tile_map(cu, n, int(tile_rows), tb, ti, count)
    return list(tb[:count]), list(ti[:count])


def paged_attn_read_probe(buf, partial, stream=None) -> None:
    """HBM read-stream probe over every byte of the contiguous device tensor
    `buf` (its size a multiple of 16 bytes); one workgroup per element of the
    int32 tensor `partial`, which receives each workgroup's XOR of the 32-bit
    words it read."""
    import torch
    _want(partial, torch.int32, "partial")
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    nbytes = buf.numel() * buf.element_size()
    _check("paged_attn_read_probe",
           library().paged_attn_read_probe(_ptr(buf), nbytes, _ptr(partial), partial.numel(), _stream(stream)))


def paged_attn_gather_probe(k_cache, v_cache, block_tables, block_prefix, whole_blocks, partial,
                            stream=None) -> None:
    """Paged-gather read probe over the K/V tiles a decode of the batch reads
    (block_prefix int32 [num_seqs + 1]: prefix sums of ceil(L / 16)); one
    workgroup per element of the int32 tensor `partial`, which receives each
    workgroup's XOR of the 32-bit words it read.  whole_blocks: 0 (or False)
    per-(kv head, block) tiles, 1 (or True) whole blocks, 2 the tiles of 0
    through load-to-LDS instructions."""
    import torch
    _want(k_cache, torch.bfloat16, "k_cache")
    _want(v_cache, torch.bfloat16, "v_cache")
    _want(block_tables, torch.int32, "block_tables")
    _want(block_prefix, torch.int32, "block_prefix")
    _want(partial, torch.int32, "partial")
    num_blocks, hkv, bs, d = k_cache.shape
    _shape(v_cache, k_cache.shape, "v_cache", "paged_attn_gather_probe")
    num_seqs = block_tables.shape[0]
    if block_prefix.numel() != num_seqs + 1:
        raise ValueError(f"paged_attn_gather_probe: block_prefix must have {num_seqs + 1} entries")
    _check("paged_attn_gather_probe",
           library().paged_attn_gather_probe(_ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                             _ptr(block_prefix), num_seqs, hkv, d, bs, block_tables.shape[1],
                                             int(whole_blocks), _ptr(partial), partial.numel(),
                                             _stream(stream)))


def paged_attn_status_string(status: int) -> str:
    return status_string(status)


# ---------------------------------------------------------------------------
# convenience: a full decode step (partials workspace from torch, two launches)
# ---------------------------------------------------------------------------
class DecodeWorkspace:
    """fp32 partial buffers sized for (num_seqs, H_q, max_num_partitions, D), plus
    the zeroed arrival counters of the fused merge ([num_seqs * num_kv_heads])."""

    def __init__(self, num_seqs, num_q_heads, head_dim, max_num_partitions, device, *,
                 num_kv_heads: int):
        import torch
        self.max_num_partitions = int(max_num_partitions)
        if num_kv_heads <= 0 or num_q_heads % num_kv_heads:
            raise ValueError("num_kv_heads must be a positive divisor of num_q_heads")
        self.counters = torch.zeros(max(1, num_seqs * num_kv_heads), dtype=torch.int32, device=device)
        self.max_logits = torch.empty((num_seqs, num_q_heads, max_num_partitions),
                                      dtype=torch.float32, device=device)
        self.exp_sums = torch.empty_like(self.max_logits)
        self.tmp_out = torch.empty((num_seqs, num_q_heads, max_num_partitions, head_dim),
                                   dtype=torch.float32, device=device)


def paged_decode(q, k_cache, v_cache, block_tables, seq_lens, scale: float, partition_size: int,
                 out=None, workspace: Optional[DecodeWorkspace] = None, stream=None,
                 fused: bool = False):
    """Decode into `out`: one pass if partition_size == 0, else partials then the
    merge (a separate launch, or fused into the partition kernel)."""
    import torch
    if out is None:
        out = torch.empty_like(q)
    if partition_size == 0:
        paged_attn_decode(q, k_cache, v_cache, block_tables, seq_lens, scale, 0, out=out,
                          stream=stream)
        return out
    bs = k_cache.shape[2]
    npart = paged_attn_num_partitions(block_tables.shape[1], bs, partition_size)
    if workspace is None:
        workspace = DecodeWorkspace(q.shape[0], q.shape[1], q.shape[2], npart, q.device,
                                    num_kv_heads=k_cache.shape[1])
    if fused:
        paged_attn_decode_fused(q, k_cache, v_cache, block_tables, seq_lens, scale, partition_size,
                                out, workspace.max_logits, workspace.exp_sums, workspace.tmp_out,
                                workspace.counters, stream=stream)
        return out
    paged_attn_decode(q, k_cache, v_cache, block_tables, seq_lens, scale, partition_size,
                      max_logits=workspace.max_logits, exp_sums=workspace.exp_sums,
                      tmp_out=workspace.tmp_out, max_num_partitions=workspace.max_num_partitions,
                      stream=stream)
    paged_attn_decode_reduce(workspace.max_logits, workspace.exp_sums, workspace.tmp_out, seq_lens,
                             partition_size, out, stream=stream)
    return out
