"""Python binding of libattn.so: exact softmax attention over a paged KV cache on gfx950.

The functions here carry the names of the C entry points declared in include/attn.h and do
argument marshalling only: they check that tensors have the dtype, device and contiguity the
C ABI expects, pass their data pointers and the current HIP stream, and turn status codes into
exceptions. Every step of the attention itself runs in the library's HIP kernels. PyTorch only
provides device memory and streams. If the library has not been built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_OK, ATTN_ERR_NULL, ATTN_ERR_SHAPE, ATTN_ERR_BLOCK_SIZE, ATTN_ERR_GQA = 0, 1, 2, 3, 4
ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_METADATA, ATTN_ERR_HIP = 5, 6, 7, 8
ATTN_BF16, ATTN_F32 = 0, 1

EXPORTED = ("attn_workspace_bytes", "attn_decode_partition_tokens", "attn_varlen_fwd", "attn_check_metadata_host",
            "attn_cascade_workspace_bytes", "attn_cascade_fwd", "attn_check_cascade_host",
            "attn_kv_cache_write", "attn_check_slot_mapping_host", "attn_kv_cache_write_fp8",
            "attn_fp8_decode_workspace_bytes", "attn_fp8_decode_fwd", "attn_schedule_bytes",
            "attn_build_schedule",
            "attn_varlen_fwd_scheduled", "attn_decode_schedule_bytes",
            "attn_build_decode_schedule", "attn_varlen_fwd_prescheduled",
            "attn_varlen_fwd_mixed",
            "attn_varlen_fwd_noalloc", "attn_status_str")
# bytes of the library's fixed device array used by attn_varlen_fwd_noalloc
NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024


class attn_desc(ctypes.Structure):
    """Mirror of struct attn_desc in include/attn.h (13 x int32)."""
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_tokens", "num_decodes", "max_query_len", "max_seq_len", "num_heads",
        "num_kv_heads", "head_size", "num_blocks", "block_size", "max_blocks_per_seq", "dtype",
        "partition_tokens")]


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {attn_status_str(status)} ({status})")


_lib = None


def lib():
    """The loaded library. torch is imported first so that the process holds one HIP runtime."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (loads the HIP runtime that torch uses)
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m exact_softmax_attention_paged_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        P = ctypes.POINTER
        L.attn_workspace_bytes.argtypes = [P(attn_desc), P(sz)]
        L.attn_workspace_bytes.restype = i32
        L.attn_decode_partition_tokens.argtypes = [P(attn_desc), P(i32)]
        L.attn_decode_partition_tokens.restype = i32
        L.attn_varlen_fwd.argtypes = [P(attn_desc), vp, vp, vp, vp, vp, f32, i32, i32, vp, vp,
                                      vp, sz, vp]
        L.attn_varlen_fwd.restype = i32
        L.attn_varlen_fwd_noalloc.argtypes = [P(attn_desc), vp, vp, vp, vp, vp, f32, i32, i32,
                                              vp, vp, vp]
        L.attn_varlen_fwd_noalloc.restype = i32
        L.attn_check_metadata_host.argtypes = [P(attn_desc), vp, vp, vp]
        L.attn_check_metadata_host.restype = i32
        L.attn_cascade_workspace_bytes.argtypes = [P(attn_desc), i32, P(sz)]
        L.attn_cascade_workspace_bytes.restype = i32
        L.attn_cascade_fwd.argtypes = [P(attn_desc), vp, vp, vp, vp, vp, i32, f32, i32, vp, vp,
                                       vp, sz, vp]
        L.attn_cascade_fwd.restype = i32
        L.attn_check_cascade_host.argtypes = [P(attn_desc), vp, vp, vp, i32]
        L.attn_check_cascade_host.restype = i32
        i64 = ctypes.c_int64
        L.attn_kv_cache_write.argtypes = [P(attn_desc), vp, i64, vp, i64, vp, vp, vp]
        L.attn_kv_cache_write.restype = i32
        L.attn_kv_cache_write_fp8.argtypes = [P(attn_desc), vp, i64, vp, i64, vp, f32, f32, vp,
                                              vp]
        L.attn_kv_cache_write_fp8.restype = i32
        L.attn_fp8_decode_workspace_bytes.argtypes = [P(attn_desc), P(sz)]
        L.attn_fp8_decode_workspace_bytes.restype = i32
        L.attn_fp8_decode_fwd.argtypes = [P(attn_desc), vp, vp, vp, vp, vp, f32, f32, f32, i32,
                                          vp, vp, vp, sz, vp]
        L.attn_fp8_decode_fwd.restype = i32
        L.attn_schedule_bytes.argtypes = [P(attn_desc), P(sz)]
        L.attn_schedule_bytes.restype = i32
        L.attn_build_schedule.argtypes = [P(attn_desc), vp, vp, i32, i32, vp, sz, vp]
        L.attn_build_schedule.restype = i32
        L.attn_varlen_fwd_scheduled.argtypes = [P(attn_desc), vp, vp, vp, vp, vp, f32, i32, i32,
                                                vp, vp, vp, sz, vp, sz, vp]
        L.attn_varlen_fwd_scheduled.restype = i32
        L.attn_decode_schedule_bytes.argtypes = [P(attn_desc), i32, P(sz)]
        L.attn_decode_schedule_bytes.restype = i32
        L.attn_build_decode_schedule.argtypes = [P(attn_desc), vp, i32, vp, sz, vp]
        L.attn_build_decode_schedule.restype = i32
        L.attn_varlen_fwd_prescheduled.argtypes = [P(attn_desc), vp, vp, vp, vp, vp, f32, i32,
                                                   i32, vp, vp, vp, sz, vp, sz, vp, sz, vp]
        L.attn_varlen_fwd_prescheduled.restype = i32
        L.attn_varlen_fwd_mixed.argtypes = [P(attn_desc), vp, vp, vp, vp, vp, f32, i32, i32,
                                            vp, vp, vp, sz, vp]
        L.attn_varlen_fwd_mixed.restype = i32
        L.attn_check_slot_mapping_host.argtypes = [P(attn_desc), vp]
        L.attn_check_slot_mapping_host.restype = i32
        L.attn_status_str.argtypes = [i32]
        L.attn_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def attn_status_str(status: int) -> str:
    return lib().attn_status_str(int(status)).decode()


def make_desc(*, num_seqs, num_tokens, num_decodes, max_query_len, max_seq_len, num_heads,
              num_kv_heads, head_size, num_blocks, block_size, max_blocks_per_seq, dtype,
              partition_tokens=0) -> attn_desc:
    return attn_desc(int(num_seqs), int(num_tokens), int(num_decodes), int(max_query_len),
                     int(max_seq_len), int(num_heads), int(num_kv_heads), int(head_size),
                     int(num_blocks), int(block_size), int(max_blocks_per_seq), int(dtype),
                     int(partition_tokens))


def attn_workspace_bytes(desc: attn_desc) -> int:
    n = ctypes.c_size_t(0)
    st = lib().attn_workspace_bytes(ctypes.byref(desc), ctypes.byref(n))
    if st != ATTN_OK:
        raise AttnError(st, "attn_workspace_bytes")
    return int(n.value)


def attn_decode_partition_tokens(desc: attn_desc) -> int:
    """The split-KV partition length (keys) the library uses for desc's decode rows."""
    n = ctypes.c_int32(0)
    st = lib().attn_decode_partition_tokens(ctypes.byref(desc), ctypes.byref(n))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_partition_tokens")
    return int(n.value)


def attn_check_metadata_host(desc: attn_desc, block_table: np.ndarray,
                             query_start_loc: np.ndarray, seq_lens: np.ndarray) -> int:
    """Returns the status code (ATTN_OK or ATTN_ERR_METADATA, ...); host arrays only."""
    arrs = [np.ascontiguousarray(a, dtype=np.int32) for a in (block_table, query_start_loc,
                                                               seq_lens)]
    ptrs = [a.ctypes.data_as(ctypes.c_void_p) for a in arrs]
    return int(lib().attn_check_metadata_host(ctypes.byref(desc), *ptrs))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_tensor(name, t, dtype, device, allow_none=False):
    if t is None:
        if allow_none:
            return
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def attn_varlen_fwd(desc: attn_desc, q, kv_cache, block_table, query_start_loc, seq_lens,
                    scale: float, causal: bool, window: int, out, lse, workspace,
                    stream=None) -> None:
    """Queue the attention of one varlen batch on ``stream`` (default: torch's current stream).

    Tensors follow include/attn.h: q/out [num_tokens, Hq, d], kv_cache
    [2, num_blocks, block_size, Hkv, d] (bf16 or f32 as desc.dtype), int32 metadata, fp32 lse
    (or None) and a uint8 workspace of attn_workspace_bytes(desc) bytes (or None if 0)."""
    import torch
    _check_call("attn_varlen_fwd", desc, q, kv_cache, block_table, query_start_loc, seq_lens,
                out, lse, workspace)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = lib().attn_varlen_fwd(ctypes.byref(desc), _ptr(q), _ptr(kv_cache), _ptr(block_table),
                               _ptr(query_start_loc), _ptr(seq_lens), float(scale),
                               1 if causal else 0, int(window), _ptr(out), _ptr(lse),
                               _ptr(workspace), ws_bytes, ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_varlen_fwd")


def attn_varlen_fwd_noalloc(desc: attn_desc, q, kv_cache, block_table, query_start_loc,
                            seq_lens, scale: float, causal: bool, window: int, out, lse,
                            stream=None) -> None:
    """attn_varlen_fwd without a workspace argument: the decode rows' partial results go to the
    library's fixed device array (NOALLOC_SCRATCH_BYTES per GPU), so the call allocates
    nothing. Calls that could overlap on one GPU race on that array and must not be issued."""
    import torch
    _check_call("attn_varlen_fwd_noalloc", desc, q, kv_cache, block_table, query_start_loc,
                seq_lens, out, lse, None)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = lib().attn_varlen_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(kv_cache),
                                       _ptr(block_table), _ptr(query_start_loc),
                                       _ptr(seq_lens), float(scale), 1 if causal else 0,
                                       int(window), _ptr(out), _ptr(lse),
                                       ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_varlen_fwd_noalloc")


def _check_call(where, desc, q, kv_cache, block_table, query_start_loc, seq_lens, out, lse,
                workspace):
    import torch
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(where + " runs on a GPU device; q is on " + str(dev))
    dt = torch.bfloat16 if desc.dtype == ATTN_BF16 else torch.float32
    _check_tensor("q", q, dt, dev)
    _check_tensor("kv_cache", kv_cache, dt, dev)
    _check_tensor("out", out, dt, dev)
    for n, t in (("block_table", block_table), ("query_start_loc", query_start_loc),
                 ("seq_lens", seq_lens)):
        _check_tensor(n, t, torch.int32, dev)
    _check_tensor("lse", lse, torch.float32, dev, allow_none=True)
    if workspace is not None:
        _check_tensor("workspace", workspace, torch.uint8, dev)
    if tuple(q.shape) != (desc.num_tokens, desc.num_heads, desc.head_size) or \
            tuple(out.shape) != tuple(q.shape):
        raise ValueError("q/out shape does not match desc")
    if tuple(kv_cache.shape) != (2, desc.num_blocks, desc.block_size, desc.num_kv_heads,
                                 desc.head_size):
        raise ValueError("kv_cache shape does not match desc")
    _check_meta_shapes(desc, block_table, query_start_loc, seq_lens, lse)


def _check_meta_shapes(desc, block_table, query_start_loc, seq_lens, lse):
    """The kernels index these arrays from the descriptor's sizes without bounds checks, so
    an undersized one would be read or written past its end on the device: refuse it here,
    before anything is queued."""
    if tuple(block_table.shape) != (desc.num_seqs, desc.max_blocks_per_seq):
        raise ValueError(f"block_table must be [num_seqs={desc.num_seqs}, max_blocks_per_seq="
                         f"{desc.max_blocks_per_seq}], got {tuple(block_table.shape)}")
    if query_start_loc.dim() != 1 or query_start_loc.numel() != desc.num_seqs + 1:
        raise ValueError(f"query_start_loc must hold num_seqs + 1 = {desc.num_seqs + 1} "
                         f"entries, got shape {tuple(query_start_loc.shape)}")
    if seq_lens.dim() != 1 or seq_lens.numel() != desc.num_seqs:
        raise ValueError(f"seq_lens must hold num_seqs = {desc.num_seqs} entries, got shape "
                         f"{tuple(seq_lens.shape)}")
    if lse is not None and tuple(lse.shape) != (desc.num_tokens, desc.num_heads):
        raise ValueError(f"lse must be [num_tokens={desc.num_tokens}, num_heads="
                         f"{desc.num_heads}], got {tuple(lse.shape)}")


def attn_cascade_workspace_bytes(desc: attn_desc, common_prefix_len: int) -> int:
    n = ctypes.c_size_t(0)
    st = lib().attn_cascade_workspace_bytes(ctypes.byref(desc), int(common_prefix_len),
                                            ctypes.byref(n))
    if st != ATTN_OK:
        raise AttnError(st, "attn_cascade_workspace_bytes")
    return int(n.value)


def attn_check_cascade_host(desc: attn_desc, block_table: np.ndarray,
                            query_start_loc: np.ndarray, seq_lens: np.ndarray,
                            common_prefix_len: int) -> int:
    """Returns the status code of the host-side cascade precondition check."""
    arrs = [np.ascontiguousarray(a, dtype=np.int32) for a in (block_table, query_start_loc,
                                                               seq_lens)]
    ptrs = [a.ctypes.data_as(ctypes.c_void_p) for a in arrs]
    return int(lib().attn_check_cascade_host(ctypes.byref(desc), *ptrs, int(common_prefix_len)))


def attn_cascade_fwd(desc: attn_desc, q, kv_cache, block_table, query_start_loc, seq_lens,
                     common_prefix_len: int, scale: float, causal: bool, out, lse, workspace,
                     stream=None) -> None:
    """Queue a cascade attention call (shared prefix computed once; see include/attn.h).

    Tensors as for attn_varlen_fwd; the workspace holds
    attn_cascade_workspace_bytes(desc, common_prefix_len) bytes."""
    import torch
    _check_call("attn_cascade_fwd", desc, q, kv_cache, block_table, query_start_loc, seq_lens,
                out, lse, workspace)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = lib().attn_cascade_fwd(ctypes.byref(desc), _ptr(q), _ptr(kv_cache), _ptr(block_table),
                                _ptr(query_start_loc), _ptr(seq_lens), int(common_prefix_len),
                                float(scale), 1 if causal else 0, _ptr(out), _ptr(lse),
                                _ptr(workspace), ws_bytes, ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_cascade_fwd")


def varlen_fwd(q, kv_cache, block_table, query_start_loc, seq_lens, *, scale, causal, window=0,
               num_decodes, max_query_len, max_seq_len, partition_tokens=0, out=None,
               lse=None, want_lse=True, workspace=None):
    """Convenience wrapper: builds the descriptor from tensor shapes plus the host scalars,
    allocates out / lse / workspace with torch when not given, and calls attn_varlen_fwd.
    Returns (out, lse)."""
    import torch
    dtype = ATTN_BF16 if q.dtype == torch.bfloat16 else ATTN_F32
    desc = make_desc(num_seqs=seq_lens.numel(), num_tokens=q.shape[0], num_decodes=num_decodes,
                     max_query_len=max_query_len, max_seq_len=max_seq_len,
                     num_heads=q.shape[1], num_kv_heads=kv_cache.shape[3],
                     head_size=q.shape[2], num_blocks=kv_cache.shape[1],
                     block_size=kv_cache.shape[2], max_blocks_per_seq=block_table.shape[1],
                     dtype=dtype, partition_tokens=partition_tokens)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=q.device)
    if workspace is None:
        n = attn_workspace_bytes(desc)
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device) if n else None
    attn_varlen_fwd(desc, q, kv_cache, block_table, query_start_loc, seq_lens, scale, causal,
                    window, out, lse, workspace)
    return out, lse


def attn_check_slot_mapping_host(desc: attn_desc, slot_mapping: np.ndarray) -> int:
    """Returns the status code of the host-side slot_mapping check."""
    a = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    return int(lib().attn_check_slot_mapping_host(ctypes.byref(desc),
                                                  a.ctypes.data_as(ctypes.c_void_p)))


def _check_kv_rows(desc, key, value, dt, dev):
    row = desc.num_kv_heads * desc.head_size
    for name, t in (("key", key), ("value", value)):
        if t.dtype != dt or t.device != dev:
            raise TypeError(f"{name} must be {dt} on {dev}")
        if tuple(t.shape) != (desc.num_tokens, desc.num_kv_heads, desc.head_size) or \
                t.stride(2) != 1 or t.stride(1) != desc.head_size or t.stride(0) < row:
            raise ValueError(f"{name} must be [num_tokens, num_kv_heads, head_size] with "
                             "contiguous heads")


def _fp8_cache_ok(kv_cache, desc, dev):
    import torch
    if kv_cache.device != dev or kv_cache.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError("the E4M3 cache must be a uint8 or float8_e4m3fn tensor on " + str(dev))
    if not kv_cache.is_contiguous() or tuple(kv_cache.shape) != (
            2, desc.num_blocks, desc.block_size, desc.num_kv_heads, desc.head_size):
        raise ValueError("kv_cache shape does not match desc")


def attn_kv_cache_write_fp8(desc: attn_desc, key, value, slot_mapping, k_scale: float,
                            v_scale: float, kv_cache, stream=None) -> None:
    """Queue the quantising write of bf16 K/V rows into an E4M3 cache (uint8 or
    float8_e4m3fn tensor of the cache shape) at slot_mapping."""
    import torch
    dev = kv_cache.device
    if dev.type != "cuda":
        raise ValueError("attn_kv_cache_write_fp8 runs on a GPU device")
    _check_kv_rows(desc, key, value, torch.bfloat16, dev)
    _check_tensor("slot_mapping", slot_mapping, torch.int64, dev)
    if slot_mapping.numel() != desc.num_tokens:
        raise ValueError("slot_mapping must hold num_tokens entries")
    _fp8_cache_ok(kv_cache, desc, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    st = lib().attn_kv_cache_write_fp8(ctypes.byref(desc), _ptr(key), int(key.stride(0)),
                                       _ptr(value), int(value.stride(0)), _ptr(slot_mapping),
                                       float(k_scale), float(v_scale), _ptr(kv_cache),
                                       ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_kv_cache_write_fp8")


def attn_fp8_decode_workspace_bytes(desc: attn_desc) -> int:
    """Workspace bytes of attn_fp8_decode_fwd for desc (its E4M3 default partition)."""
    n = ctypes.c_size_t(0)
    st = lib().attn_fp8_decode_workspace_bytes(ctypes.byref(desc), ctypes.byref(n))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fp8_decode_workspace_bytes")
    return int(n.value)


def attn_fp8_decode_fwd(desc: attn_desc, q, kv_cache, block_table, query_start_loc, seq_lens,
                        scale: float, k_scale: float, v_scale: float, window: int, out, lse,
                        workspace, stream=None) -> None:
    """Queue decode attention (num_decodes == num_seqs) over an E4M3 cache; q / out bf16."""
    import torch
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("attn_fp8_decode_fwd runs on a GPU device; q is on " + str(dev))
    _check_tensor("q", q, torch.bfloat16, dev)
    _check_tensor("out", out, torch.bfloat16, dev)
    for n, t in (("block_table", block_table), ("query_start_loc", query_start_loc),
                 ("seq_lens", seq_lens)):
        _check_tensor(n, t, torch.int32, dev)
    _check_tensor("lse", lse, torch.float32, dev, allow_none=True)
    if workspace is not None:
        _check_tensor("workspace", workspace, torch.uint8, dev)
    _fp8_cache_ok(kv_cache, desc, dev)
    if tuple(q.shape) != (desc.num_tokens, desc.num_heads, desc.head_size) or \
            tuple(out.shape) != tuple(q.shape):
        raise ValueError("q/out shape does not match desc")
    _check_meta_shapes(desc, block_table, query_start_loc, seq_lens, lse)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = lib().attn_fp8_decode_fwd(ctypes.byref(desc), _ptr(q), _ptr(kv_cache),
                                   _ptr(block_table), _ptr(query_start_loc), _ptr(seq_lens),
                                   float(scale), float(k_scale), float(v_scale), int(window),
                                   _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                   ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fp8_decode_fwd")


def attn_kv_cache_write(desc: attn_desc, key, value, slot_mapping, kv_cache,
                        stream=None) -> None:
    """Queue the write of the new tokens' K/V rows into kv_cache at slot_mapping.

    key / value: [num_tokens, num_kv_heads, head_size] views whose last two dimensions are
    contiguous (the token stride may be larger, e.g. columns of a packed QKV tensor);
    slot_mapping: int64 [num_tokens]; kv_cache: [2, num_blocks, block_size, num_kv_heads,
    head_size]; all on one GPU, dtype of desc."""
    import torch
    dev = kv_cache.device
    if dev.type != "cuda":
        raise ValueError("attn_kv_cache_write runs on a GPU device; kv_cache is on " + str(dev))
    dt = torch.bfloat16 if desc.dtype == ATTN_BF16 else torch.float32
    _check_kv_rows(desc, key, value, dt, dev)
    _check_tensor("slot_mapping", slot_mapping, torch.int64, dev)
    _check_tensor("kv_cache", kv_cache, dt, dev)
    if slot_mapping.numel() != desc.num_tokens:
        raise ValueError("slot_mapping must hold num_tokens entries")
    if tuple(kv_cache.shape) != (2, desc.num_blocks, desc.block_size, desc.num_kv_heads,
                                 desc.head_size):
        raise ValueError("kv_cache shape does not match desc")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    st = lib().attn_kv_cache_write(ctypes.byref(desc), _ptr(key), int(key.stride(0)),
                                   _ptr(value), int(value.stride(0)), _ptr(slot_mapping),
                                   _ptr(kv_cache), ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_kv_cache_write")


def attn_schedule_bytes(desc: attn_desc) -> int:
    n = ctypes.c_size_t(0)
    st = lib().attn_schedule_bytes(ctypes.byref(desc), ctypes.byref(n))
    if st != ATTN_OK:
        raise AttnError(st, "attn_schedule_bytes")
    return int(n.value)


def attn_build_schedule(desc: attn_desc, query_start_loc, seq_lens, causal: bool, window: int,
                        schedule, stream=None) -> None:
    """Queue the build of the prefill work schedule into ``schedule`` (int32 device tensor of
    at least attn_schedule_bytes(desc) / 4 elements)."""
    import torch
    dev = schedule.device
    if dev.type != "cuda":
        raise ValueError("attn_build_schedule runs on a GPU device")
    for n, t in (("query_start_loc", query_start_loc), ("seq_lens", seq_lens),
                 ("schedule", schedule)):
        _check_tensor(n, t, torch.int32, dev)
    if query_start_loc.numel() != desc.num_seqs + 1 or seq_lens.numel() != desc.num_seqs:
        raise ValueError("query_start_loc / seq_lens must hold num_seqs + 1 / num_seqs entries")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    st = lib().attn_build_schedule(ctypes.byref(desc), _ptr(query_start_loc), _ptr(seq_lens),
                                   1 if causal else 0, int(window), _ptr(schedule),
                                   schedule.numel() * 4, ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_build_schedule")


def attn_varlen_fwd_scheduled(desc: attn_desc, q, kv_cache, block_table, query_start_loc,
                              seq_lens, scale: float, causal: bool, window: int, out, lse,
                              workspace, schedule, stream=None) -> None:
    """attn_varlen_fwd with the prefill rows dispatched in the order of ``schedule``."""
    import torch
    _check_call("attn_varlen_fwd_scheduled", desc, q, kv_cache, block_table, query_start_loc,
                seq_lens, out, lse, workspace)
    _check_tensor("schedule", schedule, torch.int32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = lib().attn_varlen_fwd_scheduled(
        ctypes.byref(desc), _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(query_start_loc),
        _ptr(seq_lens), float(scale), 1 if causal else 0, int(window), _ptr(out), _ptr(lse),
        _ptr(workspace), ws_bytes, _ptr(schedule), schedule.numel() * 4,
        ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_varlen_fwd_scheduled")


def attn_decode_schedule_bytes(desc: attn_desc, window: int = 0) -> int:
    n = ctypes.c_size_t(0)
    st = lib().attn_decode_schedule_bytes(ctypes.byref(desc), int(window), ctypes.byref(n))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_schedule_bytes")
    return int(n.value)


def attn_build_decode_schedule(desc: attn_desc, seq_lens, window: int, schedule,
                               stream=None) -> None:
    """Queue the build of the decode work schedule into ``schedule`` (int32 device tensor of
    at least attn_decode_schedule_bytes(desc, window) / 4 elements)."""
    import torch
    dev = schedule.device
    if dev.type != "cuda":
        raise ValueError("attn_build_decode_schedule runs on a GPU device")
    for n, t in (("seq_lens", seq_lens), ("schedule", schedule)):
        _check_tensor(n, t, torch.int32, dev)
    if seq_lens.numel() != desc.num_seqs:
        raise ValueError("seq_lens must hold num_seqs entries")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    st = lib().attn_build_decode_schedule(ctypes.byref(desc), _ptr(seq_lens), int(window),
                                          _ptr(schedule), schedule.numel() * 4,
                                          ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_build_decode_schedule")


def attn_varlen_fwd_prescheduled(desc: attn_desc, q, kv_cache, block_table, query_start_loc,
                                 seq_lens, scale: float, causal: bool, window: int, out, lse,
                                 workspace, prefill_schedule=None, decode_schedule=None,
                                 stream=None) -> None:
    """attn_varlen_fwd that reads the prefill and / or decode work schedule built ahead
    (either may be None: that part is then scheduled by the call itself)."""
    import torch
    _check_call("attn_varlen_fwd_prescheduled", desc, q, kv_cache, block_table,
                query_start_loc, seq_lens, out, lse, workspace)
    for n, t in (("prefill_schedule", prefill_schedule), ("decode_schedule", decode_schedule)):
        _check_tensor(n, t, torch.int32, q.device, allow_none=True)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    ps_bytes = 0 if prefill_schedule is None else prefill_schedule.numel() * 4
    ds_bytes = 0 if decode_schedule is None else decode_schedule.numel() * 4
    st = lib().attn_varlen_fwd_prescheduled(
        ctypes.byref(desc), _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(query_start_loc),
        _ptr(seq_lens), float(scale), 1 if causal else 0, int(window), _ptr(out), _ptr(lse),
        _ptr(workspace), ws_bytes, _ptr(prefill_schedule), ps_bytes, _ptr(decode_schedule),
        ds_bytes, ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_varlen_fwd_prescheduled")


def attn_varlen_fwd_mixed(desc: attn_desc, q, kv_cache, block_table, query_start_loc, seq_lens,
                          scale: float, causal: bool, window: int, out, lse, prefill_schedule,
                          stream=None) -> None:
    """One launch for a mixed batch: the decode rows one wave per (request, kv head group)
    over all their keys, the prefill rows from ``prefill_schedule`` (attn_build_schedule).
    Needs no workspace."""
    import torch
    _check_call("attn_varlen_fwd_mixed", desc, q, kv_cache, block_table, query_start_loc,
                seq_lens, out, lse, None)
    _check_tensor("prefill_schedule", prefill_schedule, torch.int32, q.device, allow_none=True)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    ps_bytes = 0 if prefill_schedule is None else prefill_schedule.numel() * 4
    st = lib().attn_varlen_fwd_mixed(
        ctypes.byref(desc), _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(query_start_loc),
        _ptr(seq_lens), float(scale), 1 if causal else 0, int(window), _ptr(out), _ptr(lse),
        _ptr(prefill_schedule), ps_bytes, ctypes.c_void_p(stream.cuda_stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_varlen_fwd_mixed")
