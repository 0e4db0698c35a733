"""Thin ctypes binding of libpa.so (include/pa.h): argument marshalling only.

Every function takes torch tensors that live on the GPU (device memory and the
current stream come from torch) and calls the C entry point of the same name;
all computation happens in the HIP kernels.  There is no fallback: if the
library is missing, or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading
from typing import Optional

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# PA_LIBRARY names another build of the same library (the AddressSanitizer build of asan_check.py)
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(_PKG, "libpa.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "pa.h")

PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
KERNELS = {"slot_mapping": 0, "reshape_and_cache": 1, "decode": 2, "decode_merge": 3, "prefill": 4,
           "prefill_merge": 5, "stage_fp8": 6, "fused": 7}
STATUS = {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_DTYPE", 4: "PA_ERR_WORKSPACE",
          5: "PA_ERR_UNSUPPORTED", 6: "PA_ERR_HIP", 7: "PA_ERR_NO_SPACE", 8: "PA_ERR_STATE"}

_lock = threading.Lock()
_lib = None


class PAError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


def header_symbols() -> list:
    """Names of the functions include/pa.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(pa_\w+)\s*\(", text, flags=re.M)))


def load() -> ctypes.CDLL:
    """Loads libpa.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library {LIB_PATH} is not built; run paged_kv_cache_418_amd.build_lib.build()")
        lib = ctypes.CDLL(LIB_PATH)
        P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        sig = {
            "pa_abi_version": ([], ctypes.c_int),
            "pa_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "pa_last_error": ([], ctypes.c_char_p),
            "pa_slot_mapping": ([P, P, i32, P, P, i32, i32, i32, P], ctypes.c_int),
            "pa_reshape_and_cache": ([P, P, i64, i64, P, P, P, i32, i32, i32, i32, i32, ctypes.c_int, P],
                                     ctypes.c_int),
            "pa_reshape_and_cache_fp8": ([P, P, i64, i64, P, P, P, i32, i32, i32, i32, i32, ctypes.c_int, f32, f32,
                                          P], ctypes.c_int),
            "pa_write_kv": ([P, P, i64, i64, P, P, P, P, i32, P, P, i32, i32, i32, i32, i32, i32, i32, ctypes.c_int,
                             P], ctypes.c_int),
            "pa_write_kv_fp8": ([P, P, i64, i64, P, P, P, P, i32, P, P, i32, i32, i32, i32, i32, i32, i32,
                                 ctypes.c_int, f32, f32, P], ctypes.c_int),
            "pa_decode_workspace_bytes": ([i32, i32, i32, i32, i32, i32], sz),
            "pa_decode": ([P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32, f32, ctypes.c_int, i32, P, sz,
                           P], ctypes.c_int),
            "pa_decode_static": ([P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32, f32, ctypes.c_int, i32,
                                  P], ctypes.c_int),
            "pa_decode_fp8": ([P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32, f32, ctypes.c_int, f32, f32,
                               i32, P, sz, P], ctypes.c_int),
            "pa_decode_write": ([P, P, P, P, i64, i64, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32, f32,
                                 ctypes.c_int, i32, P, sz, P], ctypes.c_int),
            "pa_decode_write_fp8": ([P, P, P, P, i64, i64, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32, f32,
                                     ctypes.c_int, f32, f32, i32, P, sz, P], ctypes.c_int),
            "pa_decode_window_write": ([P, P, P, P, i64, i64, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32, f32,
                                        ctypes.c_int, i32, i32, P, sz, P], ctypes.c_int),
            "pa_decode_window_write_fp8": ([P, P, P, P, i64, i64, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32,
                                            f32, ctypes.c_int, f32, f32, i32, i32, P, sz, P], ctypes.c_int),
            "pa_decode_local_write": ([P, P, P, P, i64, i64, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32, f32,
                                       ctypes.c_int, i32, i32, P, sz, P], ctypes.c_int),
            "pa_decode_local_write_fp8": ([P, P, P, P, i64, i64, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32,
                                           f32, ctypes.c_int, f32, f32, i32, i32, P, sz, P], ctypes.c_int),
            "pa_decode_cascade_write": ([P, P, P, P, i64, i64, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32,
                                         f32, ctypes.c_int, i32, i32, P, sz, P], ctypes.c_int),
            "pa_decode_cascade_write_fp8": ([P, P, P, P, i64, i64, P, P, P, i32, P, i32, i32, i32, i32, i32, i32,
                                             i32, f32, ctypes.c_int, f32, f32, i32, i32, P, sz, P], ctypes.c_int),
            "pa_decode_cascade_workspace_bytes": ([i32, i32, i32, i32, i32, i32, i32], sz),
            "pa_decode_cascade": ([P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32, f32, ctypes.c_int, i32,
                                   i32, P, sz, P], ctypes.c_int),
            "pa_decode_cascade_fp8": ([P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32, f32, ctypes.c_int,
                                       f32, f32, i32, i32, P, sz, P], ctypes.c_int),
            "pa_prefill_varlen_workspace_bytes": ([P, P, i32, i32, i32, i32], sz),
            "pa_prefill_varlen": ([P, P, P, P, P, i32, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, f32,
                                   ctypes.c_int, P, sz, P], ctypes.c_int),
            "pa_prefill_varlen_write": ([P, P, P, P, i64, i64, P, P, P, i32, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                         i32, f32, ctypes.c_int, P, sz, P], ctypes.c_int),
            "pa_prefill_varlen_fp8_workspace_bytes": ([P, P, i32, i32, i32, i32, i32], sz),
            "pa_prefill_varlen_fp8": ([P, P, P, P, P, i32, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, f32,
                                       ctypes.c_int, f32, f32, P, sz, P], ctypes.c_int),
            "pa_decode_window": ([P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32, f32, ctypes.c_int, i32,
                                  i32, P, sz, P], ctypes.c_int),
            "pa_prefill_varlen_window_workspace_bytes": ([P, P, i32, i32, i32, i32, i32], sz),
            "pa_prefill_varlen_window": ([P, P, P, P, P, i32, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, f32,
                                          ctypes.c_int, i32, P, sz, P], ctypes.c_int),
            "pa_decode_local": ([P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32, f32, ctypes.c_int, i32,
                                 i32, P, sz, P], ctypes.c_int),
            "pa_prefill_varlen_local_workspace_bytes": ([P, P, i32, i32, i32, i32, i32], sz),
            "pa_prefill_varlen_local": ([P, P, P, P, P, i32, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, f32,
                                         ctypes.c_int, i32, P, sz, P], ctypes.c_int),
            "pa_decode_window_fp8": ([P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32, f32, ctypes.c_int,
                                      f32, f32, i32, i32, P, sz, P], ctypes.c_int),
            "pa_decode_local_fp8": ([P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32, f32, ctypes.c_int,
                                     f32, f32, i32, i32, P, sz, P], ctypes.c_int),
            "pa_prefill_varlen_window_fp8_workspace_bytes": ([P, P, i32, i32, i32, i32, i32, i32], sz),
            "pa_prefill_varlen_window_fp8": ([P, P, P, P, P, i32, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, f32,
                                              ctypes.c_int, f32, f32, i32, P, sz, P], ctypes.c_int),
            "pa_prefill_varlen_local_fp8_workspace_bytes": ([P, P, i32, i32, i32, i32, i32, i32], sz),
            "pa_prefill_varlen_local_fp8": ([P, P, P, P, P, i32, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, f32,
                                             ctypes.c_int, f32, f32, i32, P, sz, P], ctypes.c_int),
            "pa_pool_create": ([i32, i32, ctypes.POINTER(P)], ctypes.c_int),
            "pa_pool_destroy": ([P], None),
            "pa_pool_num_free": ([P], i32),
            "pa_pool_hash_blocks": ([P, i32, i32, ctypes.c_uint64, P], i32),
            "pa_pool_find_longest_cache_hit": ([P, P, i32, P], i32),
            "pa_pool_allocate_slots": ([P, i64, i32, P, i32, ctypes.POINTER(i32)], ctypes.c_int),
            "pa_pool_cache_blocks": ([P, i64, P, i32], ctypes.c_int),
            "pa_pool_release_before": ([P, i64, i32], ctypes.c_int),
            "pa_pool_free": ([P, i64], ctypes.c_int),
            "pa_pool_block_table": ([P, i64, P, i32], i32),
            "pa_pool_block_state": ([P, i32, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32),
                                     ctypes.POINTER(ctypes.c_uint64)], ctypes.c_int),
            "pa_pool_free_queue": ([P, P, i32], i32),
            "pa_probe_mfma_peak": ([P, i32, i32, P], ctypes.c_int),
            "pa_set_validate": ([ctypes.c_int], ctypes.c_int),
            "pa_set_fused": ([ctypes.c_int], ctypes.c_int),
            "pa_timing_enable": ([ctypes.c_int], ctypes.c_int),
            "pa_timing_reset": ([], ctypes.c_int),
            "pa_timing_read": ([ctypes.c_int, ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
            "pa_timing_read_launches": ([ctypes.c_int, P, i32, ctypes.POINTER(i32)], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
        return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise PAError(fn, status, load().pa_last_error().decode())


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    return t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    return {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.uint8: PA_FP8_E4M3}[t.dtype]


def _i32_host(x) -> torch.Tensor:
    t = torch.as_tensor(x, dtype=torch.int32, device="cpu").contiguous()
    return t


def _contig(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if nbytes == 0:
        return workspace, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def abi_version() -> int:
    return int(load().pa_abi_version())


def pa_slot_mapping(block_tables, seq_lens, query_start_loc, num_tokens: int, block_size: int = 16, out=None):
    """slot_mapping[t] = block_tables[s][p // B] * B + p % B for every new row t (device int32)."""
    lib = load()
    bt = _contig(block_tables, "block_tables")
    if out is None:
        out = torch.empty(num_tokens, dtype=torch.int32, device=bt.device)
    _check("pa_slot_mapping", lib.pa_slot_mapping(_dev(out, "out"), _dev(bt, "block_tables"), bt.shape[1],
                                                  _dev(seq_lens, "seq_lens"), _dev(query_start_loc, "qsl"),
                                                  seq_lens.shape[0], num_tokens, block_size, _stream()))
    return out


def _check_kv_write(key, value, key_cache, value_cache, fp8: bool) -> None:
    """The pools take the new rows byte for byte (or quantise them): dtypes and [Hkv, D] must agree."""
    if key.dim() != 3 or value.shape != key.shape:
        raise ValueError("key and value must both be [num_tokens, num_kv_heads, head_dim]")
    if key_cache.dim() != 4 or value_cache.shape != key_cache.shape:
        raise ValueError("key_cache and value_cache must both be [num_blocks, block_size, num_kv_heads, head_dim]")
    if tuple(key_cache.shape[2:]) != tuple(key.shape[1:]):
        raise ValueError(f"pool rows {tuple(key_cache.shape[2:])} differ from the new rows {tuple(key.shape[1:])}")
    if key.dtype != value.dtype:
        raise ValueError(f"key dtype {key.dtype} differs from value dtype {value.dtype}")
    if key_cache.dtype != value_cache.dtype:
        raise ValueError(f"key_cache dtype {key_cache.dtype} differs from value_cache dtype {value_cache.dtype}")
    if fp8:
        if key_cache.dtype != torch.uint8 or key.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("fp8 pools are uint8 E4M3 codes written from float32 or bfloat16 rows")
    elif key.dtype != key_cache.dtype or key.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"the pools ({key_cache.dtype}) must have the new rows' dtype ({key.dtype}), float32 or "
                         "bfloat16")


def _check_pools(query, key_cache, value_cache, fp8: bool) -> None:
    """The attention calls read the pools in the query's dtype (bf16 or fp32 pools) or as E4M3 codes (fp8)."""
    if key_cache.dtype != value_cache.dtype or key_cache.shape != value_cache.shape:
        raise ValueError("key_cache and value_cache must have the same dtype and shape")
    if fp8 and key_cache.dtype != torch.uint8:
        raise ValueError("fp8 pools are uint8 E4M3 codes")
    if not fp8 and key_cache.dtype != query.dtype:
        raise ValueError(f"the pools ({key_cache.dtype}) must have the query's dtype ({query.dtype})")


def pa_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping):
    """Writes key/value [T, Hkv, D] (token stride may exceed Hkv*D) into the pools."""
    lib = load()
    _check_kv_write(key, value, key_cache, value_cache, fp8=False)
    T, H, D = key.shape
    if key.stride(1) != D or key.stride(2) != 1 or value.stride(1) != D or value.stride(2) != 1:
        raise ValueError("heads and head_dim of key/value must be contiguous inside a token")
    NB, B = key_cache.shape[0], key_cache.shape[1]
    _check("pa_reshape_and_cache", lib.pa_reshape_and_cache(
        _dev(key, "key"), _dev(value, "value"), key.stride(0), value.stride(0), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(slot_mapping, "slot_mapping"), T, H, D, B, NB, _dtype_code(key_cache),
        _stream()))


def pa_reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale: float, v_scale: float):
    lib = load()
    _check_kv_write(key, value, key_cache, value_cache, fp8=True)
    T, H, D = key.shape
    if key.stride(1) != D or key.stride(2) != 1 or value.stride(1) != D or value.stride(2) != 1:
        raise ValueError("heads and head_dim of key/value must be contiguous inside a token")
    NB, B = key_cache.shape[0], key_cache.shape[1]
    _check("pa_reshape_and_cache_fp8", lib.pa_reshape_and_cache_fp8(
        _dev(key, "key"), _dev(value, "value"), key.stride(0), value.stride(0), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(slot_mapping, "slot_mapping"), T, H, D, B, NB, _dtype_code(key),
        float(k_scale), float(v_scale), _stream()))


def pa_write_kv(key, value, key_cache, value_cache, block_tables, seq_lens, query_start_loc, max_q_len: int,
                slot_mapping=None, k_scale: float = None, v_scale: float = None):
    """Slot mapping + KV write in one launch (fp8 pools when k_scale/v_scale are given); returns slot_mapping."""
    lib = load()
    _check_kv_write(key, value, key_cache, value_cache, fp8=k_scale is not None)
    T, H, D = key.shape
    if key.stride(1) != D or key.stride(2) != 1 or value.stride(1) != D or value.stride(2) != 1:
        raise ValueError("heads and head_dim of key/value must be contiguous inside a token")
    NB, B = key_cache.shape[0], key_cache.shape[1]
    S = seq_lens.shape[0]
    sm = None if slot_mapping is None else _dev(slot_mapping, "slot_mapping")
    common = (_dev(key, "key"), _dev(value, "value"), key.stride(0), value.stride(0), _dev(key_cache, "key_cache"),
              _dev(value_cache, "value_cache"), sm, _dev(block_tables, "block_tables"), block_tables.shape[1],
              _dev(seq_lens, "seq_lens"), _dev(query_start_loc, "query_start_loc"), S, T, max_q_len, H, D, B, NB)
    if k_scale is None:
        _check("pa_write_kv", lib.pa_write_kv(*common, _dtype_code(key_cache), _stream()))
    else:
        _check("pa_write_kv_fp8", lib.pa_write_kv_fp8(*common, _dtype_code(key), float(k_scale), float(v_scale),
                                                      _stream()))
    return slot_mapping


def pa_decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int, max_seq_len: int,
                              num_splits: int = 0) -> int:
    return int(load().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                                num_splits))


def pa_decode(query, key_cache, value_cache, block_tables, seq_lens, scale: float, max_seq_len: int,
              num_splits: int = 0, out=None, workspace=None):
    """One new token per sequence: query [S, Hq, D] -> out [S, Hq, D] (fp32 or bf16 pools)."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=False)
    S, Hq, D = query.shape
    NB, B, Hkv, _ = key_cache.shape
    out = torch.empty_like(query) if out is None else out
    ws, wsb = _workspace(pa_decode_workspace_bytes(S, Hq, Hkv, D, max_seq_len, num_splits), query.device, workspace)
    _check("pa_decode", lib.pa_decode(
        _dev(out, "out"), _dev(_contig(query, "query"), "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(seq_lens, "seq_lens"), S, Hq, Hkv, D, B, NB, max_seq_len, float(scale), _dtype_code(key_cache),
        num_splits, None if ws is None else ws.data_ptr(), wsb, _stream()))
    return out


def pa_decode_static(query, key_cache, value_cache, block_tables, seq_lens, scale: float, max_seq_len: int,
                     num_splits: int = 0, out=None):
    """pa_decode with the library's static scratch (no workspace, no allocation by the library)."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=False)
    S, Hq, D = query.shape
    NB, B, Hkv, _ = key_cache.shape
    out = torch.empty_like(query) if out is None else out
    _check("pa_decode_static", lib.pa_decode_static(
        _dev(out, "out"), _dev(_contig(query, "query"), "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(seq_lens, "seq_lens"), S, Hq, Hkv, D, B, NB, max_seq_len, float(scale), _dtype_code(key_cache),
        num_splits, _stream()))
    return out


def pa_decode_fp8(query, key_cache, value_cache, block_tables, seq_lens, scale: float, k_scale: float,
                  v_scale: float, max_seq_len: int, num_splits: int = 0, out=None, workspace=None):
    """pa_decode over fp8 E4M3 pools (uint8 codes) with per-tensor scales."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=True)
    S, Hq, D = query.shape
    NB, B, Hkv, _ = key_cache.shape
    out = torch.empty_like(query) if out is None else out
    ws, wsb = _workspace(pa_decode_workspace_bytes(S, Hq, Hkv, D, max_seq_len, num_splits), query.device, workspace)
    _check("pa_decode_fp8", lib.pa_decode_fp8(
        _dev(out, "out"), _dev(_contig(query, "query"), "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(seq_lens, "seq_lens"), S, Hq, Hkv, D, B, NB, max_seq_len, float(scale), _dtype_code(query),
        float(k_scale), float(v_scale), num_splits, None if ws is None else ws.data_ptr(), wsb, _stream()))
    return out


def _decode_write_args(query, key, value, key_cache, value_cache, block_tables, seq_lens, max_seq_len, num_splits,
                       out, workspace, prefix_blocks=None):
    S, Hq, D = query.shape
    NB, B, Hkv, _ = key_cache.shape
    if tuple(key.shape) != (S, Hkv, D) or tuple(value.shape) != (S, Hkv, D):
        raise ValueError(f"key/value must be [{S}, {Hkv}, {D}] (one new row per sequence)")
    if key.dtype != query.dtype or value.dtype != query.dtype:
        raise ValueError("key/value must have the query's dtype")
    _check_kv_write(key, value, key_cache, value_cache, fp8=key_cache.dtype == torch.uint8)
    if key.stride(1) != D or key.stride(2) != 1 or value.stride(1) != D or value.stride(2) != 1:
        raise ValueError("heads and head_dim of key/value must be contiguous inside a token")
    out = torch.empty_like(query) if out is None else out
    nbytes = (pa_decode_workspace_bytes(S, Hq, Hkv, D, max_seq_len, num_splits) if prefix_blocks is None else
              pa_decode_cascade_workspace_bytes(S, Hq, Hkv, D, max_seq_len, prefix_blocks, num_splits))
    ws, wsb = _workspace(nbytes, query.device, workspace)
    head = (_dev(out, "out"), _dev(_contig(query, "query"), "query"), _dev(key, "key"), _dev(value, "value"),
            key.stride(0), value.stride(0), _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
            _dev(block_tables, "block_tables"), block_tables.shape[1], _dev(seq_lens, "seq_lens"), S, Hq, Hkv, D, B,
            NB, max_seq_len)
    return out, head, (None if ws is None else ws.data_ptr(), wsb)


def pa_decode_write(query, key, value, key_cache, value_cache, block_tables, seq_lens, scale: float,
                    max_seq_len: int, num_splits: int = 0, out=None, workspace=None):
    """One decode step: stores key/value [S, Hkv, D] (row s: position seq_lens[s] - 1 of sequence s) into the
    pools and attends query [S, Hq, D] over the cache with them (fp32 or bf16 pools) -> out [S, Hq, D]."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=False)
    out, head, (ws, wsb) = _decode_write_args(query, key, value, key_cache, value_cache, block_tables, seq_lens,
                                              max_seq_len, num_splits, out, workspace)
    _check("pa_decode_write", lib.pa_decode_write(*head, float(scale), _dtype_code(key_cache), num_splits, ws, wsb,
                                                  _stream()))
    return out


def pa_decode_write_fp8(query, key, value, key_cache, value_cache, block_tables, seq_lens, scale: float,
                        k_scale: float, v_scale: float, max_seq_len: int, num_splits: int = 0, out=None,
                        workspace=None):
    """pa_decode_write over fp8 E4M3 pools (uint8 codes of x / scale) with per-tensor scales."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=True)
    out, head, (ws, wsb) = _decode_write_args(query, key, value, key_cache, value_cache, block_tables, seq_lens,
                                              max_seq_len, num_splits, out, workspace)
    _check("pa_decode_write_fp8", lib.pa_decode_write_fp8(*head, float(scale), _dtype_code(query), float(k_scale),
                                                          float(v_scale), num_splits, ws, wsb, _stream()))
    return out


def pa_decode_window_write(query, key, value, key_cache, value_cache, block_tables, seq_lens, scale: float,
                           max_seq_len: int, sliding_window: int, num_splits: int = 0, out=None, workspace=None):
    """pa_decode_write where each query sees its sequence's last sliding_window positions (pa_decode_window)."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=False)
    out, head, (ws, wsb) = _decode_write_args(query, key, value, key_cache, value_cache, block_tables, seq_lens,
                                              max_seq_len, num_splits, out, workspace)
    _check("pa_decode_window_write", lib.pa_decode_window_write(*head, float(scale), _dtype_code(key_cache),
                                                                sliding_window, num_splits, ws, wsb, _stream()))
    return out


def pa_decode_window_write_fp8(query, key, value, key_cache, value_cache, block_tables, seq_lens, scale: float,
                               k_scale: float, v_scale: float, max_seq_len: int, sliding_window: int,
                               num_splits: int = 0, out=None, workspace=None):
    """pa_decode_window_write over fp8 E4M3 pools."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=True)
    out, head, (ws, wsb) = _decode_write_args(query, key, value, key_cache, value_cache, block_tables, seq_lens,
                                              max_seq_len, num_splits, out, workspace)
    _check("pa_decode_window_write_fp8",
           lib.pa_decode_window_write_fp8(*head, float(scale), _dtype_code(query), float(k_scale), float(v_scale),
                                          sliding_window, num_splits, ws, wsb, _stream()))
    return out


def pa_decode_local_write(query, key, value, key_cache, value_cache, block_tables, seq_lens, scale: float,
                          max_seq_len: int, chunk_size: int, num_splits: int = 0, out=None, workspace=None):
    """pa_decode_write where each query sees the keys of its own chunk of chunk_size positions (pa_decode_local)."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=False)
    out, head, (ws, wsb) = _decode_write_args(query, key, value, key_cache, value_cache, block_tables, seq_lens,
                                              max_seq_len, num_splits, out, workspace)
    _check("pa_decode_local_write", lib.pa_decode_local_write(*head, float(scale), _dtype_code(key_cache), chunk_size,
                                                              num_splits, ws, wsb, _stream()))
    return out


def pa_decode_local_write_fp8(query, key, value, key_cache, value_cache, block_tables, seq_lens, scale: float,
                              k_scale: float, v_scale: float, max_seq_len: int, chunk_size: int,
                              num_splits: int = 0, out=None, workspace=None):
    """pa_decode_local_write over fp8 E4M3 pools."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=True)
    out, head, (ws, wsb) = _decode_write_args(query, key, value, key_cache, value_cache, block_tables, seq_lens,
                                              max_seq_len, num_splits, out, workspace)
    _check("pa_decode_local_write_fp8",
           lib.pa_decode_local_write_fp8(*head, float(scale), _dtype_code(query), float(k_scale), float(v_scale),
                                         chunk_size, num_splits, ws, wsb, _stream()))
    return out


def pa_decode_cascade_write(query, key, value, key_cache, value_cache, block_tables, seq_lens, scale: float,
                            max_seq_len: int, prefix_blocks: int, num_splits: int = 0, out=None, workspace=None):
    """pa_decode_write for a batch whose tables begin with the same prefix_blocks blocks (pa_decode_cascade)."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=False)
    out, head, (ws, wsb) = _decode_write_args(query, key, value, key_cache, value_cache, block_tables, seq_lens,
                                              max_seq_len, num_splits, out, workspace, prefix_blocks)
    _check("pa_decode_cascade_write", lib.pa_decode_cascade_write(*head, float(scale), _dtype_code(key_cache),
                                                                  prefix_blocks, num_splits, ws, wsb, _stream()))
    return out


def pa_decode_cascade_write_fp8(query, key, value, key_cache, value_cache, block_tables, seq_lens, scale: float,
                                k_scale: float, v_scale: float, max_seq_len: int, prefix_blocks: int,
                                num_splits: int = 0, out=None, workspace=None):
    """pa_decode_cascade_write over fp8 E4M3 pools (uint8 codes of x / scale)."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=True)
    out, head, (ws, wsb) = _decode_write_args(query, key, value, key_cache, value_cache, block_tables, seq_lens,
                                              max_seq_len, num_splits, out, workspace, prefix_blocks)
    _check("pa_decode_cascade_write_fp8",
           lib.pa_decode_cascade_write_fp8(*head, float(scale), _dtype_code(query), float(k_scale), float(v_scale),
                                           prefix_blocks, num_splits, ws, wsb, _stream()))
    return out


def pa_decode_window(query, key_cache, value_cache, block_tables, seq_lens, scale: float, max_seq_len: int,
                     sliding_window: int, num_splits: int = 0, out=None, workspace=None):
    """pa_decode where each query sees only its sequence's last sliding_window positions (bf16 pools)."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=False)
    S, Hq, D = query.shape
    NB, B, Hkv, _ = key_cache.shape
    out = torch.empty_like(query) if out is None else out
    ws, wsb = _workspace(pa_decode_workspace_bytes(S, Hq, Hkv, D, max_seq_len, num_splits), query.device, workspace)
    _check("pa_decode_window", lib.pa_decode_window(
        _dev(out, "out"), _dev(_contig(query, "query"), "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(seq_lens, "seq_lens"), S, Hq, Hkv, D, B, NB, max_seq_len, float(scale), _dtype_code(key_cache),
        sliding_window, num_splits, None if ws is None else ws.data_ptr(), wsb, _stream()))
    return out


def pa_decode_local(query, key_cache, value_cache, block_tables, seq_lens, scale: float, max_seq_len: int,
                    chunk_size: int, num_splits: int = 0, out=None, workspace=None):
    """pa_decode where each query sees only the keys of its own chunk of chunk_size positions (bf16 pools)."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=False)
    S, Hq, D = query.shape
    NB, B, Hkv, _ = key_cache.shape
    out = torch.empty_like(query) if out is None else out
    ws, wsb = _workspace(pa_decode_workspace_bytes(S, Hq, Hkv, D, max_seq_len, num_splits), query.device, workspace)
    _check("pa_decode_local", lib.pa_decode_local(
        _dev(out, "out"), _dev(_contig(query, "query"), "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(seq_lens, "seq_lens"), S, Hq, Hkv, D, B, NB, max_seq_len, float(scale), _dtype_code(key_cache),
        chunk_size, num_splits, None if ws is None else ws.data_ptr(), wsb, _stream()))
    return out


def pa_decode_cascade_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                                      max_seq_len: int, prefix_blocks: int, num_splits: int = 0) -> int:
    return int(load().pa_decode_cascade_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                                        prefix_blocks, num_splits))


def pa_decode_cascade(query, key_cache, value_cache, block_tables, seq_lens, scale: float, max_seq_len: int,
                      prefix_blocks: int, num_splits: int = 0, out=None, workspace=None):
    """pa_decode for sequences that all start with the same prefix_blocks physical blocks (bf16 pools)."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=False)
    S, Hq, D = query.shape
    NB, B, Hkv, _ = key_cache.shape
    out = torch.empty_like(query) if out is None else out
    need = pa_decode_cascade_workspace_bytes(S, Hq, Hkv, D, max_seq_len, prefix_blocks, num_splits)
    ws, wsb = _workspace(need, query.device, workspace)
    _check("pa_decode_cascade", lib.pa_decode_cascade(
        _dev(out, "out"), _dev(_contig(query, "query"), "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(seq_lens, "seq_lens"), S, Hq, Hkv, D, B, NB, max_seq_len, float(scale), _dtype_code(key_cache),
        prefix_blocks, num_splits, None if ws is None else ws.data_ptr(), wsb, _stream()))
    return out


def pa_decode_cascade_fp8(query, key_cache, value_cache, block_tables, seq_lens, scale: float, k_scale: float,
                          v_scale: float, max_seq_len: int, prefix_blocks: int, num_splits: int = 0, out=None,
                          workspace=None):
    """pa_decode_cascade over fp8 E4M3 pools (uint8 codes) with per-tensor scales."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=True)
    S, Hq, D = query.shape
    NB, B, Hkv, _ = key_cache.shape
    out = torch.empty_like(query) if out is None else out
    need = pa_decode_cascade_workspace_bytes(S, Hq, Hkv, D, max_seq_len, prefix_blocks, num_splits)
    ws, wsb = _workspace(need, query.device, workspace)
    _check("pa_decode_cascade_fp8", lib.pa_decode_cascade_fp8(
        _dev(out, "out"), _dev(_contig(query, "query"), "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(seq_lens, "seq_lens"), S, Hq, Hkv, D, B, NB, max_seq_len, float(scale), _dtype_code(query),
        float(k_scale), float(v_scale), prefix_blocks, num_splits, None if ws is None else ws.data_ptr(), wsb,
        _stream()))
    return out


def pa_prefill_varlen_workspace_bytes(query_start_loc_host, seq_lens_host, num_q_heads: int, num_kv_heads: int,
                                      head_dim: int) -> int:
    q = _i32_host(query_start_loc_host)
    s = _i32_host(seq_lens_host)
    return int(load().pa_prefill_varlen_workspace_bytes(q.data_ptr(), s.data_ptr(), s.numel(), num_q_heads,
                                                        num_kv_heads, head_dim))


def pa_prefill_varlen(query, key_cache, value_cache, block_tables, seq_lens, query_start_loc, seq_lens_host,
                      query_start_loc_host, scale: float, out=None, workspace=None):
    """Causal attention over a flattened batch of decode rows and prefill chunks: query [T, Hq, D]."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=False)
    T, Hq, D = query.shape
    NB, B, Hkv, _ = key_cache.shape
    qh = _i32_host(query_start_loc_host)
    sh = _i32_host(seq_lens_host)
    out = torch.empty_like(query) if out is None else out
    need = int(lib.pa_prefill_varlen_workspace_bytes(qh.data_ptr(), sh.data_ptr(), sh.numel(), Hq, Hkv, D))
    ws, wsb = _workspace(need, query.device, workspace)
    _check("pa_prefill_varlen", lib.pa_prefill_varlen(
        _dev(out, "out"), _dev(_contig(query, "query"), "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(seq_lens, "seq_lens"), _dev(query_start_loc, "query_start_loc"), sh.data_ptr(), qh.data_ptr(),
        sh.numel(), T, Hq, Hkv, D, B, NB, float(scale), _dtype_code(query), None if ws is None else ws.data_ptr(),
        wsb, _stream()))
    return out


def pa_prefill_varlen_write(query, key, value, key_cache, value_cache, block_tables, seq_lens, query_start_loc,
                            seq_lens_host, query_start_loc_host, scale: float, out=None, workspace=None):
    """One step of a flattened batch that also stores its new K/V: key/value [T, Hkv, D] (row t: the K/V of the
    batch's new row t), the bytes of pa_write_kv followed by pa_prefill_varlen."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=False)
    T, Hq, D = query.shape
    NB, B, Hkv, _ = key_cache.shape
    if tuple(key.shape) != (T, Hkv, D) or tuple(value.shape) != (T, Hkv, D):
        raise ValueError(f"key/value must be [{T}, {Hkv}, {D}] (one row per new token)")
    if key.dtype != query.dtype or value.dtype != query.dtype:
        raise ValueError("key/value must have the query's dtype")
    _check_kv_write(key, value, key_cache, value_cache, fp8=key_cache.dtype == torch.uint8)
    if key.stride(1) != D or key.stride(2) != 1 or value.stride(1) != D or value.stride(2) != 1:
        raise ValueError("heads and head_dim of key/value must be contiguous inside a token")
    qh = _i32_host(query_start_loc_host)
    sh = _i32_host(seq_lens_host)
    out = torch.empty_like(query) if out is None else out
    need = int(lib.pa_prefill_varlen_workspace_bytes(qh.data_ptr(), sh.data_ptr(), sh.numel(), Hq, Hkv, D))
    ws, wsb = _workspace(need, query.device, workspace)
    _check("pa_prefill_varlen_write", lib.pa_prefill_varlen_write(
        _dev(out, "out"), _dev(_contig(query, "query"), "query"), _dev(key, "key"), _dev(value, "value"),
        key.stride(0), value.stride(0), _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
        _dev(block_tables, "block_tables"), block_tables.shape[1], _dev(seq_lens, "seq_lens"),
        _dev(query_start_loc, "query_start_loc"), sh.data_ptr(), qh.data_ptr(), sh.numel(), T, Hq, Hkv, D, B, NB,
        float(scale), _dtype_code(query), None if ws is None else ws.data_ptr(), wsb, _stream()))
    return out


def pa_prefill_varlen_window_workspace_bytes(query_start_loc_host, seq_lens_host, num_q_heads: int,
                                             num_kv_heads: int, head_dim: int, sliding_window: int) -> int:
    q = _i32_host(query_start_loc_host)
    s = _i32_host(seq_lens_host)
    return int(load().pa_prefill_varlen_window_workspace_bytes(q.data_ptr(), s.data_ptr(), s.numel(), num_q_heads,
                                                               num_kv_heads, head_dim, sliding_window))


def pa_prefill_varlen_window(query, key_cache, value_cache, block_tables, seq_lens, query_start_loc, seq_lens_host,
                             query_start_loc_host, scale: float, sliding_window: int, out=None, workspace=None):
    """pa_prefill_varlen where the row at position p sees positions p-sliding_window+1 .. p (bf16)."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=False)
    T, Hq, D = query.shape
    NB, B, Hkv, _ = key_cache.shape
    qh = _i32_host(query_start_loc_host)
    sh = _i32_host(seq_lens_host)
    out = torch.empty_like(query) if out is None else out
    need = int(lib.pa_prefill_varlen_window_workspace_bytes(qh.data_ptr(), sh.data_ptr(), sh.numel(), Hq, Hkv, D,
                                                            sliding_window))
    ws, wsb = _workspace(need, query.device, workspace)
    _check("pa_prefill_varlen_window", lib.pa_prefill_varlen_window(
        _dev(out, "out"), _dev(_contig(query, "query"), "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(seq_lens, "seq_lens"), _dev(query_start_loc, "query_start_loc"), sh.data_ptr(), qh.data_ptr(),
        sh.numel(), T, Hq, Hkv, D, B, NB, float(scale), _dtype_code(query), sliding_window,
        None if ws is None else ws.data_ptr(), wsb, _stream()))
    return out


def pa_prefill_varlen_local_workspace_bytes(query_start_loc_host, seq_lens_host, num_q_heads: int,
                                            num_kv_heads: int, head_dim: int, chunk_size: int) -> int:
    q = _i32_host(query_start_loc_host)
    s = _i32_host(seq_lens_host)
    return int(load().pa_prefill_varlen_local_workspace_bytes(q.data_ptr(), s.data_ptr(), s.numel(), num_q_heads,
                                                              num_kv_heads, head_dim, chunk_size))


def pa_prefill_varlen_local(query, key_cache, value_cache, block_tables, seq_lens, query_start_loc, seq_lens_host,
                            query_start_loc_host, scale: float, chunk_size: int, out=None, workspace=None):
    """pa_prefill_varlen where the row at position p sees positions chunk_size*(p // chunk_size) .. p (bf16)."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=False)
    T, Hq, D = query.shape
    NB, B, Hkv, _ = key_cache.shape
    qh = _i32_host(query_start_loc_host)
    sh = _i32_host(seq_lens_host)
    out = torch.empty_like(query) if out is None else out
    need = int(lib.pa_prefill_varlen_local_workspace_bytes(qh.data_ptr(), sh.data_ptr(), sh.numel(), Hq, Hkv, D,
                                                           chunk_size))
    ws, wsb = _workspace(need, query.device, workspace)
    _check("pa_prefill_varlen_local", lib.pa_prefill_varlen_local(
        _dev(out, "out"), _dev(_contig(query, "query"), "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(seq_lens, "seq_lens"), _dev(query_start_loc, "query_start_loc"), sh.data_ptr(), qh.data_ptr(),
        sh.numel(), T, Hq, Hkv, D, B, NB, float(scale), _dtype_code(query), chunk_size,
        None if ws is None else ws.data_ptr(), wsb, _stream()))
    return out


def set_validate(on: int) -> None:
    """1: check device metadata on the host before every call (PA_VALIDATE's checks); 0: trust it; -1: follow the
    PA_VALIDATE environment variable."""
    _check("pa_set_validate", load().pa_set_validate(int(on)))


def set_fused(mode: int) -> None:
    """How a batch with decode rows and chunks runs: 0 two launches, 1 one launch when estimated faster (default),
    2 one launch whenever possible, -1 follow PA_FUSED."""
    _check("pa_set_fused", load().pa_set_fused(int(mode)))


def timing_enable(on: bool = True) -> None:
    """Library-side HIP events around every kernel launch (see pa_timing_enable)."""
    _check("pa_timing_enable", load().pa_timing_enable(1 if on else 0))


def timing_reset() -> None:
    _check("pa_timing_reset", load().pa_timing_reset())


def timing_read(kernel: str):
    """(launches timed, summed device milliseconds) of one kernel of the path."""
    n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
    _check("pa_timing_read", load().pa_timing_read(KERNELS[kernel], ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)


def timing_launches(kernel: str) -> list:
    """Device milliseconds of each timed launch of one kernel since the last reset, in launch order."""
    lib = load()
    n = ctypes.c_int32(0)
    _check("pa_timing_read_launches", lib.pa_timing_read_launches(KERNELS[kernel], None, 0, ctypes.byref(n)))
    buf = (ctypes.c_float * max(n.value, 1))()
    _check("pa_timing_read_launches", lib.pa_timing_read_launches(KERNELS[kernel], buf, n.value, ctypes.byref(n)))
    return [float(buf[i]) for i in range(n.value)]


def pa_prefill_varlen_fp8_workspace_bytes(query_start_loc_host, seq_lens_host, num_q_heads: int, num_kv_heads: int,
                                          head_dim: int, bt_stride: int) -> int:
    q = _i32_host(query_start_loc_host)
    s = _i32_host(seq_lens_host)
    return int(load().pa_prefill_varlen_fp8_workspace_bytes(q.data_ptr(), s.data_ptr(), s.numel(), num_q_heads,
                                                            num_kv_heads, head_dim, bt_stride))


def pa_prefill_varlen_fp8(query, key_cache, value_cache, block_tables, seq_lens, query_start_loc, seq_lens_host,
                          query_start_loc_host, scale: float, k_scale: float, v_scale: float, out=None,
                          workspace=None):
    """pa_prefill_varlen over fp8 E4M3 pools (uint8 codes) with per-tensor scales."""
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=True)
    T, Hq, D = query.shape
    NB, B, Hkv, _ = key_cache.shape
    qh = _i32_host(query_start_loc_host)
    sh = _i32_host(seq_lens_host)
    out = torch.empty_like(query) if out is None else out
    need = int(lib.pa_prefill_varlen_fp8_workspace_bytes(qh.data_ptr(), sh.data_ptr(), sh.numel(), Hq, Hkv, D,
                                                         block_tables.shape[1]))
    ws, wsb = _workspace(need, query.device, workspace)
    _check("pa_prefill_varlen_fp8", lib.pa_prefill_varlen_fp8(
        _dev(out, "out"), _dev(_contig(query, "query"), "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(seq_lens, "seq_lens"), _dev(query_start_loc, "query_start_loc"), sh.data_ptr(), qh.data_ptr(),
        sh.numel(), T, Hq, Hkv, D, B, NB, float(scale), _dtype_code(query), float(k_scale), float(v_scale),
        None if ws is None else ws.data_ptr(), wsb, _stream()))
    return out


def _decode_fp8_masked(name, query, key_cache, value_cache, block_tables, seq_lens, scale, k_scale, v_scale,
                       max_seq_len, size, num_splits, out, workspace):
    lib = load()
    S, Hq, D = query.shape
    NB, B, Hkv, _ = key_cache.shape
    out = torch.empty_like(query) if out is None else out
    ws, wsb = _workspace(pa_decode_workspace_bytes(S, Hq, Hkv, D, max_seq_len, num_splits), query.device, workspace)
    _check(name, getattr(lib, name)(
        _dev(out, "out"), _dev(_contig(query, "query"), "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(seq_lens, "seq_lens"), S, Hq, Hkv, D, B, NB, max_seq_len, float(scale), _dtype_code(query),
        float(k_scale), float(v_scale), size, num_splits, None if ws is None else ws.data_ptr(), wsb, _stream()))
    return out


def pa_decode_window_fp8(query, key_cache, value_cache, block_tables, seq_lens, scale: float, k_scale: float,
                         v_scale: float, max_seq_len: int, sliding_window: int, num_splits: int = 0, out=None,
                         workspace=None):
    """pa_decode_window over fp8 E4M3 pools (uint8 codes) with per-tensor scales."""
    return _decode_fp8_masked("pa_decode_window_fp8", query, key_cache, value_cache, block_tables, seq_lens, scale,
                              k_scale, v_scale, max_seq_len, sliding_window, num_splits, out, workspace)


def pa_decode_local_fp8(query, key_cache, value_cache, block_tables, seq_lens, scale: float, k_scale: float,
                        v_scale: float, max_seq_len: int, chunk_size: int, num_splits: int = 0, out=None,
                        workspace=None):
    """pa_decode_local over fp8 E4M3 pools (uint8 codes) with per-tensor scales."""
    return _decode_fp8_masked("pa_decode_local_fp8", query, key_cache, value_cache, block_tables, seq_lens, scale,
                              k_scale, v_scale, max_seq_len, chunk_size, num_splits, out, workspace)


def _prefill_fp8_masked(name, query, key_cache, value_cache, block_tables, seq_lens, query_start_loc, seq_lens_host,
                        query_start_loc_host, scale, k_scale, v_scale, size, out, workspace):
    lib = load()
    _check_pools(query, key_cache, value_cache, fp8=True)
    T, Hq, D = query.shape
    NB, B, Hkv, _ = key_cache.shape
    qh = _i32_host(query_start_loc_host)
    sh = _i32_host(seq_lens_host)
    out = torch.empty_like(query) if out is None else out
    need = int(getattr(lib, name + "_workspace_bytes")(qh.data_ptr(), sh.data_ptr(), sh.numel(), Hq, Hkv, D,
                                                       block_tables.shape[1], size))
    ws, wsb = _workspace(need, query.device, workspace)
    _check(name, getattr(lib, name)(
        _dev(out, "out"), _dev(_contig(query, "query"), "query"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(block_tables, "block_tables"), block_tables.shape[1],
        _dev(seq_lens, "seq_lens"), _dev(query_start_loc, "query_start_loc"), sh.data_ptr(), qh.data_ptr(),
        sh.numel(), T, Hq, Hkv, D, B, NB, float(scale), _dtype_code(query), float(k_scale), float(v_scale), size,
        None if ws is None else ws.data_ptr(), wsb, _stream()))
    return out


def pa_prefill_varlen_window_fp8(query, key_cache, value_cache, block_tables, seq_lens, query_start_loc,
                                 seq_lens_host, query_start_loc_host, scale: float, k_scale: float, v_scale: float,
                                 sliding_window: int, out=None, workspace=None):
    """pa_prefill_varlen_window over fp8 E4M3 pools (uint8 codes) with per-tensor scales."""
    return _prefill_fp8_masked("pa_prefill_varlen_window_fp8", query, key_cache, value_cache, block_tables, seq_lens,
                               query_start_loc, seq_lens_host, query_start_loc_host, scale, k_scale, v_scale,
                               sliding_window, out, workspace)


def pa_prefill_varlen_local_fp8(query, key_cache, value_cache, block_tables, seq_lens, query_start_loc,
                                seq_lens_host, query_start_loc_host, scale: float, k_scale: float, v_scale: float,
                                chunk_size: int, out=None, workspace=None):
    """pa_prefill_varlen_local over fp8 E4M3 pools (uint8 codes) with per-tensor scales."""
    return _prefill_fp8_masked("pa_prefill_varlen_local_fp8", query, key_cache, value_cache, block_tables, seq_lens,
                               query_start_loc, seq_lens_host, query_start_loc_host, scale, k_scale, v_scale,
                               chunk_size, out, workspace)


# ---- host block pool (pa_pool_*)

def _np_i32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def pool_hash_blocks(tokens, block_size: int = 16, extra_key: int = 0) -> np.ndarray:
    """Chained hashes of the full blocks of a token sequence (uint64)."""
    t = _np_i32(tokens)
    out = np.zeros(max(len(t) // block_size, 1), dtype=np.uint64)
    n = load().pa_pool_hash_blocks(t.ctypes.data, len(t), block_size, ctypes.c_uint64(extra_key), out.ctypes.data)
    if n < 0:
        raise ValueError("pa_pool_hash_blocks: invalid arguments")
    return out[:n]


class BlockPool:
    """The library's host block pool (block 0 is the null block)."""

    def __init__(self, num_blocks: int, block_size: int = 16):
        self._lib = load()
        h = ctypes.c_void_p()
        _check("pa_pool_create", self._lib.pa_pool_create(num_blocks, block_size, ctypes.byref(h)))
        self._h = h
        self.num_blocks, self.block_size = num_blocks, block_size

    def close(self):
        if self._h:
            self._lib.pa_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_free(self) -> int:
        return int(self._lib.pa_pool_num_free(self._h))

    def find_longest_cache_hit(self, hashes) -> list:
        hs = np.ascontiguousarray(np.asarray(hashes, dtype=np.uint64))
        out = np.zeros(max(len(hs), 1), dtype=np.int32)
        n = self._lib.pa_pool_find_longest_cache_hit(self._h, hs.ctypes.data, len(hs), out.ctypes.data)
        return out[:n].tolist()

    def allocate_slots(self, request_id: int, num_tokens: int, hit_blocks=()) -> int:
        hb = _np_i32(list(hit_blocks))
        n = ctypes.c_int32(0)
        _check("pa_pool_allocate_slots", self._lib.pa_pool_allocate_slots(
            self._h, request_id, num_tokens, hb.ctypes.data if len(hb) else None, len(hb), ctypes.byref(n)))
        return int(n.value)

    def cache_blocks(self, request_id: int, hashes, num_full_blocks: int) -> None:
        hs = np.ascontiguousarray(np.asarray(hashes, dtype=np.uint64))
        _check("pa_pool_cache_blocks", self._lib.pa_pool_cache_blocks(
            self._h, request_id, hs.ctypes.data if len(hs) else None, num_full_blocks))

    def release_before(self, request_id: int, position: int) -> None:
        _check("pa_pool_release_before", self._lib.pa_pool_release_before(self._h, request_id, position))

    def free(self, request_id: int) -> None:
        _check("pa_pool_free", self._lib.pa_pool_free(self._h, request_id))

    def block_table(self, request_id: int) -> list:
        n = self._lib.pa_pool_block_table(self._h, request_id, None, 0)
        if n < 0:
            raise KeyError(request_id)
        out = np.zeros(max(n, 1), dtype=np.int32)
        self._lib.pa_pool_block_table(self._h, request_id, out.ctypes.data, n)
        return out[:n].tolist()

    def block_state(self, block: int):
        """(ref_count, is_free, hash or None) of one block."""
        r, f, hh = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        h = ctypes.c_uint64()
        _check("pa_pool_block_state", self._lib.pa_pool_block_state(self._h, block, ctypes.byref(r), ctypes.byref(f),
                                                                     ctypes.byref(hh), ctypes.byref(h)))
        return int(r.value), bool(f.value), (int(h.value) if hh.value else None)

    def free_queue(self) -> list:
        n = self._lib.pa_pool_free_queue(self._h, None, 0)
        out = np.zeros(max(n, 1), dtype=np.int32)
        self._lib.pa_pool_free_queue(self._h, out.ctypes.data, n)
        return out[:n].tolist()


def probe_mfma_peak(blocks: int = 512, iters: int = 20000, reps: int = 3) -> float:
    """Measured bf16 matrix-core rate (TFLOP/s) of v_mfma_f32_32x32x16_bf16 on this GPU (best of reps)."""
    lib = load()
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    best = None
    for _ in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _check("pa_probe_mfma_peak", lib.pa_probe_mfma_peak(out.data_ptr(), blocks, iters, _stream()))
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    flop = blocks * 4 * iters * 4 * 32768.0
    return flop / (best * 1e-3) / 1e12
