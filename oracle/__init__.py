"""CPU oracle for paged-KV attention (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  It shares no code with the HIP library and the
product path never reaches it.

* :func:`attention`, :func:`slot_mapping`, :func:`reshape_and_cache`,
  :func:`reshape_and_cache_fp8`, :func:`fp8_encode`, :func:`fp8_decode` call the
  fp64 C implementation in ``pa_oracle.c`` (built on first use with gcc).
* :mod:`oracle.brute` is an independent pure-Python evaluation for tiny inputs.
* :mod:`oracle.fp8_ref` is an independent pure-Python E4M3 codec.
* :func:`blocks_needed` is the allocation arithmetic (ceil(n / block_size)).

Sources: the page "vLLM 架构概述" §2 (block pool, per-request int32 block
tables, lookup plus address arithmetic); the page "vLLM：从 KV Cache 到高吞吐推理
服务", tutorial 3 (logical/physical block, offset, slot) and tutorial 1 (head
sharing in MHA/GQA/MQA); the reading note on "Inside vLLM", core point 1
(16-token blocks, ceil allocation, the block-bytes formula) and core point 2
(flattened super-sequence with per-sequence masking).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16, FP8 = 0, 1, 2
_KIND = {"f32": F32, "bf16": BF16, "fp8": FP8}


def build(force: bool = False) -> str:
    """Compiles pa_oracle.c into liboracle.so (gcc, fp64, no contraction, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
                        "-shared", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # ORACLE_LIBRARY names another build of pa_oracle.c (the AddressSanitizer build)
            path = os.environ.get("ORACLE_LIBRARY") or build()
            lib = ctypes.CDLL(path)
            P = ctypes.c_void_p
            i32, i64, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
            lib.oracle_fp8_decode.argtypes = [ctypes.c_uint8]
            lib.oracle_fp8_decode.restype = f64
            lib.oracle_fp8_encode.argtypes = [f32]
            lib.oracle_fp8_encode.restype = ctypes.c_uint8
            lib.oracle_slot_mapping.argtypes = [P, P, i32, P, P, i32, i32]
            lib.oracle_reshape_and_cache.argtypes = [P, P, i64, i64, P, P, P, i32, i32, i32, i32, i32, i32]
            lib.oracle_reshape_and_cache_fp8.argtypes = [P, P, i64, i64, P, P, P, i32, i32, i32, i32, i32,
                                                         i32, f32, f32]
            lib.oracle_attention.argtypes = [P, P, i32, P, P, i32, f64, f64, P, i32, P, P, i32, i32, i32,
                                             i32, i32, f32, P, i32]
            lib.oracle_attention_window.argtypes = [P, P, i32, P, P, i32, f64, f64, P, i32, P, P, i32, i32,
                                                    i32, i32, i32, f32, P, i32, i32]
            lib.oracle_attention_local.argtypes = [P, P, i32, P, P, i32, f64, f64, P, i32, P, P, i32, i32,
                                                   i32, i32, i32, f32, P, i32, i32]
            lib.oracle_num_threads.restype = i32
            lib.oracle_set_threads.argtypes = [i32]
            _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def _np(x) -> np.ndarray:
    """Host array view of a CPU tensor / array; bf16 is viewed as its uint16 bits."""
    if isinstance(x, torch.Tensor):
        assert x.device.type == "cpu"
        x = x.contiguous()
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).numpy().view(np.uint16)
        return x.numpy()
    return np.ascontiguousarray(x)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _kind_of(x) -> int:
    if isinstance(x, torch.Tensor):
        return {torch.float32: F32, torch.bfloat16: BF16, torch.uint8: FP8}[x.dtype]
    return {np.dtype(np.float32): F32, np.dtype(np.uint16): BF16, np.dtype(np.uint8): FP8}[x.dtype]


def blocks_needed(num_tokens: int, block_size: int = 16) -> int:
    """Blocks a request of num_tokens needs: ceil(num_tokens / block_size)."""
    return -(-int(num_tokens) // int(block_size))


def fp8_decode(code: int) -> float:
    return float(_load().oracle_fp8_decode(int(code) & 0xFF))


def fp8_encode(x: float) -> int:
    return int(_load().oracle_fp8_encode(float(x)))


def fp8_encode_array(x: np.ndarray) -> np.ndarray:
    f = np.vectorize(lambda v: _load().oracle_fp8_encode(float(v)), otypes=[np.uint8])
    return f(np.asarray(x, dtype=np.float32))


def slot_mapping(block_tables, seq_lens, query_start_loc, block_size: int = 16) -> np.ndarray:
    bt = _np(block_tables).astype(np.int32, copy=False)
    sl = _np(seq_lens).astype(np.int32, copy=False)
    qsl = _np(query_start_loc).astype(np.int32, copy=False)
    out = np.empty(int(qsl[-1]), dtype=np.int32)
    rc = _load().oracle_slot_mapping(_ptr(out), _ptr(bt), bt.shape[1], _ptr(sl), _ptr(qsl),
                                     sl.shape[0], block_size)
    assert rc == 0
    return out


def reshape_and_cache(key, value, key_cache, value_cache, slots) -> None:
    """Writes key/value [T, Hkv, D] into the pools (torch CPU tensors, modified in place)."""
    assert key_cache.is_contiguous() and value_cache.is_contiguous()
    k, v = _np(key), _np(value)
    kc, vc = _np(key_cache), _np(value_cache)   # views share memory with the tensors
    sm = _np(slots).astype(np.int32, copy=False)
    NB, B, H, D = key_cache.shape
    T = k.shape[0]
    elem = k.dtype.itemsize
    rc = _load().oracle_reshape_and_cache(_ptr(k), _ptr(v), H * D, H * D, _ptr(kc), _ptr(vc), _ptr(sm),
                                          T, H, D, B, NB, elem)
    assert rc == 0


def reshape_and_cache_fp8(key, value, key_cache, value_cache, slots, k_scale: float, v_scale: float) -> None:
    k, v = _np(key), _np(value)
    kc, vc = _np(key_cache), _np(value_cache)
    assert kc.dtype == np.uint8
    sm = _np(slots).astype(np.int32, copy=False)
    NB, B, H, D = key_cache.shape
    rc = _load().oracle_reshape_and_cache_fp8(_ptr(k), _ptr(v), H * D, H * D, _ptr(kc), _ptr(vc), _ptr(sm),
                                              k.shape[0], H, D, B, NB, _kind_of(key), float(k_scale),
                                              float(v_scale))
    assert rc == 0


def attention(query, key_cache, value_cache, block_tables, seq_lens, query_start_loc, scale: float,
              k_scale: float = 1.0, v_scale: float = 1.0, rows=None, window: int = 0,
              chunk: int = 0) -> np.ndarray:
    """fp64 attention output [n_rows, Hq, D] for the given query rows (all rows when None).

    window > 0: sliding window, the row at position p sees keys max(0, p - window + 1) .. p.
    chunk > 0: chunked local attention, the row at position p sees keys p - p % chunk .. p."""
    assert not (window and chunk)
    q = _np(query)
    kc, vc = _np(key_cache), _np(value_cache)
    bt = _np(block_tables).astype(np.int32, copy=False)
    sl = _np(seq_lens).astype(np.int32, copy=False)
    qsl = _np(query_start_loc).astype(np.int32, copy=False)
    T, Hq, D = q.shape
    NB, B, Hkv, D2 = kc.shape
    assert D == D2
    if rows is None:
        n_rows = T
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        n_rows = rows_arr.shape[0]
    out = np.empty((n_rows, Hq, D), dtype=np.float64)
    fn, arg = (_load().oracle_attention_local, int(chunk)) if chunk else (_load().oracle_attention_window, int(window))
    rc = fn(_ptr(out), _ptr(q), _kind_of(query), _ptr(kc), _ptr(vc), _kind_of(key_cache), float(k_scale),
            float(v_scale), _ptr(bt), bt.shape[1], _ptr(sl), _ptr(qsl), sl.shape[0], Hq, Hkv, D, B, float(scale),
            None if rows_arr is None else _ptr(rows_arr), n_rows, arg)
    assert rc == 0
    return out


def attention_for(w, rows=None, pools=None, window: int = 0, chunk: int = 0) -> np.ndarray:
    """attention() on a workload's arrays; pools = (k_cache, v_cache) after the new tokens were written."""
    kc, vc = pools if pools is not None else (w.k_cache, w.v_cache)
    return attention(w.query, kc, vc, w.block_tables, w.seq_lens, w.query_start_loc, w.scale,
                     w.k_scale, w.v_scale, rows=rows, window=window, chunk=chunk)


def written_pools(w):
    """Copies of a workload's pools with its new tokens written through the oracle's slot mapping."""
    kc, vc = w.copy_pools()
    slots = slot_mapping(w.block_tables, w.seq_lens, w.query_start_loc, w.block_size)
    if w.kv_dtype == "fp8":
        reshape_and_cache_fp8(w.new_k, w.new_v, kc, vc, slots, w.k_scale, w.v_scale)
    else:
        reshape_and_cache(w.new_k, w.new_v, kc, vc, slots)
    return kc, vc
