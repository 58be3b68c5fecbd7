"""CPU oracle for paged KV-cache attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does.

The arithmetic lives in ``pa_oracle.c`` (plain C, double precision); this
module only compiles it with gcc and marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, FP8 = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile pa_oracle.c into liboracle.so next to it (gcc -O2, pthreads)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, dbl, flt = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_float
        lib.oracle_fp8_value.argtypes = [ctypes.c_uint8]
        lib.oracle_fp8_value.restype = dbl
        lib.oracle_fp8_encode.argtypes = [flt]
        lib.oracle_fp8_encode.restype = ctypes.c_uint8
        lib.oracle_fp8_quantize.argtypes = [flt, flt]
        lib.oracle_fp8_quantize.restype = ctypes.c_uint8
        lib.oracle_reshape_and_cache.argtypes = [P, P, P, P, P, i64, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_int, flt]
        lib.oracle_reshape_and_cache.restype = None
        lib.oracle_copy_blocks.argtypes = [P, P, P, i64, i64, i64]
        lib.oracle_copy_blocks.restype = None
        lib.oracle_swap_blocks.argtypes = [P, P, i64, P, P, i64, P, i64, i64]
        lib.oracle_swap_blocks.restype = None
        lib.oracle_decode.argtypes = [P, P, ctypes.c_int, P, P, ctypes.c_int, dbl, P, i32, P,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, dbl, P, P, i64,
                                      ctypes.c_int, ctypes.c_int]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_prefill.argtypes = [P, P, ctypes.c_int, P, P, ctypes.c_int, dbl, P, i32, P, P,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, dbl,
                                       P, P, i64, ctypes.c_int, ctypes.c_int]
        lib.oracle_prefill.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    """Storage code of an array: float32 -> F32, uint16 (bf16 bits) -> BF16, uint8 -> FP8."""
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return FP8
    raise TypeError(f"unsupported oracle storage dtype {a.dtype}")


def default_threads() -> int:
    return os.cpu_count() or 1


def fp8_value(code: int) -> float:
    return _load().oracle_fp8_value(int(code))


def fp8_encode(y: float) -> int:
    return int(_load().oracle_fp8_encode(float(y)))


def fp8_quantize(x: float, kv_scale: float) -> int:
    return int(_load().oracle_fp8_quantize(float(x), float(kv_scale)))


def reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, kv_scale: float = 1.0) -> None:
    """Write k/v ([T, Hkv, d]) into host pools ([slots, Hkv, d]) in place."""
    slot_mapping = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    T, hkv, d = k.shape
    assert v.shape == k.shape and k_cache.shape[1:] == (hkv, d) and v_cache.shape == k_cache.shape
    assert slot_mapping.shape == (T,)
    _load().oracle_reshape_and_cache(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(slot_mapping), T, _dtype_code(k),
                                     _dtype_code(k_cache), hkv, d, float(kv_scale))


def copy_blocks(k_cache, v_cache, pairs, block_size: int = 16) -> None:
    """Copy-on-write of whole blocks in host pools ([slots, Hkv, d],
    block_size slots per block), in place: for each (src, dst) row of
    ``pairs``, in order, block dst of both pools becomes a copy of block src."""
    pairs = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
    assert v_cache.shape == k_cache.shape and v_cache.dtype == k_cache.dtype
    assert k_cache.shape[0] % block_size == 0
    block_bytes = block_size * k_cache.shape[1] * k_cache.shape[2] * k_cache.itemsize
    _load().oracle_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(pairs), pairs.shape[0],
                               k_cache.shape[0] // block_size, block_bytes)


def swap_blocks(src_k, src_v, dst_k, dst_v, pairs, block_size: int = 16) -> None:
    """Block moves between two host pool pairs ([slots, Hkv, d], block_size
    slots per block): for each (src, dst) row of ``pairs``, in order, block
    dst of the destination pools becomes a copy of block src of the source
    pools."""
    pairs = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
    assert src_k.shape[1:] == dst_k.shape[1:] and src_k.dtype == dst_k.dtype
    assert src_v.shape == src_k.shape and dst_v.shape == dst_k.shape
    block_bytes = block_size * src_k.shape[1] * src_k.shape[2] * src_k.itemsize
    _load().oracle_swap_blocks(_ptr(src_k), _ptr(src_v), src_k.shape[0] // block_size, _ptr(dst_k),
                               _ptr(dst_v), dst_k.shape[0] // block_size, _ptr(pairs), pairs.shape[0],
                               block_bytes)


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, kv_scale=1.0,
           sel_seq=None, sel_head=None, num_threads=None, block_size: int = 16):
    """Decode attention for (seq, head) pairs; returns float64 [n_sel, d].

    q: [S, Hq, d] float32 or uint16 (bf16 bits); pools: [slots, Hkv, d].
    Without a selection every (seq, head) pair is computed, returned as [S, Hq, d].
    """
    S, hq, d = q.shape
    hkv = k_cache.shape[1]
    kv_scale = float(np.float32(kv_scale))  # the scale is an fp32 value in the C ABI
    full = sel_seq is None
    if full:
        sel_seq = np.repeat(np.arange(S, dtype=np.int32), hq)
        sel_head = np.tile(np.arange(hq, dtype=np.int32), S)
    sel_seq = np.ascontiguousarray(sel_seq, dtype=np.int32)
    sel_head = np.ascontiguousarray(sel_head, dtype=np.int32)
    block_tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    out = np.zeros((len(sel_seq), d), dtype=np.float64)
    rc = _load().oracle_decode(_ptr(out), _ptr(q), _dtype_code(q), _ptr(k_cache), _ptr(v_cache),
                               _dtype_code(k_cache), float(kv_scale), _ptr(block_tables),
                               block_tables.shape[1], _ptr(context_lens), hq, hkv, d,
                               float(scale), _ptr(sel_seq), _ptr(sel_head), len(sel_seq),
                               num_threads or default_threads(), int(block_size))
    if rc != 0:
        raise ValueError(f"oracle_decode failed ({rc})")
    return out.reshape(S, hq, d) if full else out


def prefill(q, k_cache, v_cache, block_tables, query_start, context_lens, scale, kv_scale=1.0,
            sel_row=None, sel_head=None, num_threads=None, block_size: int = 16):
    """Chunked-prefill attention for (row, head) pairs; returns float64 [n_sel, d]."""
    Tq, hq, d = q.shape
    hkv = k_cache.shape[1]
    kv_scale = float(np.float32(kv_scale))  # the scale is an fp32 value in the C ABI
    full = sel_row is None
    if full:
        sel_row = np.repeat(np.arange(Tq, dtype=np.int32), hq)
        sel_head = np.tile(np.arange(hq, dtype=np.int32), Tq)
    sel_row = np.ascontiguousarray(sel_row, dtype=np.int32)
    sel_head = np.ascontiguousarray(sel_head, dtype=np.int32)
    block_tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    query_start = np.ascontiguousarray(query_start, dtype=np.int32)
    context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    out = np.zeros((len(sel_row), d), dtype=np.float64)
    rc = _load().oracle_prefill(_ptr(out), _ptr(q), _dtype_code(q), _ptr(k_cache), _ptr(v_cache),
                                _dtype_code(k_cache), float(kv_scale), _ptr(block_tables),
                                block_tables.shape[1], _ptr(query_start), _ptr(context_lens),
                                len(context_lens), hq, hkv, d, float(scale), _ptr(sel_row),
                                _ptr(sel_head), len(sel_row), num_threads or default_threads(),
                                int(block_size))
    if rc != 0:
        raise ValueError(f"oracle_prefill failed ({rc})")
    return out.reshape(Tq, hq, d) if full else out
