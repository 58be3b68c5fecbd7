"""Thin Python binding of libpa's C ABI (include/pa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libpa.so.  Tensors are torch CUDA tensors (device memory and the
current stream come from PyTorch); they are passed to the library as raw
device pointers.  There is no CPU fallback: if libpa.so is missing or a call
fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_OK, PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = range(5)
PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2

_DTYPES = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.float8_e4m3fn: PA_FP8_E4M3}


class PAShape(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("cache_dtype", ctypes.c_int32),
        ("kv_scale", ctypes.c_float),
        ("partition_tokens", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
    ]


class PAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"libpa status {status}: {detail}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree libpa.so (built by paged_kv_cache_157_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m paged_kv_cache_157_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, S = ctypes.c_void_p, ctypes.POINTER(PAShape)
        i32, i64, f32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        lib.pa_reshape_and_cache.argtypes = [P, P, P, P, P, i64, i32, S, P]
        lib.pa_reshape_and_cache.restype = ctypes.c_int
        lib.pa_decode_workspace_bytes.argtypes = [S]
        lib.pa_decode_workspace_bytes.restype = sz
        lib.pa_decode.argtypes = [P, P, P, P, P, P, f32, S, P, sz, P]
        lib.pa_decode.restype = ctypes.c_int
        lib.pa_decode_static.argtypes = [P, P, P, P, P, P, f32, S, P]
        lib.pa_decode_static.restype = ctypes.c_int
        lib.pa_prefill_workspace_bytes.argtypes = [S, i64]
        lib.pa_prefill_workspace_bytes.restype = sz
        lib.pa_prefill_chunk.argtypes = [P, P, P, P, P, P, P, i64, f32, S, P, sz, P]
        lib.pa_prefill_chunk.restype = ctypes.c_int
        lib.pa_copy_blocks.argtypes = [P, P, P, i64, S, P]
        lib.pa_copy_blocks.restype = ctypes.c_int
        lib.pa_swap_blocks.argtypes = [P, P, i64, P, P, i64, P, i64, S, P]
        lib.pa_swap_blocks.restype = ctypes.c_int
        lib.pa_status_string.argtypes = [ctypes.c_int]
        lib.pa_status_string.restype = ctypes.c_char_p
        lib.pa_last_error.argtypes = []
        lib.pa_last_error.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _check(status: int) -> None:
    if status != PA_OK:
        lib = load()
        raise PAError(status, f"{lib.pa_status_string(status).decode()}: "
                              f"{lib.pa_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(t: torch.Tensor, name: str, device: torch.device, dtype=None, ndim=None):
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a CUDA tensor on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, has {t.dim()}")


def make_shape(q_heads: int, k_cache: torch.Tensor, q_dtype: torch.dtype, num_seqs: int,
               max_blocks: int, kv_scale: float = 1.0, partition_tokens: int = 0) -> PAShape:
    if k_cache.dim() != 4 or k_cache.shape[1] not in (8, 16, 32, 64):
        raise ValueError("KV pools must be [num_blocks, block_size, num_kv_heads, head_dim] "
                         "with block_size 8, 16, 32 or 64")
    if k_cache.dtype not in _DTYPES or q_dtype not in _DTYPES:
        raise ValueError(f"unsupported dtypes {q_dtype} / {k_cache.dtype}")
    return PAShape(num_seqs=num_seqs, num_q_heads=q_heads, num_kv_heads=k_cache.shape[2],
                   head_dim=k_cache.shape[3], num_blocks=k_cache.shape[0],
                   max_blocks_per_seq=max_blocks, q_dtype=_DTYPES[q_dtype],
                   cache_dtype=_DTYPES[k_cache.dtype], kv_scale=float(kv_scale),
                   partition_tokens=int(partition_tokens), block_size=k_cache.shape[1])


_workspaces: Dict[Tuple[int, int, str], torch.Tensor] = {}


def _workspace(device: torch.device, nbytes: int, op: str) -> Optional[torch.Tensor]:
    """Scratch buffer of one entry point, reused across its calls on one
    stream of a device.

    Calls on one stream run in order, so they can share a buffer; calls on
    different streams may run at the same time and would race on the decode's
    arrival counters and partial results, so every stream gets its own
    buffer.  The buffer is allocated (zero-filled: pa_decode's arrival
    counters must start at zero, and every call leaves them zero again) while
    that stream is current, so the caching allocator ties it to that stream;
    a buffer replaced by a larger one is released in that stream's order, after
    the calls already queued on it."""
    if nbytes == 0:
        return None
    dev = device.index if device.index is not None else torch.cuda.current_device()
    key = (dev, torch.cuda.current_stream(device).cuda_stream, op)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def workspace_of(op: str, device: Optional[torch.device] = None) -> Optional[torch.Tensor]:
    """The buffer the current stream of `device` uses for `op` ("decode" or
    "prefill"), or None before its first call."""
    device = device or torch.device("cuda", torch.cuda.current_device())
    dev = device.index if device.index is not None else torch.cuda.current_device()
    return _workspaces.get((dev, torch.cuda.current_stream(device).cuda_stream, op))


def reshape_and_cache(k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, slot_mapping: torch.Tensor,
                      kv_scale: float = 1.0) -> None:
    """pa_reshape_and_cache: write k/v rows [T, Hkv, d] into the pools' slots."""
    dev = k_cache.device
    for name, t in (("k", k), ("v", v), ("k_cache", k_cache), ("v_cache", v_cache)):
        _require(t, name, dev)
    _require(slot_mapping, "slot_mapping", dev, torch.int64, 1)
    if k.shape != v.shape or k.dim() != 3 or k.shape[0] != slot_mapping.shape[0]:
        raise ValueError("k, v must be [T, Hkv, d] with T = len(slot_mapping)")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must match")
    if tuple(k.shape[1:]) != tuple(k_cache.shape[2:]):
        raise ValueError("k rows do not match the pool's [Hkv, d]")
    shape = make_shape(k.shape[1], k_cache, k.dtype, 0, 1, kv_scale)
    lib = load()
    _check(lib.pa_reshape_and_cache(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(slot_mapping), k.shape[0], _DTYPES[k.dtype],
                                    ctypes.byref(shape), _stream(dev)))


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, block_pairs: torch.Tensor) -> None:
    """pa_copy_blocks: k_cache[dst] = k_cache[src], v_cache[dst] = v_cache[src] for
    every (src, dst) row of block_pairs ([n, 2] int64 on the pools' device)."""
    dev = k_cache.device
    _require(k_cache, "k_cache", dev)
    _require(v_cache, "v_cache", dev)
    _require(block_pairs, "block_pairs", dev, torch.int64, 2)
    if block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [n, 2] (src, dst)")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must match")
    q_dtype = torch.float32 if k_cache.dtype == torch.float32 else torch.bfloat16
    shape = make_shape(k_cache.shape[2], k_cache, q_dtype, 0, 1)
    _check(load().pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(block_pairs),
                                 block_pairs.shape[0], ctypes.byref(shape), _stream(dev)))


def swap_blocks(src_k: torch.Tensor, src_v: torch.Tensor, dst_k: torch.Tensor,
                dst_v: torch.Tensor, block_pairs: torch.Tensor,
                device: Optional[torch.device] = None) -> None:
    """pa_swap_blocks: dst[dst_id] = src[src_id] for every (src_id, dst_id) row of
    block_pairs, between pools on the GPU and pools in pinned host memory (any
    mix).  Runs on the current stream of ``device`` (default: the CUDA device of
    whichever argument is on one, else the current device)."""
    ts = (("src_k", src_k), ("src_v", src_v), ("dst_k", dst_k), ("dst_v", dst_v),
          ("block_pairs", block_pairs))
    for name, t in ts:
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{name} must be a CUDA tensor or pinned host memory")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if device is None:
        cuda = [t.device for _, t in ts if t.is_cuda]
        device = cuda[0] if cuda else torch.device("cuda", torch.cuda.current_device())
    if block_pairs.dtype != torch.int64 or block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [n, 2] int64 (src, dst)")
    for a, b in ((src_k, src_v), (dst_k, dst_v)):
        if a.shape != b.shape:
            raise ValueError("the K and V pools of one side must match")
    if (src_k.dtype != dst_k.dtype or src_v.dtype != dst_v.dtype or
            tuple(src_k.shape[1:]) != tuple(dst_k.shape[1:])):
        raise ValueError("source and destination pools differ in block layout or dtype")
    q_dtype = torch.float32 if src_k.dtype == torch.float32 else torch.bfloat16
    shape = make_shape(src_k.shape[2], src_k, q_dtype, 0, 1)
    _check(load().pa_swap_blocks(_ptr(src_k), _ptr(src_v), src_k.shape[0], _ptr(dst_k),
                                 _ptr(dst_v), dst_k.shape[0], _ptr(block_pairs),
                                 block_pairs.shape[0], ctypes.byref(shape), _stream(device)))


def decode_workspace_bytes(shape: PAShape) -> int:
    return int(load().pa_decode_workspace_bytes(ctypes.byref(shape)))


def decode(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
           partition_tokens: int = 0, kv_scale: float = 1.0,
           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """pa_decode: out[S, Hq, d] (fp32) = paged single-query attention.

    Runs on the current stream of the pools' device.  Without `workspace`,
    the stream's own cached buffer is used (one per stream, see _workspace);
    a caller-provided workspace must not be shared by calls that may run at
    the same time (different streams)."""
    dev = k_cache.device
    _require(out, "out", dev, torch.float32, 3)
    _require(q, "q", dev, None, 3)
    _require(k_cache, "k_cache", dev)
    _require(v_cache, "v_cache", dev)
    _require(block_tables, "block_tables", dev, torch.int32, 2)
    _require(context_lens, "context_lens", dev, torch.int32, 1)
    S = q.shape[0]
    if out.shape != q.shape or block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("out/q/block_tables/context_lens disagree on the sequence count")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must match")
    if q.shape[2] != k_cache.shape[3]:
        raise ValueError("head_dim of q and of the pools differ")
    shape = make_shape(q.shape[1], k_cache, q.dtype, S, block_tables.shape[1], kv_scale,
                       partition_tokens)
    lib = load()
    need = decode_workspace_bytes(shape)
    ws = workspace if workspace is not None else _workspace(dev, need, "decode")
    _check(lib.pa_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                         _ptr(context_lens), float(scale), ctypes.byref(shape), _ptr(ws),
                         0 if ws is None else ws.numel() * ws.element_size(), _stream(dev)))
    return out


def decode_static(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                  v_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                  scale: float, partition_tokens: int = 0, kv_scale: float = 1.0) -> torch.Tensor:
    """pa_decode_static: pa_decode with the library's static device scratch
    instead of a workspace (nothing is allocated).  Calls that may overlap in
    time on one device must not be issued (they share that scratch)."""
    dev = k_cache.device
    _require(out, "out", dev, torch.float32, 3)
    _require(q, "q", dev, None, 3)
    _require(k_cache, "k_cache", dev)
    _require(v_cache, "v_cache", dev)
    _require(block_tables, "block_tables", dev, torch.int32, 2)
    _require(context_lens, "context_lens", dev, torch.int32, 1)
    S = q.shape[0]
    if out.shape != q.shape or block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("out/q/block_tables/context_lens disagree on the sequence count")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must match")
    if q.shape[2] != k_cache.shape[3]:
        raise ValueError("head_dim of q and of the pools differ")
    shape = make_shape(q.shape[1], k_cache, q.dtype, S, block_tables.shape[1], kv_scale,
                       partition_tokens)
    _check(load().pa_decode_static(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(block_tables), _ptr(context_lens), float(scale),
                                   ctypes.byref(shape), _stream(dev)))
    return out


def prefill_workspace_bytes(shape: PAShape, total_query_rows: int) -> int:
    return int(load().pa_prefill_workspace_bytes(ctypes.byref(shape), int(total_query_rows)))


def prefill_chunk(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                  v_cache: torch.Tensor, block_tables: torch.Tensor, query_start: torch.Tensor,
                  context_lens: torch.Tensor, scale: float, kv_scale: float = 1.0,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """pa_prefill_chunk: out[Tq, Hq, d] (fp32) for chunks over their paged history.

    Runs on the current stream of the pools' device; the workspace rules are
    those of decode()."""
    dev = k_cache.device
    _require(out, "out", dev, torch.float32, 3)
    _require(q, "q", dev, torch.bfloat16, 3)
    _require(k_cache, "k_cache", dev)
    _require(v_cache, "v_cache", dev)
    _require(block_tables, "block_tables", dev, torch.int32, 2)
    _require(query_start, "query_start", dev, torch.int32, 1)
    _require(context_lens, "context_lens", dev, torch.int32, 1)
    R = context_lens.shape[0]
    if out.shape != q.shape or block_tables.shape[0] != R or query_start.shape[0] != R + 1:
        raise ValueError("out/q/block_tables/query_start/context_lens disagree")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must match")
    shape = make_shape(q.shape[1], k_cache, q.dtype, R, block_tables.shape[1], kv_scale)
    lib = load()
    need = prefill_workspace_bytes(shape, q.shape[0])
    ws = workspace if workspace is not None else _workspace(dev, need, "prefill")
    _check(lib.pa_prefill_chunk(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                _ptr(block_tables), _ptr(query_start), _ptr(context_lens),
                                q.shape[0], float(scale), ctypes.byref(shape), _ptr(ws),
                                0 if ws is None else ws.numel() * ws.element_size(),
                                _stream(dev)))
    return out
