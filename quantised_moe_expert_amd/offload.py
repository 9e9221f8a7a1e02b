"""ctypes binding of include/smoe_offload.h (experts in pinned host memory,
streamed to the GPU): argument marshalling only."""

from __future__ import annotations

import ctypes
from typing import Optional

from .binding import _check, load_library, smoe_layer_desc

_P = ctypes.c_void_p
_I = ctypes.c_int
_U32 = ctypes.c_uint32
_U64 = ctypes.c_uint64


class smoe_offload_stats(ctypes.Structure):
    _fields_ = [("forwards", _U64), ("hits", _U64), ("fetched", _U64), ("direct", _U64),
                ("bytes_fetched", _U64)]


def declare(lib: ctypes.CDLL) -> None:
    P = ctypes.POINTER
    lib.smoe_offload_create.restype = _I
    lib.smoe_offload_create.argtypes = [P(smoe_layer_desc), _P, _U64, _P, _U64, _P, _U64, _P,
                                        P(_P)]
    lib.smoe_offload_free.restype = None
    lib.smoe_offload_free.argtypes = [_P]
    lib.smoe_offload_forward.restype = _I
    lib.smoe_offload_forward.argtypes = [_P, _P, _I, _P, _I, _I, _I, _P, _P, _P, _P, _U64, _P]
    lib.smoe_offload_workspace_bytes.restype = _U64
    lib.smoe_offload_workspace_bytes.argtypes = [_P, _I, _I]
    lib.smoe_offload_slots.restype = _U32
    lib.smoe_offload_slots.argtypes = [_P]
    lib.smoe_offload_get_stats.restype = _I
    lib.smoe_offload_get_stats.argtypes = [_P, P(smoe_offload_stats)]


def smoe_offload_create(desc: smoe_layer_desc, h_blobs: int, nbytes: int, d_shared_blob: int,
                        shared_nbytes: int, d_cache: int, cache_bytes: int, d_table: int) -> int:
    h = _P()
    _check(load_library().smoe_offload_create(ctypes.byref(desc), h_blobs or None, nbytes,
                                               d_shared_blob or None, shared_nbytes,
                                               d_cache or None, cache_bytes, d_table or None,
                                               ctypes.byref(h)))
    return h.value


def smoe_offload_free(off: int) -> None:
    load_library().smoe_offload_free(off or None)


def smoe_offload_forward(off: int, d_x: int, x_dtype: int, d_logits: int, n_tokens: int,
                         top_k: int, norm_topk_prob: bool, d_out: int, d_topk_ids: int,
                         d_topk_w: int, d_workspace: int, ws_bytes: int,
                         hip_stream: int = 0) -> None:
    _check(load_library().smoe_offload_forward(
        off, d_x or None, x_dtype, d_logits or None, n_tokens, top_k, int(bool(norm_topk_prob)),
        d_out or None, d_topk_ids or None, d_topk_w or None, d_workspace or None, ws_bytes,
        hip_stream or None))


def smoe_offload_workspace_bytes(off: int, n_tokens: int, top_k: int) -> int:
    return load_library().smoe_offload_workspace_bytes(off, n_tokens, top_k)


def smoe_offload_slots(off: int) -> int:
    return load_library().smoe_offload_slots(off)


def smoe_offload_get_stats(off: int) -> smoe_offload_stats:
    st = smoe_offload_stats()
    _check(load_library().smoe_offload_get_stats(off, ctypes.byref(st)))
    return st


__all__ = [n for n in dir() if n.startswith("smoe_")]
