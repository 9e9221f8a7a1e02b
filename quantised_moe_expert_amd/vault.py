"""ctypes binding of include/smoe_vault.h (the .smoe vault reader and
writer): the packed on-disk records as Structures and thin wrappers with the
C names. Argument marshalling only; the work happens in libsmoe.so."""

from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

from .binding import SmoeError, _check, load_library, smoe_layer_desc

SMOE_E_FORMAT = -6
SMOE_E_IO = -7
SMOE_E_NOT_FOUND = -8
SMOE_MEM_HOST = 0
SMOE_MEM_DEVICE = 1

_P = ctypes.c_void_p
_I = ctypes.c_int
_U32 = ctypes.c_uint32
_U64 = ctypes.c_uint64


class smoe_vault_header(ctypes.Structure):
    _pack_ = 1
    _fields_ = [
        ("magic", ctypes.c_uint8 * 8), ("version", _U32), ("num_moe_layers", _U32),
        ("max_experts_per_layer", _U32), ("total_experts", _U32), ("table_offset", _U64),
        ("data_offset", _U64), ("group_size", _U32), ("bits", _U32), ("d_model", _U32),
        ("vocab_size", _U32), ("ffn_dim", _U32), ("reserved_ext", _U32),
    ]


class smoe_arch_block(ctypes.Structure):
    _pack_ = 1
    _fields_ = [
        ("magic", ctypes.c_uint8 * 4), ("block_version", _U32), ("block_size", _U32),
        ("flags", _U32), ("rope_theta", ctypes.c_float), ("num_heads", _U32),
        ("num_kv_heads", _U32), ("head_dim", _U32), ("moe_top_k", _U32), ("moe_ffn_dim", _U32),
        ("dense_ffn_dim", _U32), ("shared_expert_ffn_dim", _U32), ("activation", _U32),
        ("num_hidden_layers", _U32), ("rms_norm_eps", ctypes.c_float),
        ("model_type", ctypes.c_char * 24), ("reserved", ctypes.c_uint8 * 44),
    ]


class smoe_expert_entry(ctypes.Structure):
    _pack_ = 1
    _fields_ = [
        ("layer_id", _U32), ("expert_id", _U32), ("byte_offset", _U64), ("raw_size", _U64),
        ("padded_size", _U64), ("group_size", _U32), ("num_groups", _U64),
        ("reserved", ctypes.c_uint8 * 4),
    ]


class smoe_tensor_desc(ctypes.Structure):
    _pack_ = 1
    _fields_ = [
        ("tensor_type", ctypes.c_uint8), ("ndim", ctypes.c_uint8),
        ("reserved_0", ctypes.c_uint8 * 2), ("rows", _U32), ("cols", _U32),
        ("packed_offset", _U64), ("packed_size", _U64), ("scales_offset", _U64),
        ("scales_size", _U64),
    ]


class smoe_vault_spec(ctypes.Structure):
    _fields_ = [
        ("version", _U32), ("bits", _U32), ("d_model", _U32), ("moe_ffn_dim", _U32),
        ("vocab_size", _U32), ("ffn_dim", _U32), ("num_moe_layers", _U32),
        ("experts_per_layer", _U32), ("layer_ids", ctypes.POINTER(_U32)),
        ("arch", ctypes.POINTER(smoe_arch_block)),
    ]


def declare(lib: ctypes.CDLL) -> None:
    """Set the argument and result types of the vault functions."""
    P = ctypes.POINTER
    lib.smoe_arch_block_init.restype = None
    lib.smoe_arch_block_init.argtypes = [P(smoe_arch_block)]
    lib.smoe_vault_plan.restype = _I
    lib.smoe_vault_plan.argtypes = [P(smoe_vault_spec), P(smoe_vault_header), P(_U64)]
    lib.smoe_vault_create.restype = _I
    lib.smoe_vault_create.argtypes = [ctypes.c_char_p, P(smoe_vault_spec), P(_P)]
    lib.smoe_vault_put_expert.restype = _I
    lib.smoe_vault_put_expert.argtypes = [_P, _U32, _U32, _P, _U64, _I, _P]
    lib.smoe_vault_finish.restype = _I
    lib.smoe_vault_finish.argtypes = [_P]
    lib.smoe_vault_open.restype = _I
    lib.smoe_vault_open.argtypes = [ctypes.c_char_p, P(_P)]
    lib.smoe_vault_close.restype = None
    lib.smoe_vault_close.argtypes = [_P]
    lib.smoe_vault_get_header.restype = _I
    lib.smoe_vault_get_header.argtypes = [_P, P(smoe_vault_header), P(smoe_arch_block)]
    lib.smoe_vault_find.restype = _I
    lib.smoe_vault_find.argtypes = [_P, _U32, _U32, P(smoe_expert_entry), P(smoe_tensor_desc)]
    lib.smoe_vault_layer_desc.restype = _I
    lib.smoe_vault_layer_desc.argtypes = [_P, _U32, P(smoe_layer_desc)]
    lib.smoe_vault_read_expert.restype = _I
    lib.smoe_vault_read_expert.argtypes = [_P, _U32, _U32, _P, _U64, _I, _P]
    lib.smoe_vault_read_layer.restype = _I
    lib.smoe_vault_read_layer.argtypes = [_P, _U32, _P, _U64, _I, _P]


def smoe_arch_block_init() -> smoe_arch_block:
    a = smoe_arch_block()
    load_library().smoe_arch_block_init(ctypes.byref(a))
    return a


def make_vault_spec(version: int, bits: int, d_model: int, moe_ffn_dim: int,
                    layer_ids: Sequence[int], experts_per_layer: int,
                    arch: Optional[smoe_arch_block] = None, vocab_size: int = 0,
                    ffn_dim: int = 0) -> smoe_vault_spec:
    """A spec; it keeps its layer-id array and arch block alive."""
    ids = (_U32 * len(layer_ids))(*layer_ids)
    s = smoe_vault_spec(version, bits, d_model, moe_ffn_dim, vocab_size, ffn_dim,
                        len(layer_ids), experts_per_layer,
                        ctypes.cast(ids, ctypes.POINTER(_U32)),
                        ctypes.pointer(arch) if arch is not None else None)
    s._keep = (ids, arch)
    return s


def smoe_vault_plan(spec: smoe_vault_spec) -> Tuple[smoe_vault_header, int]:
    h = smoe_vault_header()
    size = _U64()
    _check(load_library().smoe_vault_plan(ctypes.byref(spec), ctypes.byref(h), ctypes.byref(size)))
    return h, size.value


def smoe_vault_create(path: str, spec: smoe_vault_spec) -> int:
    w = _P()
    _check(load_library().smoe_vault_create(path.encode(), ctypes.byref(spec), ctypes.byref(w)))
    return w.value


def smoe_vault_put_expert(writer: int, layer_id: int, expert_id: int, blob: int, nbytes: int,
                          location: int, hip_stream: int = 0) -> None:
    _check(load_library().smoe_vault_put_expert(writer, layer_id, expert_id, blob or None, nbytes,
                                                location, hip_stream or None))


def smoe_vault_finish(writer: int) -> None:
    _check(load_library().smoe_vault_finish(writer or None))


def smoe_vault_open(path: str) -> int:
    v = _P()
    _check(load_library().smoe_vault_open(path.encode(), ctypes.byref(v)))
    return v.value


def smoe_vault_close(vault: int) -> None:
    load_library().smoe_vault_close(vault or None)


def smoe_vault_get_header(vault: int) -> Tuple[smoe_vault_header, smoe_arch_block]:
    h = smoe_vault_header()
    a = smoe_arch_block()
    _check(load_library().smoe_vault_get_header(vault, ctypes.byref(h), ctypes.byref(a)))
    return h, a


def smoe_vault_find(vault: int, layer_id: int, expert_id: int
                    ) -> Tuple[smoe_expert_entry, Tuple[smoe_tensor_desc, ...]]:
    e = smoe_expert_entry()
    d = (smoe_tensor_desc * 3)()
    _check(load_library().smoe_vault_find(vault, layer_id, expert_id, ctypes.byref(e), d))
    return e, tuple(d)


def smoe_vault_layer_desc(vault: int, layer_id: int) -> smoe_layer_desc:
    out = smoe_layer_desc()
    _check(load_library().smoe_vault_layer_desc(vault, layer_id, ctypes.byref(out)))
    return out


def smoe_vault_read_expert(vault: int, layer_id: int, expert_id: int, dst: int, nbytes: int,
                           location: int, hip_stream: int = 0) -> None:
    _check(load_library().smoe_vault_read_expert(vault, layer_id, expert_id, dst or None, nbytes,
                                                 location, hip_stream or None))


def smoe_vault_read_layer(vault: int, layer_id: int, dst: int, nbytes: int, location: int,
                          hip_stream: int = 0) -> None:
    _check(load_library().smoe_vault_read_layer(vault, layer_id, dst or None, nbytes, location,
                                                hip_stream or None))


__all__ = [n for n in dir() if n.startswith(("smoe_", "SMOE_", "make_vault"))] + ["SmoeError"]
