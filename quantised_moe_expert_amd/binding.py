"""ctypes binding of the SMOE C ABI (include/smoe.h).

Argument marshalling only: every function forwards to the function of the
same name in ``libsmoe.so`` and turns a negative status into
:class:`SmoeError`. Pointers are plain integers (device addresses, e.g. a
torch tensor's ``data_ptr()``); streams are ``hipStream_t`` handles as
integers (e.g. ``torch.cuda.current_stream().cuda_stream``), 0 for the null
stream. The library is loaded on first use and a missing or stale build is a
hard error: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

LIB_NAME = "libsmoe.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

SMOE_OK = 0
SMOE_E_ARG = -1
SMOE_E_LAYOUT = -2
SMOE_E_UNSUPPORTED = -3
SMOE_E_HIP = -4
SMOE_E_WORKSPACE = -5

SMOE_DTYPE_F32 = 0
SMOE_DTYPE_BF16 = 1
SMOE_SCALE_F32 = 0
SMOE_SCALE_F16 = 1

SMOE_MAX_TOP_K = 16
SMOE_MAX_EXPERTS = 512
SMOE_MAX_TOKENS = 4096
SMOE_NOALLOC_SCRATCH_BYTES = 32 << 20
SMOE_MAX_QUANT_ELEMENTS = 1 << 31
SMOE_BLOB_ALIGN = 16384
SMOE_BANK_ALIGN = 16384

SMOE_KERNEL_NONE = 0
SMOE_KERNEL_GATE_UP = 1
SMOE_KERNEL_DOWN = 2

# every symbol include/smoe.h declares
EXPORTED = (
    "smoe_version", "smoe_last_error", "smoe_expert_layout_of", "smoe_load_blobs",
    "smoe_free", "smoe_workspace_bytes", "smoe_route", "smoe_moe_forward",
    "smoe_decode_step", "smoe_trace_kernel", "smoe_route_opts_init", "smoe_route_ex",
    "smoe_moe_forward_ex", "smoe_quantise", "smoe_moe_forward_noalloc",
    # include/smoe_vault.h
    "smoe_arch_block_init", "smoe_vault_plan", "smoe_vault_create", "smoe_vault_put_expert",
    "smoe_vault_finish", "smoe_vault_open", "smoe_vault_close", "smoe_vault_get_header",
    "smoe_vault_find", "smoe_vault_layer_desc", "smoe_vault_read_expert",
    "smoe_vault_read_layer",
    # include/smoe_offload.h
    "smoe_offload_create", "smoe_offload_free", "smoe_offload_forward",
    "smoe_offload_workspace_bytes", "smoe_offload_slots", "smoe_offload_get_stats",
)


class SmoeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"smoe error {code}: {message}")
        self.code = code


class smoe_route_opts(ctypes.Structure):
    """Routing variants (see smoe_route_opts in include/smoe.h)."""
    _fields_ = [
        ("sigmoid", ctypes.c_int32),
        ("scaling_factor", ctypes.c_float),
        ("d_expert_bias", ctypes.c_void_p),
        ("d_shared_gate", ctypes.c_void_p),
        ("use_mask", ctypes.c_int32),
        ("expert_mask", ctypes.c_uint32 * (SMOE_MAX_EXPERTS // 32)),
    ]


def make_route_opts(sigmoid: bool = False, scaling_factor: float = 1.0, d_expert_bias: int = 0,
                    d_shared_gate: int = 0, routable: Optional[Sequence[bool]] = None
                    ) -> smoe_route_opts:
    """smoe_route_opts from Python values; routable: one bool per expert (None =
    all), packed LSB-first into the mask words."""
    o = smoe_route_opts()
    load_library().smoe_route_opts_init(ctypes.byref(o))
    o.sigmoid = int(bool(sigmoid))
    o.scaling_factor = float(scaling_factor)
    o.d_expert_bias = d_expert_bias or None
    o.d_shared_gate = d_shared_gate or None
    if routable is not None:
        o.use_mask = 1
        for e, on in enumerate(routable):
            if on:
                o.expert_mask[e // 32] |= 1 << (e % 32)
    return o


class smoe_layer_desc(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_uint32),
        ("ffn_dim", ctypes.c_uint32),
        ("num_experts", ctypes.c_uint32),
        ("bits", ctypes.c_uint32),
        ("group_size", ctypes.c_uint32),
        ("scale_dtype", ctypes.c_uint32),
        ("blob_stride", ctypes.c_uint64),
        ("shared_ffn_dim", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


class smoe_tensor_layout(ctypes.Structure):
    _fields_ = [
        ("codes_offset", ctypes.c_uint64),
        ("codes_bytes", ctypes.c_uint64),
        ("scales_offset", ctypes.c_uint64),
        ("scales_bytes", ctypes.c_uint64),
        ("rows", ctypes.c_uint32),
        ("cols", ctypes.c_uint32),
    ]


class smoe_expert_layout(ctypes.Structure):
    _fields_ = [
        ("gate", smoe_tensor_layout),
        ("up", smoe_tensor_layout),
        ("down", smoe_tensor_layout),
        ("raw_size", ctypes.c_uint64),
        ("padded_size", ctypes.c_uint64),
    ]


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_U32 = ctypes.c_uint32
_U64 = ctypes.c_uint64


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libsmoe.so (built by __graft_entry__.build()); raises if absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} is missing: build the HIP library first (python -c "
            f"'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(p)
    lib.smoe_version.restype = _I
    lib.smoe_version.argtypes = []
    lib.smoe_last_error.restype = ctypes.c_char_p
    lib.smoe_last_error.argtypes = []
    lib.smoe_expert_layout_of.restype = _I
    lib.smoe_expert_layout_of.argtypes = [_U32, _U32, _U32, _U32,
                                          ctypes.POINTER(smoe_expert_layout)]
    lib.smoe_load_blobs.restype = _I
    lib.smoe_load_blobs.argtypes = [ctypes.POINTER(smoe_layer_desc), _P, _U64, _P, _U64,
                                    ctypes.POINTER(_P)]
    lib.smoe_free.restype = None
    lib.smoe_free.argtypes = [_P]
    lib.smoe_workspace_bytes.restype = _U64
    lib.smoe_workspace_bytes.argtypes = [_P, _I, _I]
    lib.smoe_route.restype = _I
    lib.smoe_route.argtypes = [_P, _I, _I, _I, _I, _P, _P, _P]
    lib.smoe_moe_forward.restype = _I
    lib.smoe_moe_forward.argtypes = [_P, _P, _I, _P, _I, _I, _I, _P, _P, _P, _P, _U64, _P]
    lib.smoe_decode_step.restype = _I
    lib.smoe_decode_step.argtypes = [ctypes.POINTER(_P), _I, _P, _P, _I, _I, _I,
                                     ctypes.c_float, _P, _U64, _P]
    lib.smoe_trace_kernel.restype = _I
    lib.smoe_trace_kernel.argtypes = [_I, _P, _P]
    lib.smoe_route_opts_init.restype = None
    lib.smoe_route_opts_init.argtypes = [ctypes.POINTER(smoe_route_opts)]
    lib.smoe_route_ex.restype = _I
    lib.smoe_route_ex.argtypes = [_P, _I, _I, _I, _I, ctypes.POINTER(smoe_route_opts), _P, _P,
                                  _P]
    lib.smoe_quantise.restype = _I
    lib.smoe_quantise.argtypes = [_P, _U64, _I, _I, _P, _P, _P]
    lib.smoe_moe_forward_ex.restype = _I
    lib.smoe_moe_forward_ex.argtypes = [_P, _P, _I, _P, _I, _I, _I,
                                        ctypes.POINTER(smoe_route_opts), _P, _P, _P, _P, _U64,
                                        _P]
    lib.smoe_moe_forward_noalloc.restype = _I
    lib.smoe_moe_forward_noalloc.argtypes = [_P, _P, _I, _P, _I, _I, _I, _P, _P, _P, _P]
    from .vault import declare as _declare_vault
    from .offload import declare as _declare_offload
    _declare_vault(lib)
    _declare_offload(lib)
    if path is None:
        _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != SMOE_OK:
        raise SmoeError(rc, smoe_last_error())


def smoe_version() -> int:
    return load_library().smoe_version()


def smoe_last_error() -> str:
    return load_library().smoe_last_error().decode()


def smoe_expert_layout_of(d_model: int, ffn_dim: int, bits: int,
                          scale_dtype: int = SMOE_SCALE_F32) -> smoe_expert_layout:
    out = smoe_expert_layout()
    _check(load_library().smoe_expert_layout_of(d_model, ffn_dim, bits, scale_dtype,
                                                 ctypes.byref(out)))
    return out


def aligned_buffer(nbytes: int, device="cuda:0", align: int = SMOE_BANK_ALIGN,
                   pin_memory: bool = False):
    """A uint8 torch tensor of nbytes whose data starts on an `align` boundary
    (expert banks and shared blobs must be 16 KB aligned): a view into an
    allocation `align` bytes larger, which the view keeps alive. With
    pin_memory the buffer is pinned host memory, else device memory."""
    import torch
    if pin_memory:
        base = torch.empty(nbytes + align, dtype=torch.uint8, pin_memory=True)
    else:
        base = torch.empty(nbytes + align, dtype=torch.uint8, device=device)
    off = (-base.data_ptr()) % align
    return base[off: off + nbytes]


def make_desc(d_model: int, ffn_dim: int, num_experts: int, bits: int,
              blob_stride: int, scale_dtype: int = SMOE_SCALE_F32,
              shared_ffn_dim: int = 0, group_size: int = 64) -> smoe_layer_desc:
    return smoe_layer_desc(d_model, ffn_dim, num_experts, bits, group_size, scale_dtype,
                           blob_stride, shared_ffn_dim, 0)


def smoe_load_blobs(desc: smoe_layer_desc, d_blobs: int, nbytes: int,
                    d_shared_blob: int = 0, shared_nbytes: int = 0) -> int:
    """Returns the layer handle (an opaque integer)."""
    h = _P()
    _check(load_library().smoe_load_blobs(ctypes.byref(desc), d_blobs or None, nbytes,
                                          d_shared_blob or None, shared_nbytes,
                                          ctypes.byref(h)))
    return h.value


def smoe_free(layer: Optional[int]) -> None:
    load_library().smoe_free(layer or None)


def smoe_workspace_bytes(layer: int, n_tokens: int, top_k: int) -> int:
    return load_library().smoe_workspace_bytes(layer, n_tokens, top_k)


def smoe_route(d_logits: int, n_tokens: int, n_experts: int, top_k: int,
               norm_topk_prob: bool, d_ids: int, d_weights: int, hip_stream: int = 0) -> None:
    _check(load_library().smoe_route(d_logits or None, n_tokens, n_experts, top_k,
                                     int(bool(norm_topk_prob)), d_ids or None,
                                     d_weights or None, hip_stream or None))


def smoe_moe_forward(layer: int, d_x: int, x_dtype: int, d_logits: int, n_tokens: int,
                     top_k: int, norm_topk_prob: bool, d_out: int, d_topk_ids: int,
                     d_topk_w: int, d_workspace: int, ws_bytes: int,
                     hip_stream: int = 0) -> None:
    _check(load_library().smoe_moe_forward(
        layer, d_x or None, x_dtype, d_logits or None, n_tokens, top_k,
        int(bool(norm_topk_prob)), d_out or None, d_topk_ids or None, d_topk_w or None,
        d_workspace or None, ws_bytes, hip_stream or None))


def smoe_route_ex(d_logits: int, n_tokens: int, n_experts: int, top_k: int,
                  norm_topk_prob: bool, opts: Optional[smoe_route_opts], d_ids: int,
                  d_weights: int, hip_stream: int = 0) -> None:
    _check(load_library().smoe_route_ex(d_logits or None, n_tokens, n_experts, top_k,
                                        int(bool(norm_topk_prob)),
                                        ctypes.byref(opts) if opts is not None else None,
                                        d_ids or None, d_weights or None, hip_stream or None))


def smoe_moe_forward_ex(layer: int, d_x: int, x_dtype: int, d_logits: int, n_tokens: int,
                        top_k: int, norm_topk_prob: bool, opts: Optional[smoe_route_opts],
                        d_out: int, d_topk_ids: int, d_topk_w: int, d_workspace: int,
                        ws_bytes: int, hip_stream: int = 0) -> None:
    _check(load_library().smoe_moe_forward_ex(
        layer, d_x or None, x_dtype, d_logits or None, n_tokens, top_k,
        int(bool(norm_topk_prob)), ctypes.byref(opts) if opts is not None else None,
        d_out or None, d_topk_ids or None, d_topk_w or None, d_workspace or None, ws_bytes,
        hip_stream or None))


def smoe_moe_forward_noalloc(layer: int, d_x: int, x_dtype: int, d_logits: int,
                             n_tokens: int, top_k: int, norm_topk_prob: bool, d_out: int,
                             d_topk_ids: int, d_topk_w: int, hip_stream: int = 0) -> None:
    _check(load_library().smoe_moe_forward_noalloc(
        layer, d_x or None, x_dtype, d_logits or None, n_tokens, top_k,
        int(bool(norm_topk_prob)), d_out or None, d_topk_ids or None, d_topk_w or None,
        hip_stream or None))


def smoe_decode_step(layers: Sequence[int], d_h: int, d_logits: int, n_tokens: int,
                     top_k: int, norm_topk_prob: bool, eps: float, d_workspace: int,
                     ws_bytes: int, hip_stream: int = 0) -> None:
    arr = (_P * max(1, len(layers)))(*layers)
    _check(load_library().smoe_decode_step(arr, len(layers), d_h or None, d_logits or None,
                                           n_tokens, top_k, int(bool(norm_topk_prob)),
                                           float(eps), d_workspace or None, ws_bytes,
                                           hip_stream or None))


def smoe_trace_kernel(kernel: int, hip_event_before: int = 0, hip_event_after: int = 0) -> int:
    """Arm (or, with SMOE_KERNEL_NONE, disarm) the one-shot launch events;
    disarming returns 1 when the armed pair never fired."""
    rc = load_library().smoe_trace_kernel(kernel, hip_event_before or None,
                                          hip_event_after or None)
    if rc < 0:
        raise SmoeError(rc, smoe_last_error())
    return rc


def smoe_quantise(d_w: int, n_elements: int, bits: int, scale_dtype: int, d_codes: int,
                  d_scales: int, hip_stream: int = 0) -> None:
    _check(load_library().smoe_quantise(d_w or None, n_elements, bits, scale_dtype,
                                        d_codes or None, d_scales or None, hip_stream or None))
