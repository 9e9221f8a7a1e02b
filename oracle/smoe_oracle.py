"""Plain, slow CPU definition of the SMOE routed-expert MoE FFN.

TEST INFRASTRUCTURE. This module is the oracle that the HIP path is checked
against. It shares no code with the GPU library and imports nothing from it.
Only the test suite, the smoke check and the CPU-baseline leg of the bench
may use it. Everything is NumPy in float64 unless a step's precision is fixed
by the pages (fp32 router logits are compared as fp32, stored scales are
rounded to their storage dtype before they are used).

Sources (page title, section):

* ".smoe Binary Format" -- "Expert Blob Architecture": per expert, the gate,
  up and down tensors follow one another, each as packed codes
  (ceil(rows*cols*bits/8) bytes) then its scales (one per group of
  ``group_size`` weights over the flattened tensor), then zero padding to the
  16 KB boundary; "Immutable Encoding": little-endian, 16,384-byte blob
  alignment; "Tensor Descriptor": rows/cols are the weight's original
  [out, in] shape.
* "SMOE Quantisation" -- "Quantisation Levels" (Q2: four levels -1, -1/3,
  +1/3, +1; Q4: sixteen symmetric levels), "L2-MSE Scale Optimiser" (64
  candidate scales from 0.1 to 1.0 times the group absmax, keep the one with
  the smallest squared error; encoders for Q2 and Q4), "Bit Packing" (4 or 2
  codes per byte, least significant bits first), "Decoding: Metal Kernel"
  (weight = (code - m) / m * scale with m = 1.5 for Q2, 7.5 for Q4).
* "CMF v2 Format Specification" -- section 2.2 "MoE": softmax over all router
  logits, top-k with ties going to the lower expert index, optional
  renormalisation of the selected weights, weighted sum of the expert FFN
  outputs, shared expert added with weight 1 when it has no gate.
* "Model Agnosticism" -- the engine implements SiLU/SwiGLU only and caps the
  routing width at 16 experts per token; norm_topk_prob is a per-model flag.
* ".smoe Binary Format" -- "Arch Block": the kernels compile an RMS-norm
  epsilon of 1e-6 (used by the stacked decode step).

Readings where the pages are silent (each also listed in the design notes):
the rounding mode of ``round()`` in the encoders is round-half-to-even; the
candidate grid is NumPy ``linspace`` (last candidate exactly 1.0 x absmax);
each candidate scale is rounded to the storage dtype before it is scored and
used for encoding; MSE ties keep the first (smallest) candidate; an all-zero
group gets scale 0; experts are selected on the raw fp32 logits (softmax is
monotone); RMSNorm has unit gain; the stacked residual stream is float64
here; the shared expert's weights use the same blob layout as a routed
expert.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "GROUP_SIZE", "BLOB_ALIGN", "MAX_TOP_K",
    "level_midpoint", "level_table",
    "packed_size", "scale_count", "pad_to_blob",
    "pack_codes", "unpack_codes", "unpack_codes_scalar",
    "dequantise", "encode_codes", "decode_codes",
    "candidate_fractions", "mse_grid_scale", "quantise_tensor",
    "TensorSpan", "ExpertLayout", "expert_layout",
    "build_expert_blob", "read_expert_tensors",
    "OracleLayer", "route", "softmax64", "silu", "swiglu_expert",
    "RouteOpts", "route_ex",
    "moe_forward", "rms_norm", "decode_step",
]

GROUP_SIZE = 64          # quantisation group (".smoe Binary Format", File Header)
BLOB_ALIGN = 16384       # expert blob alignment ("Immutable Encoding")
MAX_TOP_K = 16           # routing width cap ("Model Agnosticism", Expanding the Frontier)

_SCALE_DTYPES = {"f32": np.float32, "f16": np.float16}


# --------------------------------------------------------------------------
# Levels ("SMOE Quantisation": Quantisation Levels; Decoding: Metal Kernel)
# --------------------------------------------------------------------------

def level_midpoint(bits: int) -> float:
    """m in weight = (code - m)/m * scale: 1.5 for Q2, 7.5 for Q4."""
    if bits == 2:
        return 1.5
    if bits == 4:
        return 7.5
    raise ValueError(f"bits must be 2 or 4, got {bits}")


def level_table(bits: int) -> np.ndarray:
    """Normalised level of every code value, (c - m)/m, in float64."""
    m = level_midpoint(bits)
    return np.array([(c - m) / m for c in range(1 << bits)], dtype=np.float64)


# --------------------------------------------------------------------------
# Sizes (".smoe Binary Format": Expert Blob Architecture)
# --------------------------------------------------------------------------

def packed_size(n_codes: int, bits: int) -> int:
    """Bytes of a packed code stream: ceil(n * bits / 8)."""
    return (int(n_codes) * int(bits) + 7) // 8


def scale_count(n_codes: int, group: int = GROUP_SIZE) -> int:
    """Number of group scales of a tensor: ceil(n / group)."""
    return (int(n_codes) + group - 1) // group


def pad_to_blob(nbytes: int) -> int:
    """Round a raw blob size up to the 16 KB boundary."""
    return (int(nbytes) + BLOB_ALIGN - 1) // BLOB_ALIGN * BLOB_ALIGN


# --------------------------------------------------------------------------
# Bit packing ("SMOE Quantisation": Bit Packing), LSB-first
# --------------------------------------------------------------------------

def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes (flat order) LSB-first: code i sits in byte i // per at bit
    (i % per) * bits, per = 8 / bits codes per byte. A partial last byte is
    zero-filled in its high bits."""
    per = 8 // bits
    c = np.asarray(codes).reshape(-1).astype(np.uint16)
    if c.size and int(c.max()) >= (1 << bits):
        raise ValueError("code out of range")
    n = c.size
    nbytes = packed_size(n, bits)
    padded = np.zeros(nbytes * per, dtype=np.uint16)
    padded[:n] = c
    padded = padded.reshape(nbytes, per)
    out = np.zeros(nbytes, dtype=np.uint16)
    for j in range(per):
        out |= padded[:, j] << (j * bits)
    return out.astype(np.uint8)


def unpack_codes_scalar(packed: Sequence[int], n: int, bits: int) -> List[int]:
    """Scalar definition of unpacking: for each flat index i, shift the byte
    holding it right by (i % per) * bits and keep the low `bits` bits. Pure
    Python; for small cases."""
    per = 8 // bits
    mask = (1 << bits) - 1
    out = []
    for i in range(int(n)):
        byte = int(packed[i // per])
        out.append((byte >> ((i % per) * bits)) & mask)
    return out


def unpack_codes(packed: np.ndarray, n: int, bits: int) -> np.ndarray:
    """Vectorised form of :func:`unpack_codes_scalar` (same definition, one
    bit position at a time)."""
    per = 8 // bits
    mask = (1 << bits) - 1
    b = np.asarray(packed, dtype=np.uint8).reshape(-1)
    if b.size < packed_size(n, bits):
        raise ValueError("packed stream too short")
    out = np.empty(b.size * per, dtype=np.uint8)
    for j in range(per):
        out[j::per] = (b >> (j * bits)) & mask
    return out[: int(n)]


# --------------------------------------------------------------------------
# Dequantisation ("SMOE Quantisation": Decoding; ".smoe": scale per group)
# --------------------------------------------------------------------------

def decode_codes(codes: np.ndarray, scale: float, bits: int) -> np.ndarray:
    """(code - m)/m * scale in float64 for codes sharing one scale."""
    m = level_midpoint(bits)
    return (np.asarray(codes, dtype=np.float64) - m) / m * float(scale)


def dequantise(packed: np.ndarray, scales: np.ndarray, rows: int, cols: int,
               bits: int, group: int = GROUP_SIZE,
               out: Optional[np.ndarray] = None) -> np.ndarray:
    """Dense float64 [rows, cols] weight. Flat element i (row-major) uses
    scale[i // group]; groups run over the flattened tensor and may straddle
    rows when cols is not a multiple of the group. `out` (optional, float64,
    rows * cols elements) receives the result."""
    n = int(rows) * int(cols)
    codes = unpack_codes(packed, n, bits)
    s = np.asarray(scales).reshape(-1).astype(np.float64)
    ng = scale_count(n, group)
    if s.size < ng:
        raise ValueError("too few scales")
    w = np.empty(n, np.float64) if out is None else out.reshape(-1)
    if w.size != n or w.dtype != np.float64:
        raise ValueError("out must hold rows * cols float64 values")
    # the level (c - m)/m of every code from the table of all 2^bits levels
    # (the same float64 values), times the scale of its group
    np.take(level_table(bits), codes, out=w)
    if n % group == 0:
        w.reshape(ng, group)[...] *= s[:ng, None]
    else:
        w *= s[np.arange(n) // group]
    return w.reshape(int(rows), int(cols))


# --------------------------------------------------------------------------
# Quantiser ("SMOE Quantisation": L2-MSE Scale Optimiser)
# --------------------------------------------------------------------------

def encode_codes(w: np.ndarray, scale: float, bits: int) -> np.ndarray:
    """Encoder: clamp(round(w/scale * m + m), 0, 2^bits - 1), with
    round-half-to-even. A zero scale maps every weight to round(m)."""
    m = level_midpoint(bits)
    w = np.asarray(w, dtype=np.float64)
    if scale == 0.0:
        n = np.zeros_like(w)
    else:
        n = w / float(scale)
    return np.clip(np.rint(n * m + m), 0, (1 << bits) - 1).astype(np.uint8)


def candidate_fractions() -> np.ndarray:
    """The 64 candidate fractions of absmax, 0.1 ... 1.0 (NumPy linspace)."""
    return np.linspace(0.1, 1.0, 64)


def mse_grid_scale(group_w: np.ndarray, bits: int,
                   scale_dtype: str = "f32") -> Tuple[float, np.ndarray, int]:
    """Choose a group's scale by the 64-candidate squared-error search.

    Each candidate fraction * absmax is rounded to the storage dtype first;
    the group is encoded and decoded with that stored value and the squared
    error is summed in float64 in element order (the pages fix neither the
    precision nor the order; a fixed order makes the choice reproducible);
    the first minimum wins. Returns (stored scale as float, codes, candidate
    index)."""
    st = _SCALE_DTYPES[scale_dtype]
    w = np.asarray(group_w, dtype=np.float64).reshape(-1)
    absmax = float(np.max(np.abs(w))) if w.size else 0.0
    best = None
    for i, frac in enumerate(candidate_fractions()):
        s = float(st(frac * absmax))
        codes = encode_codes(w, s, bits)
        d = w - decode_codes(codes, s, bits)
        err = 0.0
        for v in (d * d).tolist():
            err += v
        if best is None or err < best[0]:
            best = (err, s, codes, i)
    _, s, codes, i = best
    return s, codes, i


def quantise_tensor(W: np.ndarray, bits: int, scale_dtype: str = "f32",
                    group: int = GROUP_SIZE) -> Tuple[np.ndarray, np.ndarray]:
    """Quantise a [rows, cols] tensor group by group over its flattened
    order. Returns (packed LSB-first codes, scales in the storage dtype)."""
    flat = np.asarray(W, dtype=np.float64).reshape(-1)
    n = flat.size
    ng = scale_count(n, group)
    codes = np.empty(n, dtype=np.uint8)
    scales = np.empty(ng, dtype=_SCALE_DTYPES[scale_dtype])
    for g in range(ng):
        lo, hi = g * group, min(n, (g + 1) * group)
        s, c, _ = mse_grid_scale(flat[lo:hi], bits, scale_dtype)
        codes[lo:hi] = c
        scales[g] = s
    return pack_codes(codes, bits), scales


# --------------------------------------------------------------------------
# Expert blob layout (".smoe Binary Format": Expert Blob Architecture)
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class TensorSpan:
    rows: int
    cols: int
    codes_offset: int
    codes_bytes: int
    scales_offset: int
    scales_bytes: int
    n_scales: int


@dataclasses.dataclass(frozen=True)
class ExpertLayout:
    d_model: int
    ffn_dim: int
    bits: int
    scale_dtype: str
    gate: TensorSpan
    up: TensorSpan
    down: TensorSpan
    raw_size: int
    padded_size: int

    def spans(self) -> Dict[str, TensorSpan]:
        return {"gate": self.gate, "up": self.up, "down": self.down}


def expert_layout(d_model: int, ffn_dim: int, bits: int,
                  scale_dtype: str = "f32") -> ExpertLayout:
    """Offsets of gate [ffn, d], up [ffn, d] and down [d, ffn] inside one
    expert blob: codes then scales for each tensor, packed back to back."""
    ssize = np.dtype(_SCALE_DTYPES[scale_dtype]).itemsize
    off = 0
    spans = []
    for rows, cols in ((ffn_dim, d_model), (ffn_dim, d_model), (d_model, ffn_dim)):
        n = rows * cols
        cb = packed_size(n, bits)
        ns = scale_count(n)
        sb = ns * ssize
        spans.append(TensorSpan(rows, cols, off, cb, off + cb, sb, ns))
        off += cb + sb
    return ExpertLayout(d_model, ffn_dim, bits, scale_dtype, spans[0], spans[1],
                        spans[2], off, pad_to_blob(off))


def build_expert_blob(layout: ExpertLayout,
                      tensors: Dict[str, Tuple[np.ndarray, np.ndarray]]) -> np.ndarray:
    """Assemble one padded expert blob from {'gate'|'up'|'down': (packed
    codes, scales)}; padding bytes are zero."""
    blob = np.zeros(layout.padded_size, dtype=np.uint8)
    st = _SCALE_DTYPES[layout.scale_dtype]
    for name, span in layout.spans().items():
        codes, scales = tensors[name]
        codes = np.asarray(codes, dtype=np.uint8).reshape(-1)
        scales = np.asarray(scales, dtype=st).reshape(-1)
        if codes.size != span.codes_bytes or scales.size != span.n_scales:
            raise ValueError(f"{name}: size mismatch")
        blob[span.codes_offset: span.codes_offset + span.codes_bytes] = codes
        blob[span.scales_offset: span.scales_offset + span.scales_bytes] = \
            scales.view(np.uint8)
    return blob


def read_expert_tensors(blob: np.ndarray, layout: ExpertLayout,
                        out: Optional[Dict[str, np.ndarray]] = None
                        ) -> Dict[str, np.ndarray]:
    """Dense float64 gate, up, down weights of one expert blob (into the
    arrays of `out` when given, one per tensor name)."""
    b = np.asarray(blob, dtype=np.uint8).reshape(-1)
    st = _SCALE_DTYPES[layout.scale_dtype]
    res = {}
    for name, span in layout.spans().items():
        codes = b[span.codes_offset: span.codes_offset + span.codes_bytes]
        scales = b[span.scales_offset: span.scales_offset + span.scales_bytes
                   ].copy().view(st)
        res[name] = dequantise(codes, scales, span.rows, span.cols, layout.bits,
                               out=None if out is None else out[name])
    return res


# --------------------------------------------------------------------------
# Routing ("CMF v2 Format Specification", 2.2 MoE; "Model Agnosticism")
# --------------------------------------------------------------------------

def softmax64(logits: np.ndarray) -> np.ndarray:
    """Max-subtracted softmax over all entries, in float64."""
    l = np.asarray(logits, dtype=np.float64)
    e = np.exp(l - np.max(l))
    return e / np.sum(e)


def route(logits_row: np.ndarray, top_k: int, norm_topk_prob: bool
          ) -> Tuple[List[int], np.ndarray]:
    """Top-k expert ids of one token and their weights.

    Selection compares the fp32 logits exactly: larger logit first, equal
    logits in ascending expert id. Weights are the full softmax's
    probabilities of the chosen experts, divided by their sum when
    norm_topk_prob is set."""
    l32 = np.asarray(logits_row, dtype=np.float32).reshape(-1)
    E = l32.size
    if not (1 <= top_k <= min(MAX_TOP_K, E)):
        raise ValueError(f"top_k must be in [1, min(16, E)], got {top_k}")
    vals = [float(v) for v in l32]
    order = sorted(range(E), key=lambda e: (-vals[e], e))
    ids = order[:top_k]
    p = softmax64(l32)
    w = np.array([p[e] for e in ids], dtype=np.float64)
    if norm_topk_prob:
        w = w / np.sum(w)
    return ids, w


class RouteOpts:
    """Routing variants ("CMF v2 Format Specification", 2.2 MoE; 5. Masks
    section). Defaults reproduce plain softmax routing.

    sigmoid        score each expert with sigmoid(logit) instead of the
                   softmax over all logits.
    expert_bias    [E] added to the scores for the top-k selection only; the
                   weights are the unbiased scores.
    scaling        routed_scaling_factor, applied to the routed weights after
                   the optional renormalisation.
    mask           [E] bools, the routable experts: selection runs over them
                   only and the softmax is taken over them only (other
                   experts get no probability mass); None = all routable.
    shared_gate    [T] fp32 logits; the shared expert's output is weighted by
                   sigmoid(shared_gate[t]) instead of 1."""

    def __init__(self, sigmoid: bool = False, expert_bias=None, scaling: float = 1.0,
                 mask=None, shared_gate=None):
        self.sigmoid = bool(sigmoid)
        self.expert_bias = None if expert_bias is None else np.asarray(expert_bias, np.float32)
        self.scaling = float(np.float32(scaling))
        self.mask = None if mask is None else np.asarray(mask, dtype=bool)
        self.shared_gate = None if shared_gate is None else np.asarray(shared_gate, np.float32)

    def is_default(self) -> bool:
        return (not self.sigmoid and self.expert_bias is None and self.scaling == 1.0
                and self.mask is None and self.shared_gate is None)


def route_ex(logits_row: np.ndarray, top_k: int, norm_topk_prob: bool,
             opts: "RouteOpts") -> Tuple[List[int], np.ndarray]:
    """Top-k routing with the variants of RouteOpts, in the order the format
    states: score (softmax over the routable experts, or sigmoid per expert),
    select the top-k by score + bias (ties to the lower id), gather the
    unbiased scores, renormalise if asked, then multiply by the scaling
    factor.

    Without a bias the selection compares the fp32 logits (the scores are
    monotone in them, and the logits are exact); with a bias it compares the
    float64 sum score + bias, the score being the float64 softmax or sigmoid
    of the fp32 logits and the bias its fp32 value taken exactly. Weights are
    float64."""
    l32 = np.asarray(logits_row, dtype=np.float32).reshape(-1)
    E = l32.size
    mask = np.ones(E, dtype=bool) if opts.mask is None else opts.mask.reshape(-1)
    if mask.size != E:
        raise ValueError("mask needs one entry per expert")
    routable = [e for e in range(E) if mask[e]]
    if not (1 <= top_k <= min(MAX_TOP_K, len(routable))):
        raise ValueError(f"top_k must be in [1, min(16, routable experts)], got {top_k}")
    if opts.sigmoid:
        p = 1.0 / (1.0 + np.exp(-l32.astype(np.float64)))
    else:
        p = np.zeros(E, dtype=np.float64)
        p[mask] = softmax64(l32[mask])
    if opts.expert_bias is None:
        keyv = [float(v) for v in l32]
    else:
        b64 = opts.expert_bias.reshape(-1).astype(np.float64)
        keyv = [float(p[e] + b64[e]) for e in range(E)]
    ids = sorted(routable, key=lambda e: (-keyv[e], e))[:top_k]
    w = np.array([p[e] for e in ids], dtype=np.float64)
    if norm_topk_prob:
        w = w / np.sum(w)
    return ids, w * opts.scaling


# --------------------------------------------------------------------------
# Expert FFN (SwiGLU) and the layer
# --------------------------------------------------------------------------

def silu(g: np.ndarray) -> np.ndarray:
    """g * sigmoid(g) = g / (1 + exp(-g)), float64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_expert(Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray,
                  x: np.ndarray) -> np.ndarray:
    """y = Wd @ (silu(Wg @ x) * (Wu @ x)); Wg, Wu are [ffn, d], Wd [d, ffn]."""
    x = np.asarray(x, dtype=np.float64)
    g = Wg @ x
    u = Wu @ x
    return Wd @ (silu(g) * u)


class OracleLayer:
    """One MoE layer held as host bytes: E routed expert blobs at a fixed
    stride plus an optional shared-expert blob (same layout, its own ffn)."""

    def __init__(self, d_model: int, ffn_dim: int, num_experts: int, bits: int,
                 blobs: np.ndarray, blob_stride: Optional[int] = None,
                 scale_dtype: str = "f32", shared_ffn_dim: int = 0,
                 shared_blob: Optional[np.ndarray] = None,
                 expert_blobs: Optional[Dict[int, np.ndarray]] = None):
        self.layout = expert_layout(d_model, ffn_dim, bits, scale_dtype)
        self.d_model, self.ffn_dim, self.num_experts, self.bits = \
            d_model, ffn_dim, num_experts, bits
        self.stride = blob_stride or self.layout.padded_size
        self.blobs = None if blobs is None else np.asarray(blobs, dtype=np.uint8).reshape(-1)
        # alternatively, only some experts given as {id: blob bytes}
        self.expert_blobs = expert_blobs
        self.shared_layout = (expert_layout(d_model, shared_ffn_dim, bits, scale_dtype)
                              if shared_ffn_dim else None)
        self.shared_blob = shared_blob
        self._cache: Dict[int, Dict[str, np.ndarray]] = {}

    def expert_weights(self, e: int) -> Dict[str, np.ndarray]:
        if e not in self._cache:
            if self.expert_blobs is not None and e in self.expert_blobs:
                b = self.expert_blobs[e]
            else:
                b = self.blobs[e * self.stride: e * self.stride + self.layout.raw_size]
            self._cache[e] = read_expert_tensors(b, self.layout)
        return self._cache[e]

    def expert_weights_into(self, e: int, out: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
        """As expert_weights, into caller-owned float64 arrays (not cached)."""
        if self.expert_blobs is not None and e in self.expert_blobs:
            b = self.expert_blobs[e]
        else:
            b = self.blobs[e * self.stride: e * self.stride + self.layout.raw_size]
        return read_expert_tensors(b, self.layout, out=out)

    def shared_weights(self) -> Optional[Dict[str, np.ndarray]]:
        if self.shared_layout is None:
            return None
        if -1 not in self._cache:
            self._cache[-1] = read_expert_tensors(self.shared_blob, self.shared_layout)
        return self._cache[-1]

    def drop_cache(self):
        self._cache.clear()


def moe_forward(layer: OracleLayer, x: np.ndarray, logits: np.ndarray,
                top_k: int, norm_topk_prob: bool,
                tokens: Optional[Sequence[int]] = None,
                opts: Optional["RouteOpts"] = None
                ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """out[t] = sum_j w[t,j] * FFN_{ids[t,j]}(x[t]) (+ shared FFN(x[t]) with
    weight 1, or sigmoid(opts.shared_gate[t])). x is [T, d] (any float dtype,
    taken exactly), logits [T, E] fp32. Routing is route(), or route_ex()
    with opts. Returns (out float64 [T', d], ids int [T', k], w float64
    [T', k]) for the requested tokens (all by default)."""
    x = np.asarray(x, dtype=np.float64)
    logits = np.asarray(logits, dtype=np.float32)
    T = x.shape[0]
    toks = list(range(T)) if tokens is None else list(tokens)
    out = np.zeros((len(toks), layer.d_model), dtype=np.float64)
    ids_all = np.zeros((len(toks), top_k), dtype=np.int64)
    w_all = np.zeros((len(toks), top_k), dtype=np.float64)
    sh = layer.shared_weights()
    for i, t in enumerate(toks):
        if opts is None:
            ids, w = route(logits[t], top_k, norm_topk_prob)
        else:
            ids, w = route_ex(logits[t], top_k, norm_topk_prob, opts)
        ids_all[i] = ids
        w_all[i] = w
        for j, e in enumerate(ids):
            W = layer.expert_weights(e)
            out[i] += w[j] * swiglu_expert(W["gate"], W["up"], W["down"], x[t])
        if sh is not None:
            ws = 1.0
            if opts is not None and opts.shared_gate is not None:
                ws = 1.0 / (1.0 + np.exp(-np.float64(opts.shared_gate.reshape(-1)[t])))
            out[i] += ws * swiglu_expert(sh["gate"], sh["up"], sh["down"], x[t])
    return out, ids_all, w_all


# --------------------------------------------------------------------------
# Stacked decode step (".smoe": Arch Block, RMS-norm eps 1e-6)
# --------------------------------------------------------------------------

def rms_norm(h: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """h / sqrt(mean(h^2) + eps) per token (unit gain), float64."""
    h = np.asarray(h, dtype=np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps)


def decode_step(layers: Sequence[OracleLayer], x: np.ndarray,
                logits_per_layer: Sequence[np.ndarray], top_k: int,
                norm_topk_prob: bool, eps: float = 1e-6) -> np.ndarray:
    """h = x; for each layer: h = h + MoE(rms_norm(h)). Returns h float64."""
    h = np.asarray(x, dtype=np.float64).copy()
    for layer, lg in zip(layers, logits_per_layer):
        y, _, _ = moe_forward(layer, rms_norm(h, eps), lg, top_k, norm_topk_prob)
        h = h + y
        layer.drop_cache()
    return h
