"""Test helpers: build seeded synthetic layers on the host (random draws from
synth, blob assembly by the oracle), upload them, and run the HIP path
through the C ABI binding."""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

import oracle as O
import synth

SCALE_CODE = {"f32": 0, "f16": 1}


@dataclasses.dataclass
class HostLayer:
    d: int
    ffn: int
    E: int
    bits: int
    scale_dtype: str
    shared_ffn: int
    bank: np.ndarray          # [E * stride] uint8
    stride: int
    shared_blob: Optional[np.ndarray]

    def oracle(self) -> O.OracleLayer:
        return O.OracleLayer(self.d, self.ffn, self.E, self.bits, self.bank, self.stride,
                             self.scale_dtype, self.shared_ffn, self.shared_blob)


def random_blob(r, layout: O.ExpertLayout, zero_scales: bool = False,
                mu: float = float(np.log(0.02)), sigma: float = 0.5) -> np.ndarray:
    st = np.float32 if layout.scale_dtype == "f32" else np.float16
    t = {}
    for name, span in layout.spans().items():
        codes = synth.uniform_bytes(r, span.codes_bytes)
        sc = synth.lognormal_f32(r, span.n_scales, mu, sigma).astype(st)
        if zero_scales:
            sc[:] = 0
        t[name] = (codes, sc)
    return O.build_expert_blob(layout, t)


def random_layer(seed: int, d: int, ffn: int, E: int, bits: int, scale_dtype: str = "f32",
                 shared_ffn: int = 0, stride_extra_pages: int = 0) -> HostLayer:
    """Codes uniform (random bytes), scales lognormal(ln 0.02, 0.5)."""
    r = synth.rng(seed)
    L = O.expert_layout(d, ffn, bits, scale_dtype)
    stride = L.padded_size + stride_extra_pages * O.BLOB_ALIGN
    bank = np.zeros(E * stride, dtype=np.uint8)
    for e in range(E):
        bank[e * stride: e * stride + L.padded_size] = random_blob(r, L)
    sh = None
    if shared_ffn:
        sh = random_blob(r, O.expert_layout(d, shared_ffn, bits, scale_dtype))
    return HostLayer(d, ffn, E, bits, scale_dtype, shared_ffn, bank, stride, sh)


def tiny_swiglu_layer(seed: int = 0):
    """The tiny single-expert case: x fp32 N(0,1); gate/up/down fp32
    N(0, 0.02) with 1% x10 outliers, quantised Q4 by the MSE grid."""
    r = synth.rng(seed)
    x = synth.normal_f32(r, (1, 256))
    L = O.expert_layout(256, 128, 4, "f32")
    t = {}
    for name, span in L.spans().items():
        W = synth.outlier_weights_f32(r, (span.rows, span.cols))
        t[name] = O.quantise_tensor(W, 4, "f32")
    blob = O.build_expert_blob(L, t)
    return x, HostLayer(256, 128, 1, 4, "f32", 0, blob, L.padded_size, None)


def to_device_aligned(host: np.ndarray, device="cuda:0", pin_memory: bool = False):
    """Bytes of `host` in a 16 KB-aligned device (or pinned host) buffer, as
    the library requires for expert banks and shared blobs."""
    import torch
    import quantised_moe_expert_amd as smoe
    buf = smoe.aligned_buffer(host.size, device=device, pin_memory=pin_memory)
    buf.copy_(torch.from_numpy(np.ascontiguousarray(host).reshape(-1)))
    return buf


def oracle_by_expert(ol: O.OracleLayer, x: np.ndarray, logits: np.ndarray, k: int,
                     norm: bool):
    """The oracle's layer output for every token, evaluated expert by expert:
    each selected expert is dequantised once, into three reused arrays, and
    applied to every token routed to it, so a batch over many experts never
    holds more than one dense expert. Same terms as O.moe_forward,
    out[t] = sum_j w[t, j] FFN_{ids[t, j]}(x[t]) (+ the shared expert with
    weight 1); only the order of the per-token sum differs."""
    T = x.shape[0]
    X = np.asarray(x, np.float64)
    routes = [O.route(logits[t], k, norm) for t in range(T)]
    by_e = {}
    for t, (ids, _) in enumerate(routes):
        for j, e in enumerate(ids):
            by_e.setdefault(e, []).append((t, j))
    out = np.zeros((T, ol.d_model))
    bufs = {n: np.empty(sp.rows * sp.cols, np.float64) for n, sp in ol.layout.spans().items()}
    for e in sorted(by_e):
        W = ol.expert_weights_into(e, bufs)
        for t, j in by_e[e]:
            out[t] += routes[t][1][j] * O.swiglu_expert(W["gate"], W["up"], W["down"], X[t])
    S = ol.shared_weights()
    if S is not None:
        for t in range(T):
            out[t] += O.swiglu_expert(S["gate"], S["up"], S["down"], X[t])
        ol.drop_cache()
    return out, routes


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / n) if n > 0 else float(np.linalg.norm(a - b))


class DeviceLayer:
    """A HostLayer uploaded to the GPU and registered with the library."""

    def __init__(self, hl: HostLayer, device="cuda:0", bank_tensor=None, shared_tensor=None):
        import torch
        import quantised_moe_expert_amd as smoe
        self.hl = hl
        self.smoe = smoe
        self.bank = bank_tensor if bank_tensor is not None else \
            to_device_aligned(hl.bank, device)
        self.shared = None
        if hl.shared_blob is not None:
            self.shared = shared_tensor if shared_tensor is not None else \
                to_device_aligned(hl.shared_blob, device)
        desc = smoe.make_desc(hl.d, hl.ffn, hl.E, hl.bits, hl.stride, SCALE_CODE[hl.scale_dtype],
                              hl.shared_ffn)
        self.handle = smoe.smoe_load_blobs(
            desc, self.bank.data_ptr(), self.bank.numel(),
            self.shared.data_ptr() if self.shared is not None else 0,
            self.shared.numel() if self.shared is not None else 0)

    def close(self):
        if self.handle:
            self.smoe.smoe_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def forward(self, x: np.ndarray, logits: np.ndarray, k: int, norm: bool,
                x_dtype: str = "bf16", device="cuda:0"):
        """Returns (out float32 [T, d], ids int32 [T, k], w float32 [T, k])."""
        import torch
        smoe = self.smoe
        T = x.shape[0]
        xt = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)
        if x_dtype == "bf16":
            xt = xt.to(torch.bfloat16)
        lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).to(device)
        out = torch.full((T, self.hl.d), float("nan"), dtype=torch.float32, device=device)
        ids = torch.full((max(T, 1), k), -1, dtype=torch.int32, device=device)
        w = torch.full((max(T, 1), k), float("nan"), dtype=torch.float32, device=device)
        nws = smoe.smoe_workspace_bytes(self.handle, T, k)
        ws = torch.zeros(max(nws, 256), dtype=torch.uint8, device=device)
        smoe.smoe_moe_forward(self.handle, xt.data_ptr(),
                              smoe.SMOE_DTYPE_BF16 if x_dtype == "bf16" else smoe.SMOE_DTYPE_F32,
                              lg.data_ptr(), T, k, norm, out.data_ptr(), ids.data_ptr(),
                              w.data_ptr(), ws.data_ptr(), nws,
                              torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        return out.cpu().numpy(), ids.cpu().numpy()[:T], w.cpu().numpy()[:T]
