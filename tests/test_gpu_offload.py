"""Host offload ("SMOE Quantisation", Why Quantise; "CMF v2 Format
Specification", 2.2 MoE): experts in pinned host memory, read directly by the
kernels or fetched into a device cache. Outputs equal the device-resident
forward bit for bit and the oracle within tolerance; the cache counters add
up."""

import numpy as np
import pytest

import oracle as O
import synth
from helpers import to_device_aligned, SCALE_CODE, DeviceLayer, random_layer, rel_l2

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _torch():
    import torch
    # a GPU test fails where no device is visible (it must not pass by skipping)
    assert torch.cuda.is_available(), "no GPU visible to torch"
    return torch


class Offloaded:
    """A HostLayer registered for offload: the bank in pinned host memory, an
    optional device cache of `slots` blobs, the expert table."""

    def __init__(self, hl, slots):
        torch = _torch()
        import quantised_moe_expert_amd as smoe
        self.smoe, self.hl = smoe, hl
        self.host = to_device_aligned(hl.bank, pin_memory=True)
        self.shared = to_device_aligned(hl.shared_blob) if hl.shared_blob is not None else None
        self.cache = smoe.aligned_buffer(max(slots, 1) * hl.stride)
        self.cache.zero_()
        self.table = torch.zeros(hl.E, dtype=torch.int64, device="cuda:0")
        desc = smoe.make_desc(hl.d, hl.ffn, hl.E, hl.bits, hl.stride, SCALE_CODE[hl.scale_dtype],
                              hl.shared_ffn)
        self.h = smoe.smoe_offload_create(
            desc, self.host.data_ptr(), self.host.numel(),
            self.shared.data_ptr() if self.shared is not None else 0,
            self.shared.numel() if self.shared is not None else 0,
            self.cache.data_ptr() if slots else 0, slots * hl.stride, self.table.data_ptr())

    def forward(self, x, logits, k, norm):
        torch = _torch()
        smoe = self.smoe
        T = x.shape[0]
        xt = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda:0").to(torch.bfloat16)
        lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).to("cuda:0")
        out = torch.full((T, self.hl.d), float("nan"), dtype=torch.float32, device="cuda:0")
        n = smoe.smoe_offload_workspace_bytes(self.h, T, k)
        ws = torch.zeros(n, dtype=torch.uint8, device="cuda:0")
        smoe.smoe_offload_forward(self.h, xt.data_ptr(), smoe.SMOE_DTYPE_BF16, lg.data_ptr(), T, k,
                                  norm, out.data_ptr(), 0, 0, ws.data_ptr(), n,
                                  torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def stats(self):
        return self.smoe.smoe_offload_get_stats(self.h)

    def close(self):
        self.smoe.smoe_offload_free(self.h)


@pytest.mark.parametrize("T,slots,shared", [(1, 0, 0), (1, 4, 0), (6, 0, 0), (6, 5, 256),
                                            (1, 16, 0), (6, 1, 0),
                                            # the 1-4-token launches through the table
                                            (3, 0, 256), (4, 2, 0), (1, 0, 512)])
def test_offload_equals_device_forward_and_oracle(T, slots, shared):
    _torch()
    d, ffn, E, k = 512, 256, 16, 4
    hl = random_layer(600 + T + slots, d, ffn, E, 4, "f32", shared_ffn=shared)
    r = synth.rng(610 + slots)
    dl = DeviceLayer(hl)
    off = Offloaded(hl, slots)
    print(f"offload T={T} slots={slots} shared={shared}", flush=True)
    try:
        unique, touched = 0, set()
        for step in range(5):
            x = synth.round_to_bf16(synth.normal_f32(r, (T, d)))
            logits = synth.normal_f32(r, (T, E))
            if step == 4:
                logits = prev  # a repeated routing: resident experts hit
            got = off.forward(x, logits, k, True)
            want, _, _ = dl.forward(x, logits, k, True, "bf16")
            assert np.array_equal(got, want), step
            ref, _, _ = O.moe_forward(hl.oracle(), x, logits, k, True)
            assert rel_l2(got, ref) <= TOL
            sel = {e for t in range(T) for e in O.route(logits[t], k, True)[0]}
            unique += len(sel)
            touched |= sel
            prev = logits
        st = off.stats()
        assert st.forwards == 5
        if slots:
            assert st.hits + st.fetched + st.direct == unique
            assert st.bytes_fetched == st.fetched * O.expert_layout(d, ffn, 4, "f32").raw_size
            assert st.fetched >= 1
            if slots >= T * k:
                assert st.direct == 0
            if slots >= E:  # nothing is ever evicted
                assert st.fetched == len(touched)
        else:
            assert st.hits == st.fetched == st.direct == 0
    finally:
        off.close()
        dl.close()


def test_cache_keeps_recent_experts():
    """With room for every expert, a second pass over the same routings only
    hits."""
    _torch()
    d, ffn, E, k, T = 256, 128, 8, 2, 3
    hl = random_layer(620, d, ffn, E, 2, "f16")
    r = synth.rng(621)
    off = Offloaded(hl, E)
    try:
        xs = [synth.round_to_bf16(synth.normal_f32(r, (T, d))) for _ in range(3)]
        lgs = [synth.normal_f32(r, (T, E)) for _ in range(3)]
        for x, lg in zip(xs, lgs):
            off.forward(x, lg, k, False)
        first = off.stats()
        outs = [off.forward(x, lg, k, False) for x, lg in zip(xs, lgs)]
        second = off.stats()
        assert second.fetched == first.fetched and second.direct == 0
        touched = {e for lg in lgs for t in range(T) for e in O.route(lg[t], k, False)[0]}
        assert first.fetched == len(touched)
        for x, lg, got in zip(xs, lgs, outs):
            ref, _, _ = O.moe_forward(hl.oracle(), x, lg, k, False)
            assert rel_l2(got, ref) <= TOL
    finally:
        off.close()


def test_pageable_host_memory_is_refused():
    torch = _torch()
    import quantised_moe_expert_amd as smoe
    hl = random_layer(630, 256, 128, 4, 4, "f32")
    table = torch.zeros(4, dtype=torch.int64, device="cuda:0")
    desc = smoe.make_desc(256, 128, 4, 4, hl.stride)
    pageable = np.zeros(hl.bank.size + 4096, np.uint8)
    p = (pageable.ctypes.data + 4095) // 4096 * 4096
    with pytest.raises(smoe.SmoeError) as e:
        smoe.smoe_offload_create(desc, p, hl.bank.size, 0, 0, 0, 0, table.data_ptr())
    assert e.value.code == smoe.SMOE_E_LAYOUT
