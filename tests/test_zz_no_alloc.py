"""smoe_moe_forward_noalloc (the variant for callers that cannot allocate:
its workspace is the library's static per-GPU scratch) against
smoe_moe_forward with a caller workspace, through the C ABI: two calls in a
row on each layer, the second with fewer tokens, so the second call runs on
scratch that still holds the first call's contents.

The two entry points launch the same kernels on the same inputs (the shared
expert on the caller's stream instead of a side stream), so routing and
outputs must agree bit for bit; the first call of each layer is also held to
the oracle at the parity bar (1e-3 relative L2, ids exact).
"""

import numpy as np
import pytest

import oracle as O
import synth
from helpers import DeviceLayer, random_layer, rel_l2

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _run(dl, x, lg, k, norm, x_dtype, noalloc):
    torch = _torch()
    smoe = dl.smoe
    T, d = x.shape
    xt = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    if x_dtype == "bf16":
        xt = xt.to(torch.bfloat16)
    code = smoe.SMOE_DTYPE_BF16 if x_dtype == "bf16" else smoe.SMOE_DTYPE_F32
    lt = torch.from_numpy(np.ascontiguousarray(lg, np.float32)).cuda()
    out = torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda")
    ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        smoe.smoe_moe_forward_noalloc(dl.handle, xt.data_ptr(), code, lt.data_ptr(), T, k, norm,
                                      out.data_ptr(), ids.data_ptr(), w.data_ptr(), stream)
    else:
        nws = smoe.smoe_workspace_bytes(dl.handle, T, k)
        # a workspace full of garbage: neither entry point may need clearing
        ws = torch.full((max(nws, 256),), 0xA5, dtype=torch.uint8, device="cuda")
        smoe.smoe_moe_forward(dl.handle, xt.data_ptr(), code, lt.data_ptr(), T, k, norm,
                              out.data_ptr(), ids.data_ptr(), w.data_ptr(), ws.data_ptr(), nws,
                              stream)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


CASES = [
    # d, ffn, E, k, bits, scales, shared, tokens of the two calls, x dtype
    (4096, 1536, 128, 8, 4, "f32", 0, (40, 1), "bf16"),
    (2048, 1408, 8, 3, 4, "f16", 2816, (64, 5), "f32"),
    (512, 320, 16, 4, 2, "f16", 0, (9, 3), "bf16"),
    (192, 64, 8, 8, 4, "f16", 128, (2, 1), "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"d{c[0]}_E{c[2]}_k{c[3]}_s{c[6]}_T{c[7][0]}-{c[7][1]}"
                                            for c in CASES])
def test_noalloc_matches_workspace_entry_point(case):
    _torch()
    d, ffn, E, k, bits, sd, shared, Ts, x_dtype = case
    hl = random_layer(900 + d + E, d, ffn, E, bits, sd, shared)
    dl = DeviceLayer(hl)
    try:
        for call, T in enumerate(Ts):
            r = synth.rng(910 + 7 * call + T)
            x = synth.normal_f32(r, (T, d))
            if x_dtype == "bf16":
                x = synth.round_to_bf16(x)
            lg = synth.normal_f32(r, (T, E))
            norm = call == 0
            na_out, na_ids, na_w = _run(dl, x, lg, k, norm, x_dtype, noalloc=True)
            ws_out, ws_ids, ws_w = _run(dl, x, lg, k, norm, x_dtype, noalloc=False)
            assert np.array_equal(na_ids, ws_ids), (call, T)
            assert np.array_equal(na_w, ws_w), (call, T)
            assert np.all(np.isfinite(na_out))
            assert np.array_equal(na_out, ws_out), (call, T, rel_l2(na_out, ws_out))
            if call == 0:
                ref, rids, rw = O.moe_forward(hl.oracle(), x, lg, k, norm)
                assert np.array_equal(na_ids, rids)
                assert np.allclose(na_w, rw, rtol=1e-5, atol=1e-7)
                assert rel_l2(na_out, ref) <= TOL
    finally:
        dl.close()


def test_noalloc_rejects_a_batch_beyond_the_scratch():
    torch = _torch()
    import quantised_moe_expert_amd as smoe
    hl = random_layer(950, 4096, 1536, 128, 4, "f32")
    dl = DeviceLayer(hl)
    try:
        T, k = 187, 8   # 187 tokens at top-8 need more than the 32 MB of scratch
        assert smoe.smoe_workspace_bytes(dl.handle, T, k) > smoe.SMOE_NOALLOC_SCRATCH_BYTES
        x = torch.zeros((T, 4096), dtype=torch.bfloat16, device="cuda")
        lg = torch.zeros((T, 128), dtype=torch.float32, device="cuda")
        out = torch.full((T, 4096), 7.0, dtype=torch.float32, device="cuda")
        with pytest.raises(smoe.SmoeError) as e:
            smoe.smoe_moe_forward_noalloc(dl.handle, x.data_ptr(), smoe.SMOE_DTYPE_BF16,
                                          lg.data_ptr(), T, k, True, out.data_ptr(), 0, 0,
                                          torch.cuda.current_stream().cuda_stream)
        assert e.value.code == smoe.SMOE_E_WORKSPACE
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())  # nothing was launched
    finally:
        dl.close()
