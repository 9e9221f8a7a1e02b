"""Routing variants on the GPU ("CMF v2 Format Specification", 2.2 MoE;
5. Masks section) against the oracle's route_ex / moe_forward with opts:
ids bit-exact, weights and outputs within tolerance."""

import numpy as np
import pytest

import oracle as O
import synth
from helpers import DeviceLayer, random_layer, rel_l2

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _torch():
    import torch
    # a GPU test fails where no device is visible (it must not pass by skipping)
    assert torch.cuda.is_available(), "no GPU visible to torch"
    return torch


def _variant(kind, E, r):
    """(oracle RouteOpts, kwargs for make_route_opts, bias array or None)."""
    bias = None
    kw = {}
    ro = {}
    if "sigmoid" in kind:
        kw["sigmoid"] = True
        ro["sigmoid"] = True
    if "bias" in kind:
        bias = (r.standard_normal(E) * 0.05).astype(np.float32)
        ro["expert_bias"] = bias
    if "scale" in kind:
        kw["scaling_factor"] = 2.5
        ro["scaling"] = 2.5
    if "mask" in kind:
        m = r.random(E) < 0.6
        m[:max(E // 4, 8)] = True  # enough routable experts for top_k
        kw["routable"] = [bool(v) for v in m]
        ro["mask"] = m
    return O.RouteOpts(**ro), kw, bias


KINDS = ["sigmoid", "bias", "sigmoid+bias", "scale", "mask", "sigmoid+bias+mask+scale"]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("T,E,k,norm", [(32, 128, 8, True), (5, 16, 4, False), (9, 512, 16, True)])
def test_route_ex_matches_oracle(kind, T, E, k, norm):
    torch = _torch()
    import quantised_moe_expert_amd as smoe
    r = synth.rng(500 + T + E + len(kind))
    lg = synth.normal_f32(r, (T, E))
    ro, kw, bias = _variant(kind, E, r)
    d_lg = torch.from_numpy(lg).cuda()
    d_bias = torch.from_numpy(bias).cuda() if bias is not None else None
    opts = smoe.make_route_opts(d_expert_bias=d_bias.data_ptr() if d_bias is not None else 0,
                                **kw)
    ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    smoe.smoe_route_ex(d_lg.data_ptr(), T, E, k, norm, opts, ids.data_ptr(), w.data_ptr(),
                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    for t in range(T):
        want, wt = O.route_ex(lg[t], k, norm, ro)
        assert ids[t].tolist() == want, (t, ids[t], want)
        assert np.allclose(w[t], wt, rtol=1e-5, atol=1e-7), (t, w[t], wt)


@pytest.mark.parametrize("kind", ["sigmoid+bias+mask+scale", "bias", "mask"])
@pytest.mark.parametrize("T", [1, 6])
def test_forward_ex_matches_oracle_with_shared_gate(kind, T):
    torch = _torch()
    import quantised_moe_expert_amd as smoe
    E, k = 16, 4
    hl = random_layer(600 + T, 512, 320, E, 4, "f32", shared_ffn=256)
    dl = DeviceLayer(hl)
    r = synth.rng(601 + T)
    x = synth.round_to_bf16(synth.normal_f32(r, (T, 512)))
    lg = synth.normal_f32(r, (T, E))
    gate = synth.normal_f32(r, (T,))
    ro, kw, bias = _variant(kind, E, r)
    ro.shared_gate = gate
    d_x = torch.from_numpy(x).cuda().to(torch.bfloat16)
    d_lg = torch.from_numpy(lg).cuda()
    d_gate = torch.from_numpy(gate).cuda()
    d_bias = torch.from_numpy(bias).cuda() if bias is not None else None
    opts = smoe.make_route_opts(d_expert_bias=d_bias.data_ptr() if d_bias is not None else 0,
                                d_shared_gate=d_gate.data_ptr(), **kw)
    out = torch.full((T, 512), float("nan"), dtype=torch.float32, device="cuda")
    ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    nws = smoe.smoe_workspace_bytes(dl.handle, T, k)
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")
    smoe.smoe_moe_forward_ex(dl.handle, d_x.data_ptr(), smoe.SMOE_DTYPE_BF16, d_lg.data_ptr(), T,
                             k, True, opts, out.data_ptr(), ids.data_ptr(), w.data_ptr(),
                             ws.data_ptr(), nws, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref, rids, rw = O.moe_forward(hl.oracle(), x, lg, k, True, opts=ro)
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert np.allclose(w.cpu().numpy(), rw, rtol=1e-5, atol=1e-7)
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o))
    assert rel_l2(o, ref) <= TOL


@pytest.mark.parametrize("sigmoid", [False, True])
def test_biased_near_tie_decided_in_float64(sigmoid):
    # the near-tie pinned for the oracle (CPU, closed form): two logits 2^-20
    # apart and a bias on expert 0 just short of the score gap. Float64
    # score + bias puts expert 1 first; an fp32 sum would tie and pick
    # expert 0.
    torch = _torch()
    import quantised_moe_expert_amd as smoe
    E = 2
    lg = np.array([[0.0, 2.0 ** -20]], np.float32)
    bias = np.zeros(E, np.float32)
    bias[0] = (2.0 ** -22 - 2.0 ** -31) if sigmoid else (2.0 ** -21 - 2.0 ** -30)
    ro = O.RouteOpts(sigmoid=sigmoid, expert_bias=bias)
    for k in (1, 2):
        want, wt = O.route_ex(lg[0], k, False, ro)
        assert want == [1, 0][:k]
        d_lg = torch.from_numpy(lg).cuda()
        d_bias = torch.from_numpy(bias).cuda()
        opts = smoe.make_route_opts(sigmoid=sigmoid, d_expert_bias=d_bias.data_ptr())
        ids = torch.full((1, k), -1, dtype=torch.int32, device="cuda")
        w = torch.empty((1, k), dtype=torch.float32, device="cuda")
        smoe.smoe_route_ex(d_lg.data_ptr(), 1, E, k, False, opts, ids.data_ptr(), w.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert ids.cpu().numpy()[0].tolist() == want
        assert np.allclose(w.cpu().numpy()[0], wt, rtol=1e-5, atol=1e-7)
