"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

Bars: routing ids bit-exact (set and order, ties to the lower id); routing
weights within 1e-5 relative (fp32 exp against the oracle's fp64); layer
outputs within 1e-3 relative L2, overall and per token.
"""

import numpy as np
import pytest

import oracle as O
import synth
from helpers import DeviceLayer, oracle_by_expert, random_layer, rel_l2, tiny_swiglu_layer

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _x(r, T, d, dtype):
    x = synth.normal_f32(r, (T, d))
    return synth.round_to_bf16(x) if dtype == "bf16" else x


def _check_layer(hl, x, logits, k, norm, x_dtype, tokens=None, dl=None):
    dl = dl or DeviceLayer(hl)
    out, ids, w = dl.forward(x, logits, k, norm, x_dtype)
    ref, rids, rw = O.moe_forward(hl.oracle(), x, logits, k, norm, tokens=tokens)
    toks = list(range(x.shape[0])) if tokens is None else list(tokens)
    # routing of every token is exact
    for t in range(x.shape[0]):
        want, wt = O.route(logits[t], k, norm)
        assert ids[t].tolist() == want, (t, ids[t], want)
        assert np.allclose(w[t], wt, rtol=1e-5, atol=1e-7), (t, w[t], wt)
    sel = out[toks]
    assert np.all(np.isfinite(sel))
    err = rel_l2(sel, ref)
    per_tok = [rel_l2(sel[i], ref[i]) for i in range(len(toks))]
    assert err <= TOL and max(per_tok) <= TOL, (err, max(per_tok))
    return err


# ------------------------------------------------------------------ routing --

@pytest.mark.parametrize("T,E,k,norm", [(1, 128, 8, True), (32, 128, 8, True), (8, 64, 6, False),
                                        (5, 8, 8, True), (3, 1, 1, True), (17, 512, 16, False),
                                        (1024, 128, 8, True)])
def test_route_matches_oracle(T, E, k, norm):
    torch = _torch()
    import quantised_moe_expert_amd as smoe
    r = synth.rng(100 + T + E)
    lg = synth.normal_f32(r, (T, E))
    d_lg = torch.from_numpy(lg).cuda()
    ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    smoe.smoe_route(d_lg.data_ptr(), T, E, k, norm, ids.data_ptr(), w.data_ptr(),
                    torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    for t in range(T):
        want, wt = O.route(lg[t], k, norm)
        assert ids[t].tolist() == want
        assert np.allclose(w[t], wt, rtol=1e-5, atol=1e-7)


def test_route_ties_go_to_lower_id():
    torch = _torch()
    import quantised_moe_expert_amd as smoe
    r = synth.rng(7)
    T, E, k = 64, 128, 8
    lg = (r.integers(0, 3, (T, E)) * 0.5).astype(np.float32)  # massive ties
    lg[3] = 0.0                                               # all equal
    d_lg = torch.from_numpy(lg).cuda()
    ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    smoe.smoe_route(d_lg.data_ptr(), T, E, k, True, ids.data_ptr(), w.data_ptr(), 0)
    torch.cuda.synchronize()
    ids = ids.cpu().numpy()
    for t in range(T):
        assert ids[t].tolist() == O.route(lg[t], k, True)[0]
    assert ids[3].tolist() == list(range(8))


# ------------------------------------------------------- small full parity --

SMALL = [
    # d, ffn, E, k, T, bits, scales, norm, shared
    (512, 320, 16, 4, 5, 4, "f32", True, 0),
    (512, 320, 16, 4, 5, 2, "f16", False, 0),
    (192, 64, 8, 8, 3, 4, "f16", True, 128),
    (1024, 192, 32, 16, 9, 2, "f32", True, 0),
    (256, 128, 1, 1, 1, 4, "f32", True, 0),
    (2048, 1408, 4, 2, 2, 4, "f32", False, 2816),
    (2048, 1408, 6, 3, 3, 2, "f16", True, 2816),
    (640, 448, 12, 5, 7, 4, "f32", True, 0),
    # shared experts 4x and 3x the routed ffn (run as extra slots of the
    # routed launches) and one that is not a multiple (launches of its own)
    (512, 320, 16, 4, 5, 4, "f16", True, 1280),
    (640, 448, 12, 5, 7, 2, "f32", False, 1344),
    (512, 320, 16, 4, 6, 4, "f32", True, 448),
    # one token: the single-launch path for these widths ...
    (512, 320, 16, 4, 1, 4, "f32", True, 0),
    (512, 320, 16, 4, 1, 2, "f16", False, 0),
    (2048, 1408, 64, 6, 1, 4, "f16", False, 0),
    (2048, 1408, 64, 6, 1, 2, "f32", True, 0),
    (4096, 1536, 128, 16, 1, 2, "f32", True, 0),
    (4096, 1536, 512, 1, 1, 4, "f16", True, 0),
    (256, 128, 4, 4, 1, 2, "f32", True, 0),
    # ... and one-token shapes that take the multi-kernel path
    (192, 64, 8, 8, 1, 4, "f16", True, 128),
    (1024, 192, 32, 16, 1, 2, "f32", True, 0),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"d{c[0]}_f{c[1]}_E{c[2]}_k{c[3]}_T{c[4]}_q{c[5]}"
                                            f"_{c[6]}_n{int(c[7])}_s{c[8]}" for c in SMALL])
@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_small_layers(case, x_dtype):
    _torch()
    d, ffn, E, k, T, bits, sd, norm, shared = case
    hl = random_layer(1000 + d + ffn + E, d, ffn, E, bits, sd, shared)
    r = synth.rng(55 + T)
    x = _x(r, T, d, x_dtype)
    lg = synth.normal_f32(r, (T, E))
    _check_layer(hl, x, lg, k, norm, x_dtype)


# Two to four tokens take the small-batch path: routing and grouping inside
# the gate/up launch (every workgroup), the grouped layout published by the
# first workgroup, then the grouped down stage and the combine.
SMALL_BATCH = [
    # d, ffn, E, k, T, bits, scales, norm, shared
    (4096, 1536, 128, 8, 3, 4, "f32", True, 0),
    (1024, 256, 512, 16, 4, 4, "f16", True, 768),
    (512, 320, 16, 16, 2, 2, "f32", True, 640),
    (2048, 1408, 64, 6, 4, 4, "f32", False, 2816),
    (768, 192, 40, 7, 4, 2, "f16", False, 0),
    # one token with a shared expert; a row count that leaves the last
    # workgroup of the down stage a partial block (12 rows per workgroup);
    # pairs whose h exceeds the down stage's LDS (grouped down and combine)
    (2048, 1408, 64, 6, 1, 4, "f16", False, 2816),
    (2560, 512, 32, 6, 3, 4, "f32", True, 1024),
    (1024, 1536, 64, 16, 4, 4, "f16", True, 0),
]


@pytest.mark.parametrize("case", SMALL_BATCH,
                         ids=[f"d{c[0]}_f{c[1]}_E{c[2]}_k{c[3]}_T{c[4]}_q{c[5]}_{c[6]}"
                              f"_n{int(c[7])}_s{c[8]}" for c in SMALL_BATCH])
@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_small_batch_path(case, x_dtype):
    _torch()
    d, ffn, E, k, T, bits, sd, norm, shared = case
    hl = random_layer(3100 + d + E + T, d, ffn, E, bits, sd, shared)
    r = synth.rng(3200 + T + E)
    x = _x(r, T, d, x_dtype)
    lg = synth.normal_f32(r, (T, E))
    _check_layer(hl, x, lg, k, norm, x_dtype)


# Five to sixteen tokens: the grouped routing and gate/up stages, then the
# down stage and the combine in one launch, the pairs' h staged in LDS in
# chunks of whole experts (several chunks for all but the smallest rows).
SMALL_DOWN = [
    # d, ffn, E, k, T, bits, scales, norm, shared
    (4096, 1536, 128, 8, 8, 4, "f32", True, 0),
    (1024, 1536, 64, 16, 12, 4, "f16", True, 0),
    (2048, 1408, 64, 6, 16, 4, "f32", False, 2816),
    (768, 192, 40, 7, 16, 2, "f16", False, 0),
    (2560, 512, 32, 6, 9, 2, "f32", True, 1024),
]


@pytest.mark.parametrize("case", SMALL_DOWN,
                         ids=[f"d{c[0]}_f{c[1]}_E{c[2]}_k{c[3]}_T{c[4]}_q{c[5]}_{c[6]}"
                              f"_n{int(c[7])}_s{c[8]}" for c in SMALL_DOWN])
def test_small_down_path(case):
    _torch()
    d, ffn, E, k, T, bits, sd, norm, shared = case
    hl = random_layer(3500 + d + E + T, d, ffn, E, bits, sd, shared)
    r = synth.rng(3600 + T + E)
    x = _x(r, T, d, "bf16")
    lg = synth.normal_f32(r, (T, E))
    _check_layer(hl, x, lg, k, norm, "bf16")


def test_small_batch_path_ties_and_shared_experts():
    """Logits drawn from a handful of values, so every token has ties (to the
    lower expert id) and several tokens pick the same experts."""
    _torch()
    d, ffn, E, k, T = 512, 192, 24, 6, 4
    hl = random_layer(3300, d, ffn, E, 4, "f16", 384)
    r = synth.rng(3301)
    x = _x(r, T, d, "bf16")
    lg = np.round(synth.normal_f32(r, (T, E)) * 2.0).astype(np.float32) / 2.0
    lg[1] = lg[0]  # two tokens with identical routing
    _check_layer(hl, x, lg, k, True, "bf16")


# Routing and grouping of batches around 64 tokens, up to 16 selections per
# token, 512 experts, every expert selected, and one selection per token.
@pytest.mark.parametrize("T,E,k", [(64, 256, 16), (65, 256, 16), (64, 512, 8), (2, 3, 3),
                                   (33, 64, 1)])
def test_route_group_batch_edges(T, E, k):
    _torch()
    hl = random_layer(90 + T + E, 256, 128, E, 4, "f16")
    r = synth.rng(91 + T)
    _check_layer(hl, _x(r, T, 256, "bf16"), synth.normal_f32(r, (T, E)), k, True, "bf16")


# the widest activation vectors the library registers (wider ones are
# refused at load): one token, and batches through the grouped stages
@pytest.mark.parametrize("d,ffn,shared", [(11392, 128, 0), (128, 19072, 19072)])
@pytest.mark.parametrize("T", [1, 3])
@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_maximum_widths(d, ffn, shared, T, x_dtype):
    _torch()
    hl = random_layer(70 + d + T, d, ffn, 4, 4, "f16", shared)
    r = synth.rng(71 + T)
    _check_layer(hl, _x(r, T, d, x_dtype), synth.normal_f32(r, (T, 4)), 2, True, x_dtype)


def test_stride_larger_than_padded_blob():
    _torch()
    hl = random_layer(5, 512, 320, 8, 4, "f32", stride_extra_pages=3)
    r = synth.rng(6)
    x = _x(r, 4, 512, "bf16")
    _check_layer(hl, x, synth.normal_f32(r, (4, 8)), 3, True, "bf16")


def test_zero_tokens_is_a_no_op():
    torch = _torch()
    import quantised_moe_expert_amd as smoe
    hl = random_layer(9, 256, 128, 4, 4)
    dl = DeviceLayer(hl)
    out = torch.full((1, 256), 3.0, device="cuda")
    smoe.smoe_moe_forward(dl.handle, 0, smoe.SMOE_DTYPE_BF16, 0, 0, 2, True, out.data_ptr(), 0, 0,
                          0, 0, 0)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


def test_repeat_calls_are_bitwise_identical():
    _torch()
    hl = random_layer(11, 1024, 320, 16, 4)
    r = synth.rng(12)
    x = _x(r, 6, 1024, "bf16")
    lg = synth.normal_f32(r, (6, 16))
    dl = DeviceLayer(hl)
    a = dl.forward(x, lg, 4, True)[0]
    b = dl.forward(x, lg, 4, True)[0]
    assert np.array_equal(a, b)


@pytest.mark.parametrize("T", [3, 40])
def test_shared_expert_side_stream_back_to_back(T):
    """The shared expert runs on the layer's own stream, forked from and
    joined back into the caller's: several forwards enqueued back to back on
    one (non-default) stream with one workspace, no synchronisation between
    them, each equal bit for bit to the same forward run alone."""
    torch = _torch()
    import quantised_moe_expert_amd as smoe
    d, ffn, E, k, sh = 512, 256, 16, 4, 384
    hl = random_layer(4500 + T, d, ffn, E, 4, "f32", shared_ffn=sh)
    r = synth.rng(4501 + T)
    dl = DeviceLayer(hl)
    xs = [_x(r, T, d, "bf16") for _ in range(4)]
    lgs = [synth.normal_f32(r, (T, E)) for _ in range(4)]
    alone = [dl.forward(x, lg, k, True)[0] for x, lg in zip(xs, lgs)]
    stream = torch.cuda.Stream()
    nws = smoe.smoe_workspace_bytes(dl.handle, T, k)
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda:0")
    dx = [torch.from_numpy(x).cuda().to(torch.bfloat16) for x in xs]
    dlg = [torch.from_numpy(lg).cuda() for lg in lgs]
    outs = [torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda:0")
            for _ in range(4)]
    torch.cuda.synchronize()
    for i in range(4):
        smoe.smoe_moe_forward(dl.handle, dx[i].data_ptr(), smoe.SMOE_DTYPE_BF16,
                              dlg[i].data_ptr(), T, k, True, outs[i].data_ptr(), 0, 0,
                              ws.data_ptr(), nws, stream.cuda_stream)
    stream.synchronize()
    for i in range(4):
        assert np.array_equal(outs[i].cpu().numpy(), alone[i]), i
    ref, _, _ = O.moe_forward(hl.oracle(), xs[3], lgs[3], k, True)
    assert rel_l2(alone[3], ref) <= TOL
    dl.close()


def test_single_token_repeated_launches_and_streams():
    # the single-launch kernel's grid barrier must stay consistent across many
    # launches, across layers, and across streams
    torch = _torch()
    hl = random_layer(21, 4096, 1536, 16, 4)
    hl2 = random_layer(22, 4096, 1536, 16, 4)
    dl, dl2 = DeviceLayer(hl), DeviceLayer(hl2)
    r = synth.rng(23)
    x = _x(r, 1, 4096, "bf16")
    lgs = [synth.normal_f32(r, (1, 16)) for _ in range(3)]
    ref = [O.moe_forward(hl.oracle(), x, lg, 8, True)[0] for lg in lgs]
    ref2 = O.moe_forward(hl2.oracle(), x, lgs[0], 8, True)[0]
    first = dl.forward(x, lgs[0], 8, True)[0]
    assert rel_l2(first, ref[0]) <= TOL
    for i in range(40):
        out = dl.forward(x, lgs[i % 3], 8, True)[0]
        assert rel_l2(out, ref[i % 3]) <= TOL, i
        if i % 3 == 0:
            assert np.array_equal(out, first)
        if i % 5 == 0:
            assert rel_l2(dl2.forward(x, lgs[0], 8, True)[0], ref2) <= TOL
    s2 = torch.cuda.Stream()
    with torch.cuda.stream(s2):
        out = dl.forward(x, lgs[1], 8, True)[0]
    assert rel_l2(out, ref[1]) <= TOL


def test_single_token_workspace_reuse():
    # many one-token forwards on one workspace, two layers, alternating
    torch = _torch()
    import quantised_moe_expert_amd as smoe
    hl = random_layer(31, 4096, 1536, 16, 4)
    hl2 = random_layer(32, 4096, 1536, 16, 4)
    dl, dl2 = DeviceLayer(hl), DeviceLayer(hl2)
    r = synth.rng(33)
    x = _x(r, 1, 4096, "bf16")
    lgs = [synth.normal_f32(r, (1, 16)) for _ in range(4)]
    refs = [O.moe_forward(hl.oracle(), x, lg, 8, True)[0] for lg in lgs]
    refs2 = [O.moe_forward(hl2.oracle(), x, lg, 8, True)[0] for lg in lgs]
    nws = smoe.smoe_workspace_bytes(dl.handle, 1, 8)
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")
    xt = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda().to(torch.bfloat16)
    out = torch.empty((1, 4096), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for i in range(24):
        lg = torch.from_numpy(lgs[i % 4]).cuda()
        layer, ref = (dl, refs) if i % 2 == 0 else (dl2, refs2)
        smoe.smoe_moe_forward(layer.handle, xt.data_ptr(), smoe.SMOE_DTYPE_BF16, lg.data_ptr(), 1,
                              8, True, out.data_ptr(), 0, 0, ws.data_ptr(), nws, s)
        torch.cuda.synchronize()
        assert rel_l2(out.cpu().numpy(), ref[i % 4]) <= TOL, i


@pytest.mark.parametrize("T,shared", [(3, 0), (2, 640)])
def test_decode_step_multi_token_small(T, shared):
    torch = _torch()
    import quantised_moe_expert_amd as smoe
    hls = [random_layer(40 + l + shared, 512, 320, 16, 4, "f16", shared) for l in range(3)]
    r = synth.rng(41 + T)
    x = synth.normal_f32(r, (T, 512))
    lg = synth.normal_f32(r, (3, T, 16))
    dls = [DeviceLayer(h) for h in hls]
    h_d = torch.from_numpy(x.copy()).cuda()
    lg_d = torch.from_numpy(lg).cuda()
    nws = smoe.smoe_workspace_bytes(dls[0].handle, T, 4)
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")
    smoe.smoe_decode_step([d.handle for d in dls], h_d.data_ptr(), lg_d.data_ptr(), T, 4, False,
                          1e-6, ws.data_ptr(), nws, 0)
    torch.cuda.synchronize()
    got = h_d.cpu().numpy()
    ref = O.decode_step([h.oracle() for h in hls], x, list(lg), 4, False, 1e-6)
    assert rel_l2(got - x, ref - x) <= TOL
    for t in range(T):
        assert rel_l2(got[t] - x[t], ref[t] - x[t]) <= TOL


def test_activation_range_is_scale_free():
    # outputs scale linearly with x; the per-vector power-of-two rescale keeps
    # fp16 in range for large and tiny activations
    _torch()
    hl = random_layer(13, 512, 320, 8, 4)
    dl = DeviceLayer(hl)
    r = synth.rng(14)
    x = synth.normal_f32(r, (2, 512))
    lg = synth.normal_f32(r, (2, 8))
    for s in (2.0 ** 40, 2.0 ** -40):
        xs = (x * np.float32(s)).astype(np.float32)
        out = dl.forward(xs, lg, 2, True, "f32")[0]
        ref = O.moe_forward(hl.oracle(), xs, lg, 2, True)[0]
        assert rel_l2(out, ref) <= TOL
        out1 = dl.forward(xs[:1], lg[:1], 2, True, "f32")[0]
        assert rel_l2(out1, ref[:1]) <= TOL


# ------------------------------------------------------------ the workloads --

def test_tiny_swiglu_workload():
    _torch()
    x, hl = tiny_swiglu_layer(0)
    _check_layer(hl, x, np.zeros((1, 1), np.float32), 1, True, "f32")


def test_qwen235b_q4_b1_full():
    _torch()
    W = synth.WORKLOADS["qwen235b_q4_b1"]
    hl = random_layer(W.seed, W.d_model, W.ffn_dim, W.num_experts, W.bits)
    r = synth.rng(W.seed + 1000)
    x = _x(r, 1, W.d_model, "bf16")
    lg = synth.normal_f32(r, (1, W.num_experts))
    _check_layer(hl, x, lg, W.top_k, W.norm_topk_prob, "bf16")


@pytest.mark.parametrize("name", ["qwen235b_q4_b32", "qwen235b_q2_b32"])
def test_qwen235b_b32_every_token(name):
    # "CMF v2 Format Specification", 2.2 MoE: out[t] = sum_j w_j FFN_j(x[t])
    # for each of the 32 tokens (about 112 distinct experts, each dequantised
    # once by the oracle and applied to all of its tokens)
    _torch()
    W = synth.WORKLOADS[name]
    hl = random_layer(W.seed + W.bits, W.d_model, W.ffn_dim, W.num_experts, W.bits)
    r = synth.rng(W.seed + 2000)
    x = _x(r, W.n_tokens, W.d_model, "bf16")
    lg = synth.normal_f32(r, (W.n_tokens, W.num_experts))
    print(f"{name}: all {W.n_tokens} tokens", flush=True)
    out, ids, w = DeviceLayer(hl).forward(x, lg, W.top_k, W.norm_topk_prob, "bf16")
    ref, routes = oracle_by_expert(hl.oracle(), x, lg, W.top_k, W.norm_topk_prob)
    for t, (want, wt) in enumerate(routes):
        assert ids[t].tolist() == want, (t, ids[t], want)
        assert np.allclose(w[t], wt, rtol=1e-5, atol=1e-7)
    assert np.all(np.isfinite(out))
    per_tok = [rel_l2(out[t], ref[t]) for t in range(W.n_tokens)]
    assert rel_l2(out, ref) <= TOL and max(per_tok) <= TOL, (rel_l2(out, ref), max(per_tok))


# Prefill-sized batches: 32 pairs per expert fill whole 16-token chunks; with
# d = 2304 a 16-token chunk needs more than 64 KB of LDS, so the gate/up
# stage runs in eight-wave workgroups.
@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_prefill_sized_batch_eight_wave_chunks(x_dtype):
    _torch()
    hl = random_layer(4242, 2304, 256, 8, 4, "f32")
    r = synth.rng(4243)
    T = 128
    x = _x(r, T, 2304, x_dtype)
    lg = synth.normal_f32(r, (T, 8))
    _check_layer(hl, x, lg, 2, True, x_dtype)


@pytest.mark.parametrize("bits,sd,d,ffn", [(2, "f16", 640, 192), (4, "f16", 576, 320),
                                           (4, "f32", 1024, 512)])
def test_k_sliced_stage_many_tokens_per_expert(bits, sd, d, ffn):
    """Slots of 64 tokens and more (several 64-token chunks per slot, ragged
    last chunks), K slices with a partial last slice, rows that are not a
    multiple of the 64/128-row blocks, scale groups per row not a multiple
    of four (scalar scale loads)."""
    _torch()
    hl = random_layer(4300 + bits + d, d, ffn, 4, bits, sd)
    r = synth.rng(4301 + d)
    T = 300
    x = _x(r, T, d, "bf16")
    lg = synth.normal_f32(r, (T, 4))
    _check_layer(hl, x, lg, 2, True, "bf16")


@pytest.mark.parametrize("E,T,d,ffn,sd", [(12, 400, 512, 256, "f32"), (20, 640, 576, 320, "f16")])
def test_k_sliced_stage_xcd_order_with_remainder_slots(E, T, d, ffn, sd):
    """Eight or more slots: the K-sliced stage hands each XCD whole slots
    (the first multiple of eight) and keeps the plain order for the rest;
    every token of every slot is checked."""
    _torch()
    hl = random_layer(4400 + E, d, ffn, E, 4, sd)
    r = synth.rng(4401 + E)
    x = _x(r, T, d, "bf16")
    lg = synth.normal_f32(r, (T, E))
    _check_layer(hl, x, lg, 2, True, "bf16")


def test_qwen235b_q4_t512_sampled():
    _torch()
    W = synth.WORKLOADS["qwen235b_q4_t512"]
    hl = random_layer(W.seed, W.d_model, W.ffn_dim, W.num_experts, W.bits)
    r = synth.rng(W.seed + 4000)
    x = _x(r, W.n_tokens, W.d_model, "bf16")
    lg = synth.normal_f32(r, (W.n_tokens, W.num_experts))
    _check_layer(hl, x, lg, W.top_k, W.norm_topk_prob, "bf16", tokens=[0, 257, 511])


def test_max_tokens_grouping_beyond_64k_lds():
    # 4096 tokens over 128 experts: the grouping's token bitmasks take 65.5 KB,
    # and its 32768 pairs take two batches of id loads; every token is checked
    # (a pair placed in another's position changes two tokens' outputs)
    _torch()
    import quantised_moe_expert_amd as smoe
    T = smoe.SMOE_MAX_TOKENS
    hl = random_layer(77, 256, 128, 128, 4, "f16")
    r = synth.rng(78)
    x = _x(r, T, 256, "bf16")
    lg = synth.normal_f32(r, (T, 128))
    print(f"grouping: all {T} tokens, d 256, ffn 128, 128 experts, top-8", flush=True)
    out, ids, w = DeviceLayer(hl).forward(x, lg, 8, True, "bf16")
    ref, routes = oracle_by_expert(hl.oracle(), x, lg, 8, True)
    for t, (want, wt) in enumerate(routes):
        assert ids[t].tolist() == want, (t, ids[t], want)
        assert np.allclose(w[t], wt, rtol=1e-5, atol=1e-7)
    assert np.all(np.isfinite(out))
    per_tok = [rel_l2(out[t], ref[t]) for t in range(T)]
    assert rel_l2(out, ref) <= TOL and max(per_tok) <= TOL, (rel_l2(out, ref), max(per_tok))


def test_deepseek16b_q4_b8_full():
    _torch()
    W = synth.WORKLOADS["deepseek16b_q4_b8"]
    hl = random_layer(W.seed, W.d_model, W.ffn_dim, W.num_experts, W.bits,
                      shared_ffn=W.shared_ffn_dim)
    r = synth.rng(W.seed + 3000)
    x = _x(r, W.n_tokens, W.d_model, "bf16")
    lg = synth.normal_f32(r, (W.n_tokens, W.num_experts))
    _check_layer(hl, x, lg, W.top_k, W.norm_topk_prob, "bf16")


def test_qwen_stack_three_layers_full_width():
    torch = _torch()
    import quantised_moe_expert_amd as smoe
    W = synth.WORKLOADS["qwen235b_q4_stack94"]
    nl = 3
    hls = [random_layer(W.seed * 100 + l, W.d_model, W.ffn_dim, W.num_experts, W.bits)
           for l in range(nl)]
    r = synth.rng(W.seed + 4000)
    x = synth.normal_f32(r, (1, W.d_model))
    lg = synth.normal_f32(r, (nl, 1, W.num_experts))
    dls = [DeviceLayer(h) for h in hls]
    h_d = torch.from_numpy(x.copy()).cuda()
    lg_d = torch.from_numpy(lg).cuda()
    nws = smoe.smoe_workspace_bytes(dls[0].handle, 1, W.top_k)
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")
    smoe.smoe_decode_step([d.handle for d in dls], h_d.data_ptr(), lg_d.data_ptr(), 1, W.top_k,
                          True, 1e-6, ws.data_ptr(), nws, 0)
    torch.cuda.synchronize()
    got = h_d.cpu().numpy()
    ref = O.decode_step([h.oracle() for h in hls], x, list(lg), W.top_k, True, 1e-6)
    assert rel_l2(got, ref) <= TOL
    assert rel_l2(got - x, ref - x) <= TOL   # the accumulated MoE delta


def test_qwen_stack_94_layers_full_width():
    # the 94 MoE layers of the Qwen3-235B shape ("SMOE Quantisation", Why
    # Quantise), d 4096, ffn 1536, Q4, RMSNorm eps 1e-6 (".smoe Binary Format",
    # Arch Block), one token, distinct logits per layer. To fit the oracle's
    # time and memory the layers alternate over two banks of 8 experts
    # (top-8: every expert of the layer's bank is selected, in the order and
    # with the weights of that layer's logits); the oracle dequantises each
    # of the 16 experts once. Checked on h and on the accumulated MoE delta h - x, so
    # an error that grows with depth shows.
    torch = _torch()
    import quantised_moe_expert_amd as smoe
    W = synth.WORKLOADS["qwen235b_q4_stack94"]
    nl, nb, E, k = 94, 2, 8, 8
    print(f"stack: {nl} layers over {nb} banks of {E} experts", flush=True)
    hls = [random_layer(W.seed * 1000 + b, W.d_model, W.ffn_dim, E, W.bits) for b in range(nb)]
    r = synth.rng(W.seed + 9400)
    x = synth.normal_f32(r, (1, W.d_model))
    lg = synth.normal_f32(r, (nl, 1, E))
    dls = [DeviceLayer(h) for h in hls]
    h_d = torch.from_numpy(x.copy()).cuda()
    lg_d = torch.from_numpy(lg).cuda()
    nws = smoe.smoe_workspace_bytes(dls[0].handle, 1, k)
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")
    smoe.smoe_decode_step([dls[l % nb].handle for l in range(nl)], h_d.data_ptr(),
                          lg_d.data_ptr(), 1, k, True, 1e-6, ws.data_ptr(), nws, 0)
    torch.cuda.synchronize()
    got = h_d.cpu().numpy().astype(np.float64)
    # oracle: h = x; per layer h += MoE_l(rms_norm(h)), each bank's experts
    # dequantised once
    ols = [h.oracle() for h in hls]
    dense = [{e: ol.expert_weights(e) for e in range(E)} for ol in ols]
    h = x.astype(np.float64)
    for l in range(nl):
        n = O.rms_norm(h, 1e-6)[0]
        ids, w = O.route(lg[l, 0], k, True)
        y = np.zeros(W.d_model)
        for j, e in enumerate(ids):
            D = dense[l % nb][e]
            y += w[j] * O.swiglu_expert(D["gate"], D["up"], D["down"], n)
        h = h + y
    err_h, err_d = rel_l2(got, h), rel_l2(got - x, h - x)
    print(f"stack: rel L2 h {err_h:.2e}, delta {err_d:.2e}", flush=True)
    assert err_h <= TOL and err_d <= TOL
