"""GPU quantiser ("SMOE Quantisation", L2-MSE Scale Optimiser; Bit Packing)
against the oracle's quantise_tensor / mse_grid_scale: packed codes and
stored scales bit-exact, nothing written past the outputs."""

import numpy as np
import pytest

import oracle as O
import synth

pytestmark = pytest.mark.gpu
GUARD = 64  # sentinel bytes after each output


def _torch():
    import torch
    # a GPU test fails where no device is visible (it must not pass by skipping)
    assert torch.cuda.is_available(), "no GPU visible to torch"
    return torch


def _gpu_quantise(w: np.ndarray, bits: int, scale_dtype: str):
    """(packed codes uint8, scales) from smoe_quantise, checking the guard
    bytes after both outputs."""
    torch = _torch()
    import quantised_moe_expert_amd as smoe
    flat = np.ascontiguousarray(w, np.float32).reshape(-1)
    n = flat.size
    nb = O.packed_size(n, bits)
    ns = O.scale_count(n)
    ssz = 4 if scale_dtype == "f32" else 2
    wd = torch.from_numpy(flat).to("cuda:0")
    cd = torch.full((nb + GUARD,), 0xAB, dtype=torch.uint8, device="cuda:0")
    sd = torch.full((ns * ssz + GUARD,), 0xCD, dtype=torch.uint8, device="cuda:0")
    s = torch.cuda.current_stream().cuda_stream
    print(f"smoe_quantise n={n} bits={bits} scales={scale_dtype}", flush=True)
    smoe.smoe_quantise(wd.data_ptr(), n, bits, 0 if scale_dtype == "f32" else 1, cd.data_ptr(),
                       sd.data_ptr(), s)
    torch.cuda.synchronize()
    c = cd.cpu().numpy()
    sc = sd.cpu().numpy()
    assert np.all(c[nb:] == 0xAB), "codes written past the end"
    assert np.all(sc[ns * ssz:] == 0xCD), "scales written past the end"
    st = np.float32 if scale_dtype == "f32" else np.float16
    return c[:nb], sc[:ns * ssz].view(st)


def _same_bits(a: np.ndarray, b: np.ndarray) -> bool:
    u = np.uint32 if a.dtype == np.float32 else np.uint16
    return np.array_equal(a.view(u), b.view(u))


def _special_groups(r) -> np.ndarray:
    """Groups that exercise the search's corners, then a ragged tail."""
    g = []
    g.append(np.zeros(64))                                   # zero group
    w = r.standard_normal(64) * 1e-3
    w[17] = 1.0
    g.append(w)                                              # one loud outlier
    g.append(r.standard_normal(64) * 1e-7)                   # f16 scales go subnormal
    g.append(r.standard_normal(64) * 3e4)                    # f16 candidates overflow
    g.append(np.full(64, 0.75))                              # constant
    g.append(-np.abs(r.standard_normal(64)) * 0.02)          # one sign
    g.append(r.standard_normal(64) * 1e-40)                  # fp32 subnormal weights
    lv = (np.arange(16) - 7.5) / 7.5 * 0.5
    g.append(lv[r.integers(0, 16, 64)])                      # on a Q4 grid
    lv2 = (np.arange(4) - 1.5) / 1.5 * 0.25
    g.append(lv2[r.integers(0, 4, 64)])                      # on a Q2 grid
    w = r.standard_normal(64) * 0.02
    w[::9] = 0.0
    g.append(w)
    g.append(r.standard_normal(17) * 0.02)                   # ragged tail
    return np.concatenate(g).astype(np.float32)


CASES = [(b, st) for b in (4, 2) for st in ("f32", "f16")]


@pytest.mark.parametrize("bits,scale_dtype", CASES)
def test_outlier_weights_bit_exact(bits, scale_dtype):
    """A [96, 448] tensor of N(0, 0.02^2) weights with 1% x10 outliers:
    672 groups, several per row and straddling rows."""
    r = synth.rng(300 + bits)
    W = synth.outlier_weights_f32(r, (96, 448))
    codes, scales = _gpu_quantise(W, bits, scale_dtype)
    rc, rs = O.quantise_tensor(W, bits, scale_dtype)
    assert np.array_equal(codes, rc)
    assert _same_bits(scales, rs)


@pytest.mark.parametrize("bits,scale_dtype", CASES)
def test_special_groups_and_ragged_tail_bit_exact(bits, scale_dtype):
    w = _special_groups(synth.rng(310))
    assert w.size % 64 == 17
    codes, scales = _gpu_quantise(w, bits, scale_dtype)
    rc, rs = O.quantise_tensor(w, bits, scale_dtype)
    assert np.array_equal(codes, rc)
    assert _same_bits(scales, rs)


@pytest.mark.parametrize("n", [1, 3, 63, 65, 130])
def test_short_tensors(n):
    w = synth.normal_f32(synth.rng(320 + n), (n,), std=0.05)
    for bits in (4, 2):
        codes, scales = _gpu_quantise(w, bits, "f16")
        rc, rs = O.quantise_tensor(w, bits, "f16")
        assert np.array_equal(codes, rc)
        assert _same_bits(scales, rs)


def test_empty_tensor_is_a_no_op():
    _torch()
    import quantised_moe_expert_amd as smoe
    smoe.smoe_quantise(0, 0, 4, 0, 0, 0, 0)


def test_quantised_blob_equals_oracle_blob():
    """Gate, up and down quantised on the GPU straight into their places in a
    .smoe expert blob: the blob matches the oracle's byte for byte."""
    torch = _torch()
    import quantised_moe_expert_amd as smoe
    r = synth.rng(330)
    L = O.expert_layout(256, 128, 4, "f32")
    ws = {name: synth.outlier_weights_f32(r, (sp.rows, sp.cols)) for name, sp in L.spans().items()}
    blob_d = smoe.aligned_buffer(L.padded_size)
    blob_d.zero_()
    s = torch.cuda.current_stream().cuda_stream
    keep = []
    for name, sp in L.spans().items():
        wd = torch.from_numpy(ws[name].reshape(-1)).to("cuda:0")
        keep.append(wd)
        smoe.smoe_quantise(wd.data_ptr(), wd.numel(), 4, 0, blob_d.data_ptr() + sp.codes_offset,
                           blob_d.data_ptr() + sp.scales_offset, s)
    torch.cuda.synchronize()
    ref = O.build_expert_blob(L, {n: O.quantise_tensor(ws[n], 4, "f32") for n in ws})
    assert np.array_equal(blob_d.cpu().numpy(), ref)


@pytest.mark.parametrize("bits", [4, 2])
def test_full_size_expert_tensor_sampled(bits):
    """A [1536, 4096] gate tensor (one Qwen3-235B-A22B-shaped expert
    projection, 98,304 groups) quantised in one call; 192 sampled groups
    checked against the oracle's search one by one (groups are independent)."""
    r = synth.rng(340 + bits)
    W = synth.outlier_weights_f32(r, (1536, 4096))
    codes, scales = _gpu_quantise(W, bits, "f32")
    flat = W.reshape(-1)
    bpg = 64 * bits // 8
    for g in np.sort(r.choice(flat.size // 64, 192, replace=False)):
        s, c, _ = O.mse_grid_scale(flat[g * 64:(g + 1) * 64], bits, "f32")
        assert np.float32(s).view(np.uint32) == scales[g].view(np.uint32), g
        assert np.array_equal(codes[g * bpg:(g + 1) * bpg], O.pack_codes(c, bits)), g
