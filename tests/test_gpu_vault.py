""".smoe vault to and from the GPU (".smoe Binary Format"): a vault written
by the oracle is read by the library straight into a device bank and runs
the forward (checked against the oracle's forward on the same blobs); experts
quantised on the GPU and written by the library give the oracle's vault byte
for byte."""

import numpy as np
import pytest

import oracle as O
import synth
from helpers import DeviceLayer, HostLayer, random_blob, rel_l2

pytestmark = pytest.mark.gpu
V = O.smoe_vault
TOL = 1e-3


def _torch():
    import torch
    # a GPU test fails where no device is visible (it must not pass by skipping)
    assert torch.cuda.is_available(), "no GPU visible to torch"
    return torch


@pytest.mark.parametrize("bits,order", [(4, ("gate", "up", "down")), (2, ("down", "up", "gate"))])
def test_vault_layer_read_to_device_runs_the_forward(tmp_path, bits, order):
    torch = _torch()
    import quantised_moe_expert_amd as smoe
    d, ffn, E, layers = 256, 128, 8, [1, 2]
    r = synth.rng(500 + bits)
    L = O.expert_layout(d, ffn, bits, "f16")
    blobs = {(l, e): random_blob(r, L) for l in layers for e in range(E)}
    buf = V.write_vault(2, bits, d, ffn, layers, E, lambda l, e: blobs[(l, e)],
                        tensor_order=order)
    path = tmp_path / "layer.smoe"
    path.write_bytes(buf)
    print(f"vault read_layer bits={bits} order={order}", flush=True)
    v = smoe.smoe_vault_open(str(path))
    try:
        desc = smoe.smoe_vault_layer_desc(v, 2)
        assert desc.blob_stride == L.padded_size and desc.num_experts == E
        bank = smoe.aligned_buffer(E * L.padded_size)
        bank.fill_(0xEE)
        s = torch.cuda.current_stream().cuda_stream
        smoe.smoe_vault_read_layer(v, 2, bank.data_ptr(), bank.numel(), smoe.SMOE_MEM_DEVICE, s)
        host = np.concatenate([blobs[(2, e)] for e in range(E)])
        assert np.array_equal(bank.cpu().numpy(), host)
        one = torch.zeros(L.padded_size, dtype=torch.uint8, device="cuda:0")
        smoe.smoe_vault_read_expert(v, 1, 5, one.data_ptr(), one.numel(), smoe.SMOE_MEM_DEVICE, s)
        assert np.array_equal(one.cpu().numpy(), blobs[(1, 5)])
    finally:
        smoe.smoe_vault_close(v)
    hl = HostLayer(d, ffn, E, bits, "f16", 0, host, L.padded_size, None)
    dl = DeviceLayer(hl, bank_tensor=bank)
    try:
        x = synth.round_to_bf16(synth.normal_f32(r, (5, d)))
        logits = synth.normal_f32(r, (5, E))
        out, ids, w = dl.forward(x, logits, 2, True, "bf16")
        ref, rids, rw = O.moe_forward(hl.oracle(), x, logits, 2, True)
        assert np.array_equal(ids, rids)
        assert rel_l2(out, ref) <= TOL
    finally:
        dl.close()


def test_gpu_quantised_experts_written_by_the_library_equal_the_oracle_vault(tmp_path):
    torch = _torch()
    import quantised_moe_expert_amd as smoe
    d, ffn, E, layers, bits = 256, 128, 2, [3, 5], 4
    r = synth.rng(510)
    L = O.expert_layout(d, ffn, bits, "f16")
    weights = {(l, e): {n: synth.outlier_weights_f32(r, (sp.rows, sp.cols))
                        for n, sp in L.spans().items()}
               for l in layers for e in range(E)}
    arch = smoe.smoe_arch_block_init()
    arch.moe_top_k, arch.num_heads, arch.num_kv_heads, arch.head_dim = 2, 8, 2, 64
    arch.moe_ffn_dim = ffn
    spec = smoe.make_vault_spec(2, bits, d, ffn, layers, E, arch)
    path = tmp_path / "gpu.smoe"
    w = smoe.smoe_vault_create(str(path), spec)
    s = torch.cuda.current_stream().cuda_stream
    print("vault put_expert from GPU-quantised blobs", flush=True)
    for (l, e), ws in weights.items():
        blob = torch.zeros(L.padded_size, dtype=torch.uint8, device="cuda:0")
        keep = []
        for n, sp in L.spans().items():
            wd = torch.from_numpy(ws[n].reshape(-1)).to("cuda:0")
            keep.append(wd)
            smoe.smoe_quantise(wd.data_ptr(), wd.numel(), bits, smoe.SMOE_SCALE_F16,
                               blob.data_ptr() + sp.codes_offset,
                               blob.data_ptr() + sp.scales_offset, s)
        smoe.smoe_vault_put_expert(w, l, e, blob.data_ptr(), blob.numel(), smoe.SMOE_MEM_DEVICE, s)
    smoe.smoe_vault_finish(w)

    def oracle_blob(l, e):
        return O.build_expert_blob(L, {n: O.quantise_tensor(W, bits, "f16")
                                       for n, W in weights[(l, e)].items()})

    a = V.default_arch(flags=0, rope_theta=0.0, num_heads=8, num_kv_heads=2, head_dim=64,
                       moe_top_k=2, moe_ffn_dim=ffn, rms_norm_eps=float(np.float32(1e-6)),
                       model_type=b"")
    ref = V.write_vault(2, bits, d, ffn, layers, E, oracle_blob, arch=a)
    assert path.read_bytes() == ref
