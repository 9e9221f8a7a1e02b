"""CPU-side checks of the C ABI library: it loads, exports every symbol the
header declares, and its host-only logic (layouts, validation, workspace
sizing) behaves as documented. Nothing here launches GPU work: the device
pointers passed are never dereferenced because every call is rejected, or is a
no-op, before any HIP call.
"""

import os
import re

import numpy as np
import pytest

import oracle as O
import quantised_moe_expert_amd as smoe
from conftest import ROOT

HEADERS = [os.path.join(ROOT, "include", h) for h in ("smoe.h", "smoe_vault.h", "smoe_offload.h")]
FAKE = 1 << 40  # a 16 KB-aligned address that is never dereferenced


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smoe_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = smoe.load_library()
    names = declared_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(smoe.EXPORTED) == names
    assert smoe.smoe_version() == 1


def test_missing_library_is_a_hard_error(tmp_path):
    with pytest.raises(FileNotFoundError):
        smoe.load_library(str(tmp_path / "nope.so"))


@pytest.mark.parametrize("d,ffn,bits,sd", [(4096, 1536, 4, 0), (4096, 1536, 2, 0),
                                            (2048, 1408, 4, 1), (256, 128, 4, 0),
                                            (2048, 2816, 2, 1)])
def test_expert_layout_matches_oracle(d, ffn, bits, sd):
    L = smoe.smoe_expert_layout_of(d, ffn, bits, sd)
    R = O.expert_layout(d, ffn, bits, "f32" if sd == 0 else "f16")
    for name in ("gate", "up", "down"):
        a, b = getattr(L, name), getattr(R, name)
        assert (a.codes_offset, a.codes_bytes, a.scales_offset, a.scales_bytes, a.rows, a.cols) \
            == (b.codes_offset, b.codes_bytes, b.scales_offset, b.scales_bytes, b.rows, b.cols)
    assert L.raw_size == R.raw_size and L.padded_size == R.padded_size


@pytest.mark.parametrize("args", [(100, 128, 4, 0), (256, 0, 4, 0), (256, 128, 3, 0),
                                   (256, 128, 4, 7)])
def test_expert_layout_rejects_bad_shapes(args):
    with pytest.raises(smoe.SmoeError) as e:
        smoe.smoe_expert_layout_of(*args)
    assert e.value.code == smoe.SMOE_E_ARG


def _desc(**kw):
    base = dict(d_model=4096, ffn_dim=1536, num_experts=128, bits=4,
                blob_stride=O.expert_layout(4096, 1536, 4).padded_size)
    base.update(kw)
    return smoe.make_desc(**base)


def test_load_blobs_accepts_a_valid_bank_and_frees():
    desc = _desc()
    h = smoe.smoe_load_blobs(desc, FAKE, 128 * desc.blob_stride)
    assert h
    assert smoe.smoe_workspace_bytes(h, 1, 8) > 0
    assert smoe.smoe_workspace_bytes(h, 32, 8) > smoe.smoe_workspace_bytes(h, 1, 8)
    assert smoe.smoe_workspace_bytes(h, 1, 0) == 0
    assert smoe.smoe_workspace_bytes(h, smoe.SMOE_MAX_TOKENS + 1, 8) == 0
    assert smoe.smoe_workspace_bytes(h, smoe.SMOE_MAX_TOKENS, 8) > 0
    smoe.smoe_free(h)
    smoe.smoe_free(None)


def test_grouping_that_does_not_fit_lds_is_unsupported():
    # 512 experts x 4096 tokens: 256 KB of token bitmasks (the limit is 160 KB)
    desc = _desc(num_experts=512)
    h = smoe.smoe_load_blobs(desc, FAKE, 512 * desc.blob_stride)
    try:
        assert smoe.smoe_workspace_bytes(h, 4096, 8) == 0
        assert smoe.smoe_workspace_bytes(h, 2048, 8) > 0
        # the edge: 2144 tokens take 67 + 9 + 3 words per expert (161,796 B),
        # 2145 tokens 69 + 9 + 3 (the bitmask rows padded to odd lengths)
        assert smoe.smoe_workspace_bytes(h, 2144, 8) > 0
        assert smoe.smoe_workspace_bytes(h, 2145, 8) == 0
        with pytest.raises(smoe.SmoeError) as e:
            smoe.smoe_moe_forward(h, FAKE, smoe.SMOE_DTYPE_BF16, FAKE, 4096, 8, True, FAKE, 0, 0,
                                  FAKE, 1 << 40, 0)
        assert e.value.code == smoe.SMOE_E_UNSUPPORTED
    finally:
        smoe.smoe_free(h)


@pytest.mark.parametrize("kw,nbytes_delta,ptr,code", [
    (dict(bits=3), 0, FAKE, smoe.SMOE_E_ARG),
    (dict(group_size=32), 0, FAKE, smoe.SMOE_E_ARG),
    (dict(num_experts=0), 0, FAKE, smoe.SMOE_E_ARG),
    (dict(num_experts=513), 0, FAKE, smoe.SMOE_E_ARG),
    (dict(d_model=4000), 0, FAKE, smoe.SMOE_E_ARG),
    (dict(blob_stride=10_616_832 - 16384), 0, FAKE, smoe.SMOE_E_LAYOUT),
    (dict(blob_stride=10_616_832 + 64), 0, FAKE, smoe.SMOE_E_LAYOUT),
    (dict(), -1, FAKE, smoe.SMOE_E_LAYOUT),
    (dict(), 0, FAKE + 16, smoe.SMOE_E_LAYOUT),
    # banks start on the 16 KB page boundary (".smoe Binary Format", Immutable
    # Encoding): a 256-byte-aligned base is refused
    (dict(), 0, FAKE + 256, smoe.SMOE_E_LAYOUT),
    (dict(), 0, FAKE + 8192, smoe.SMOE_E_LAYOUT),
    (dict(), 0, 0, smoe.SMOE_E_ARG),
    # one fp32 token (hi + lo pairs, offsets, k-split partial sums) of width
    # 12800 exceeds the batched stages' 64 KB staging
    (dict(d_model=64 * 200), 0, FAKE, smoe.SMOE_E_UNSUPPORTED),
])
def test_load_blobs_validation(kw, nbytes_delta, ptr, code):
    desc = _desc(**kw)
    raw = O.expert_layout(4096, 1536, 4).raw_size
    nbytes = max(desc.num_experts - 1, 0) * desc.blob_stride + raw + nbytes_delta
    with pytest.raises(smoe.SmoeError) as e:
        smoe.smoe_load_blobs(desc, ptr, nbytes)
    assert e.value.code == code
    assert smoe.smoe_last_error()


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("d,ffn,ok", [(11392, 1536, True), (11456, 1536, False),
                                      (4096, 19072, True), (4096, 19136, False)])
def test_activation_width_limits_at_load(bits, d, ffn, ok):
    # the batched stages stage one fp32 token as hi + lo fp16 pairs plus
    # offsets and partial sums (1.25 d + 2072 words), one h row as pairs
    # (0.75 ffn + 2072 words), in 16384 words of LDS
    st = O.expert_layout(d, ffn, bits).padded_size
    desc = smoe.make_desc(d, ffn, 2, bits, st)
    if ok:
        smoe.smoe_free(smoe.smoe_load_blobs(desc, FAKE, 2 * st))
        return
    with pytest.raises(smoe.SmoeError) as e:
        smoe.smoe_load_blobs(desc, FAKE, 2 * st)
    assert e.value.code == smoe.SMOE_E_UNSUPPORTED


def test_shared_blob_alignment_and_width():
    SL = O.expert_layout(2048, 2816, 4)
    st = O.expert_layout(2048, 1408, 4).padded_size
    desc = smoe.make_desc(2048, 1408, 64, 4, st, shared_ffn_dim=2816)
    for off in (256, 8192):
        with pytest.raises(smoe.SmoeError) as e:
            smoe.smoe_load_blobs(desc, FAKE, 64 * st, FAKE + off, SL.raw_size)
        assert e.value.code == smoe.SMOE_E_LAYOUT
    wide = smoe.make_desc(2048, 1408, 64, 4, st, shared_ffn_dim=19136)
    with pytest.raises(smoe.SmoeError) as e:
        smoe.smoe_load_blobs(wide, FAKE, 64 * st, FAKE,
                             O.expert_layout(2048, 19136, 4).raw_size)
    assert e.value.code == smoe.SMOE_E_UNSUPPORTED


def test_load_blobs_exact_minimum_size_is_enough():
    desc = _desc()
    raw = O.expert_layout(4096, 1536, 4).raw_size
    h = smoe.smoe_load_blobs(desc, FAKE, 127 * desc.blob_stride + raw)
    smoe.smoe_free(h)


def test_shared_blob_validation():
    SL = O.expert_layout(2048, 2816, 4)
    desc = smoe.make_desc(2048, 1408, 64, 4, O.expert_layout(2048, 1408, 4).padded_size,
                          shared_ffn_dim=2816)
    with pytest.raises(smoe.SmoeError) as e:
        smoe.smoe_load_blobs(desc, FAKE, 64 * desc.blob_stride)
    assert e.value.code == smoe.SMOE_E_ARG
    with pytest.raises(smoe.SmoeError) as e:
        smoe.smoe_load_blobs(desc, FAKE, 64 * desc.blob_stride, FAKE, SL.raw_size - 1)
    assert e.value.code == smoe.SMOE_E_LAYOUT
    h = smoe.smoe_load_blobs(desc, FAKE, 64 * desc.blob_stride, FAKE, SL.raw_size)
    smoe.smoe_free(h)
    nodesc = smoe.make_desc(2048, 1408, 64, 4, desc.blob_stride)
    with pytest.raises(smoe.SmoeError) as e:
        smoe.smoe_load_blobs(nodesc, FAKE, 64 * desc.blob_stride, FAKE, SL.raw_size)
    assert e.value.code == smoe.SMOE_E_ARG


def test_forward_argument_checks_before_any_launch():
    desc = _desc()
    h = smoe.smoe_load_blobs(desc, FAKE, 128 * desc.blob_stride)
    try:
        ws = smoe.smoe_workspace_bytes(h, 1, 8)
        ok = dict(layer=h, d_x=FAKE, x_dtype=smoe.SMOE_DTYPE_BF16, d_logits=FAKE, n_tokens=1,
                  top_k=8, norm_topk_prob=True, d_out=FAKE, d_topk_ids=0, d_topk_w=0,
                  d_workspace=FAKE, ws_bytes=ws)
        cases = [
            (dict(top_k=0), smoe.SMOE_E_ARG), (dict(top_k=17), smoe.SMOE_E_ARG),
            (dict(n_tokens=-1), smoe.SMOE_E_ARG),
            (dict(n_tokens=smoe.SMOE_MAX_TOKENS + 1), smoe.SMOE_E_ARG),
            (dict(x_dtype=5), smoe.SMOE_E_ARG), (dict(d_x=0), smoe.SMOE_E_ARG),
            (dict(d_out=0), smoe.SMOE_E_ARG), (dict(d_x=FAKE + 2), smoe.SMOE_E_ARG),
            (dict(ws_bytes=ws - 1), smoe.SMOE_E_WORKSPACE),
            (dict(d_workspace=0), smoe.SMOE_E_WORKSPACE),
            (dict(d_workspace=FAKE + 64), smoe.SMOE_E_WORKSPACE),
        ]
        for over, code in cases:
            args = dict(ok, **over)
            with pytest.raises(smoe.SmoeError) as e:
                smoe.smoe_moe_forward(**args)
            assert e.value.code == code, over
        # zero tokens is a valid no-op (nothing is launched)
        smoe.smoe_moe_forward(**dict(ok, n_tokens=0, d_x=0, d_out=0, d_logits=0))
    finally:
        smoe.smoe_free(h)


def test_noalloc_argument_checks_before_any_launch():
    # every case is refused (or is a no-op) before the library looks up its
    # scratch or touches a device
    desc = _desc()
    h = smoe.smoe_load_blobs(desc, FAKE, 128 * desc.blob_stride)
    try:
        ok = dict(layer=h, d_x=FAKE, x_dtype=smoe.SMOE_DTYPE_BF16, d_logits=FAKE, n_tokens=1,
                  top_k=8, norm_topk_prob=True, d_out=FAKE, d_topk_ids=0, d_topk_w=0)
        assert smoe.smoe_workspace_bytes(h, 186, 8) <= smoe.SMOE_NOALLOC_SCRATCH_BYTES
        assert smoe.smoe_workspace_bytes(h, 187, 8) > smoe.SMOE_NOALLOC_SCRATCH_BYTES
        cases = [
            (dict(n_tokens=187), smoe.SMOE_E_WORKSPACE),
            (dict(n_tokens=smoe.SMOE_MAX_TOKENS), smoe.SMOE_E_WORKSPACE),
            (dict(n_tokens=smoe.SMOE_MAX_TOKENS + 1), smoe.SMOE_E_ARG),
            (dict(n_tokens=-1), smoe.SMOE_E_ARG),
            (dict(top_k=0), smoe.SMOE_E_ARG), (dict(top_k=17), smoe.SMOE_E_ARG),
            (dict(x_dtype=5), smoe.SMOE_E_ARG), (dict(d_x=0), smoe.SMOE_E_ARG),
            (dict(d_out=0), smoe.SMOE_E_ARG), (dict(d_logits=0), smoe.SMOE_E_ARG),
            (dict(d_x=FAKE + 2), smoe.SMOE_E_ARG), (dict(d_out=FAKE + 2), smoe.SMOE_E_ARG),
            (dict(layer=0), smoe.SMOE_E_ARG),
        ]
        for over, code in cases:
            with pytest.raises(smoe.SmoeError) as e:
                smoe.smoe_moe_forward_noalloc(**dict(ok, **over))
            assert e.value.code == code, over
        smoe.smoe_moe_forward_noalloc(**dict(ok, n_tokens=0, d_x=0, d_out=0))  # no-op
    finally:
        smoe.smoe_free(h)


def test_route_and_decode_argument_checks():
    with pytest.raises(smoe.SmoeError):
        smoe.smoe_route(FAKE, 1, 128, 17, True, FAKE, FAKE)
    with pytest.raises(smoe.SmoeError):
        smoe.smoe_route(FAKE, 1, 4, 5, True, FAKE, FAKE)
    with pytest.raises(smoe.SmoeError):
        smoe.smoe_route(FAKE, 1, 600, 8, True, FAKE, FAKE)
    smoe.smoe_route(0, 0, 128, 8, True, 0, 0)  # zero tokens: no-op
    desc = _desc()
    h = smoe.smoe_load_blobs(desc, FAKE, 128 * desc.blob_stride)
    h2 = smoe.smoe_load_blobs(_desc(d_model=2048, blob_stride=O.expert_layout(
        2048, 1536, 4).padded_size), FAKE, 128 * O.expert_layout(2048, 1536, 4).padded_size)
    try:
        ws = smoe.smoe_workspace_bytes(h, 1, 8)
        with pytest.raises(smoe.SmoeError):
            smoe.smoe_decode_step([], FAKE, FAKE, 1, 8, True, 1e-6, FAKE, ws)
        with pytest.raises(smoe.SmoeError):
            smoe.smoe_decode_step([h], FAKE, FAKE, 1, 8, True, 0.0, FAKE, ws)
        with pytest.raises(smoe.SmoeError):
            smoe.smoe_decode_step([h, h2], FAKE, FAKE, 1, 8, True, 1e-6, FAKE, ws)
        smoe.smoe_decode_step([h, h], 0, 0, 0, 8, True, 1e-6, FAKE, ws)
    finally:
        smoe.smoe_free(h)
        smoe.smoe_free(h2)


def test_trace_kernel_argument_checks():
    # arming validates the kernel id and the events; nothing is recorded
    # until a forward launches the armed kernel, so fake handles are safe here
    with pytest.raises(smoe.SmoeError) as e:
        smoe.smoe_trace_kernel(7, FAKE, FAKE)
    assert e.value.code == smoe.SMOE_E_ARG
    with pytest.raises(smoe.SmoeError):
        smoe.smoe_trace_kernel(smoe.SMOE_KERNEL_GATE_UP, 0, FAKE)
    smoe.smoe_trace_kernel(smoe.SMOE_KERNEL_DOWN, FAKE, FAKE)
    assert smoe.smoe_trace_kernel(smoe.SMOE_KERNEL_NONE) == 1  # was armed, never fired
    assert smoe.smoe_trace_kernel(smoe.SMOE_KERNEL_NONE) == 0


def test_route_options_are_validated_before_launch():
    # "CMF v2 Format Specification", 5. Masks section: bits past the
    # dimension must be zero; routing needs top_k routable experts
    def call(**kw):
        o = smoe.make_route_opts(**{k: v for k, v in kw.items() if k != "raw"})
        for k, v in kw.get("raw", {}).items():
            setattr(o, k, v)
        with pytest.raises(smoe.SmoeError) as e:
            smoe.smoe_route_ex(FAKE, 1, 8, 4, True, o, FAKE, FAKE)
        return e.value.code
    assert call(routable=[True] * 3 + [False] * 5) == smoe.SMOE_E_ARG      # 3 < top_k
    o = smoe.make_route_opts(routable=[True] * 8)
    o.expert_mask[0] |= 1 << 9                                              # past E
    with pytest.raises(smoe.SmoeError) as e:
        smoe.smoe_route_ex(FAKE, 1, 8, 4, True, o, FAKE, FAKE)
    assert e.value.code == smoe.SMOE_E_ARG
    assert call(scaling_factor=float("inf")) == smoe.SMOE_E_ARG
    assert call(raw={"sigmoid": 2}) == smoe.SMOE_E_ARG
    # defaults and zero tokens pass validation and launch nothing
    smoe.smoe_route_ex(FAKE, 0, 8, 4, True, smoe.make_route_opts(), FAKE, FAKE)
    smoe.smoe_route_ex(FAKE, 0, 8, 4, True, None, FAKE, FAKE)


def test_quantise_argument_checks_before_any_launch():
    def code(*a):
        with pytest.raises(smoe.SmoeError) as e:
            smoe.smoe_quantise(*a)
        return e.value.code
    assert code(FAKE, 64, 3, 0, FAKE, FAKE) == smoe.SMOE_E_ARG            # bits
    assert code(FAKE, 64, 4, 2, FAKE, FAKE) == smoe.SMOE_E_ARG            # scale dtype
    assert code(FAKE, smoe.SMOE_MAX_QUANT_ELEMENTS + 1, 4, 0, FAKE, FAKE) == smoe.SMOE_E_ARG
    assert code(0, 64, 4, 0, FAKE, FAKE) == smoe.SMOE_E_ARG               # null weights
    assert code(FAKE, 64, 2, 1, FAKE, 0) == smoe.SMOE_E_ARG               # null scales
    assert code(FAKE + 2, 64, 4, 0, FAKE, FAKE) == smoe.SMOE_E_ARG        # misaligned weights
    assert code(FAKE, 64, 4, 0, FAKE, FAKE + 2) == smoe.SMOE_E_ARG        # misaligned f32 scales
    smoe.smoe_quantise(0, 0, 4, 0, 0, 0)                                   # empty: no-op
