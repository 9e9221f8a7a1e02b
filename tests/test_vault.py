""".smoe vault (".smoe Binary Format"): the Python writer/reader of the
oracle pinned to the pages' record tables, and the library's C++ writer and
reader checked against it byte for byte. Host-only: nothing here touches a
GPU (blobs come from and go to host memory)."""

import ctypes
import struct

import numpy as np
import pytest

import oracle as O
import quantised_moe_expert_amd as smoe
import synth
from conftest import read_golden
from helpers import random_blob

V = O.smoe_vault
SIZES = {"header": 64, "arch": 128, "entry": 48, "desc": 44}
FIELDS = {"header": V.HEADER_FIELDS, "arch": V.ARCH_FIELDS, "entry": V.ENTRY_FIELDS,
          "desc": V.DESC_FIELDS}
CTYPES = {"header": smoe.smoe_vault_header, "arch": smoe.smoe_arch_block,
          "entry": smoe.smoe_expert_entry, "desc": smoe.smoe_tensor_desc}


# ------------------------------------------------------------ oracle pins

def test_record_tables_match_the_pages():
    rows = read_golden("vault_records.txt")
    for rec in SIZES:
        page = [(r[4], int(r[1]), int(r[2])) for r in rows if r[0] == rec]
        mine = [(n, o, struct.calcsize("<" + c)) for n, o, c in FIELDS[rec]]
        assert mine == page, rec
        # the fields tile the record: no gap, no overlap, the stated size
        end = 0
        for _, off, size in page:
            assert off == end
            end += size
        assert end == SIZES[rec]


def test_ctypes_records_match_the_pages():
    rows = read_golden("vault_records.txt")
    for rec, cls in CTYPES.items():
        assert ctypes.sizeof(cls) == SIZES[rec]
        for r in rows:
            if r[0] == rec:
                assert getattr(cls, r[4]).offset == int(r[1]), (rec, r[4])


def test_magic_bytes():
    # File Header: 53 4D 4F 45 DE EA 00 01, "SMOE" then a model marker
    assert V.MAGIC.hex(" ").upper() == "53 4D 4F 45 DE EA 00 01"
    assert V.MAGIC[:4] == b"SMOE" and V.SARC_MAGIC == bytes.fromhex("53415243")


def _blobs(seed, d, ffn, bits, layer_ids, E):
    r = synth.rng(seed)
    L = O.expert_layout(d, ffn, bits, "f16")
    return L, {(l, e): random_blob(r, L) for l in layer_ids for e in range(E)}


def test_python_vault_layout_rules_and_round_trip():
    layers = [1, 3, 4]
    L, blobs = _blobs(400, 128, 64, 4, layers, 4)
    buf = V.write_vault(2, 4, 128, 64, layers, 4, lambda l, e: blobs[(l, e)],
                        vocab_size=151936, ffn_dim=0)
    v = V.read_vault(buf)
    h = v["header"]
    n = 12
    assert h["table_offset"] == 64 and h["total_experts"] == n
    assert h["num_moe_layers"] == 3 and h["max_experts_per_layer"] == 4
    # descriptors right after the table, the arch block 64-aligned after
    # them, the data on a 16 KB page
    assert h["reserved_ext"] % 64 == 0 and h["reserved_ext"] >= 64 + n * 180
    assert h["reserved_ext"] - (64 + n * 180) < 64
    assert h["data_offset"] % 16384 == 0 and h["data_offset"] >= h["reserved_ext"] + 128
    assert buf[h["reserved_ext"]:h["reserved_ext"] + 4] == b"SARC"
    assert len(buf) == h["data_offset"] + n * L.padded_size
    for i, e in enumerate(v["entries"]):
        assert (e["layer_id"], e["expert_id"]) == (layers[i // 4], i % 4)
        assert e["byte_offset"] == h["data_offset"] + i * L.padded_size
        assert e["raw_size"] == L.raw_size and e["padded_size"] == L.padded_size
        # groups over the three tensors: 2 * 64*128/64 + 128*64/64
        assert e["num_groups"] == 3 * 128
        assert [d["tensor_type"] for d in v["descs"][3 * i:3 * i + 3]] == [0, 1, 2]
    for (l, e), b in blobs.items():
        assert np.array_equal(V.expert_blob(v, buf, l, e), b)
    # metadata gap and blob padding are zero
    assert not any(buf[h["reserved_ext"] + 128:h["data_offset"]])
    first = v["entries"][0]["byte_offset"]
    assert not any(buf[first + L.raw_size:first + L.padded_size])


def test_python_reader_follows_descriptors_not_a_fixed_layout():
    # Expert Blob Architecture: readers take the descriptors' offsets
    L, blobs = _blobs(401, 128, 64, 2, [0], 3)
    buf = V.write_vault(1, 2, 128, 64, [0], 3, lambda l, e: blobs[(l, e)],
                        tensor_order=("down", "gate", "up"))
    v = V.read_vault(buf)
    d = v["descs"][0:3]
    assert d[2]["packed_offset"] == 0 and d[0]["packed_offset"] > 0
    for e in range(3):
        assert np.array_equal(V.expert_blob(v, buf, 0, e), blobs[(0, e)])


# ------------------------------------------------------------ corruptions

def _patch(buf, fields, base, name, value):
    b = bytearray(buf)
    for n, off, code in fields:
        if n == name:
            struct.pack_into("<" + code, b, base + off, value)
            return bytes(b)
    raise KeyError(name)


def _valid():
    layers = [0, 2]
    _, blobs = _blobs(402, 128, 64, 4, layers, 3)
    return V.write_vault(2, 4, 128, 64, layers, 3, lambda l, e: blobs[(l, e)])


def _corruptions():
    """(name, function of a valid v2 vault's bytes -> invalid bytes)."""
    H, A, EN, D = V.HEADER_FIELDS, V.ARCH_FIELDS, V.ENTRY_FIELDS, V.DESC_FIELDS

    def hdr(name, val):
        return lambda b: _patch(b, H, 0, name, val)

    def arch(name, val):
        return lambda b: _patch(b, A, V.read_vault(b)["header"]["reserved_ext"], name, val)

    def ent(i, name, val):
        return lambda b: _patch(b, EN, 64 + 48 * i, name, val)

    def desc(j, name, val):
        return lambda b: _patch(b, D, 64 + 48 * 6 + 44 * j, name, val)

    def ent_of(i, name, f):
        return lambda b: _patch(b, EN, 64 + 48 * i, name,
                                f(V.read_vault(b)["entries"][i][name], b))

    def desc_of(j, name, f):
        return lambda b: _patch(b, D, 64 + 48 * 6 + 44 * j, name,
                                f(V.read_vault(b)["descs"][j][name], b))

    def hdr_of(name, f):
        return lambda b: _patch(b, H, 0, name, f(V.read_vault(b)["header"][name], b))

    return [
        ("short file", lambda b: b[:40]),
        ("magic", lambda b: b[:5] + b"\x00" + b[6:]),
        ("version 0", hdr("version", 0)),
        ("version 3", hdr("version", 3)),
        ("table_offset", hdr("table_offset", 128)),
        ("group_size", hdr("group_size", 32)),
        ("bits", hdr("bits", 3)),
        ("empty table", hdr("total_experts", 0)),
        ("data_offset alignment", hdr_of("data_offset", lambda v, b: v + 64)),
        ("data_offset past the end", hdr_of("data_offset", lambda v, b: len(b) + 16384)),
        ("data_offset inside metadata", hdr("data_offset", 0)),
        ("num_moe_layers", hdr("num_moe_layers", 3)),
        ("max_experts_per_layer", hdr("max_experts_per_layer", 4)),
        ("arch offset zero", hdr("reserved_ext", 0)),
        ("arch offset alignment", hdr_of("reserved_ext", lambda v, b: v + 4)),
        ("arch into data", hdr_of("reserved_ext",
                                  lambda v, b: V.read_vault(b)["header"]["data_offset"] - 64)),
        ("SARC magic", arch("magic", b"SARX")),
        ("block_version", arch("block_version", 2)),
        ("block_size", arch("block_size", 64)),
        ("activation", arch("activation", 1)),
        ("top_k 0", arch("moe_top_k", 0)),
        ("top_k 17", arch("moe_top_k", 17)),
        ("head_dim", arch("head_dim", 257)),
        ("kv heads 0", arch("num_kv_heads", 0)),
        ("head divisibility", arch("num_kv_heads", 3)),
        ("arch reserved", arch("reserved", b"\x01")),
        ("table order", ent(1, "expert_id", 0)),
        ("entry group_size", ent(2, "group_size", 32)),
        ("entry reserved", ent(2, "reserved", b"\x00\x01")),
        ("blob offset alignment", ent_of(3, "byte_offset", lambda v, b: v + 4096)),
        ("blob before data", ent(0, "byte_offset", 0)),
        ("padded_size", ent_of(4, "padded_size", lambda v, b: v + 16384)),
        ("blob past the end", lambda b: b[:-1]),
        ("blobs overlap", ent_of(1, "byte_offset", lambda v, b: v - 16384)),
        ("num_groups", ent_of(5, "num_groups", lambda v, b: v + 1)),
        ("tensor_type", desc(4, "tensor_type", 2)),
        ("ndim", desc(4, "ndim", 3)),
        ("descriptor reserved", desc(4, "reserved_0", b"\x00\x07")),
        ("packed_size", desc_of(0, "packed_size", lambda v, b: v - 1)),
        ("scales_size", desc_of(1, "scales_size", lambda v, b: v + 2)),
        ("shape", lambda b: desc(2, "cols", 128)(desc(2, "rows", 64)(b))),   # down transposed
        ("range past raw", desc_of(5, "scales_offset", lambda v, b: v + 16384)),
        ("ranges overlap", desc_of(4, "packed_offset", lambda v, b: 0)),
    ]


def _v1_with_arch_offset(b):
    layers = [0]
    _, blobs = _blobs(403, 128, 64, 4, layers, 2)
    v1 = V.write_vault(1, 4, 128, 64, layers, 2, lambda l, e: blobs[(l, e)])
    return _patch(v1, V.HEADER_FIELDS, 0, "reserved_ext", 448)


CORRUPTIONS = _corruptions() + [("v1 with an arch offset", _v1_with_arch_offset)]


@pytest.mark.parametrize("name,mutate", CORRUPTIONS, ids=[c[0] for c in CORRUPTIONS])
def test_both_readers_refuse(tmp_path, name, mutate):
    bad = mutate(_valid())
    with pytest.raises(V.VaultFormatError):
        V.read_vault(bad)
    p = tmp_path / "bad.smoe"
    p.write_bytes(bad)
    with pytest.raises(smoe.SmoeError) as e:
        smoe.smoe_vault_open(str(p))
    assert e.value.code == smoe.SMOE_E_FORMAT, (name, str(e.value))


def test_valid_vault_opens_in_both(tmp_path):
    good = _valid()
    V.read_vault(good)
    p = tmp_path / "good.smoe"
    p.write_bytes(good)
    smoe.smoe_vault_close(smoe.smoe_vault_open(str(p)))


# ------------------------------------------------ C++ writer and reader

def _arch_ctypes(a: dict) -> "smoe.smoe_arch_block":
    c = smoe.smoe_arch_block_init()
    for k, v in a.items():
        if k in ("magic", "reserved"):
            continue
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("version,bits", [(1, 4), (2, 2), (2, 4)])
def test_cpp_writer_equals_python_writer(tmp_path, version, bits):
    layers, E, d, ffn = [1, 3, 4], 4, 128, 64
    _, blobs = _blobs(410 + bits + version, d, ffn, bits, layers, E)
    arch = V.default_arch(moe_top_k=4, moe_ffn_dim=ffn, num_hidden_layers=5,
                          model_type=b"qwen3_moe") if version == 2 else None
    ref = V.write_vault(version, bits, d, ffn, layers, E, lambda l, e: blobs[(l, e)], arch=arch,
                        vocab_size=1000, ffn_dim=384)
    spec = smoe.make_vault_spec(version, bits, d, ffn, layers, E,
                                _arch_ctypes(arch) if arch else None, vocab_size=1000,
                                ffn_dim=384)
    h, size = smoe.smoe_vault_plan(spec)
    assert size == len(ref) and bytes(h) == ref[:64]
    path = tmp_path / "w.smoe"
    w = smoe.smoe_vault_create(str(path), spec)
    # any order, one expert written twice
    keys = list(blobs)[::-1] + [list(blobs)[0]]
    for (l, e) in keys:
        b = blobs[(l, e)]
        smoe.smoe_vault_put_expert(w, l, e, b.ctypes.data, b.size, smoe.SMOE_MEM_HOST)
    smoe.smoe_vault_finish(w)
    assert path.read_bytes() == ref


@pytest.mark.parametrize("order", [("gate", "up", "down"), ("up", "down", "gate")])
def test_cpp_reader_on_python_vault(tmp_path, order):
    layers, E, d, ffn, bits = [0, 7], 5, 192, 128, 4
    L, blobs = _blobs(420, d, ffn, bits, layers, E)
    buf = V.write_vault(2, bits, d, ffn, layers, E, lambda l, e: blobs[(l, e)],
                        arch=V.default_arch(flags=5, rope_theta=5e5, model_type=b"x"),
                        tensor_order=order)
    ref = V.read_vault(buf)
    p = tmp_path / "r.smoe"
    p.write_bytes(buf)
    v = smoe.smoe_vault_open(str(p))
    try:
        h, a = smoe.smoe_vault_get_header(v)
        assert bytes(h) == buf[:64]
        ra = ref["header"]["reserved_ext"]
        assert bytes(a) == buf[ra:ra + 128]
        for i, ent in enumerate(ref["entries"]):
            e, ds = smoe.smoe_vault_find(v, ent["layer_id"], ent["expert_id"])
            assert bytes(e) == buf[64 + 48 * i:64 + 48 * (i + 1)]
            base = 64 + 48 * len(ref["entries"]) + 132 * i
            assert b"".join(bytes(x) for x in ds) == buf[base:base + 132]
        out = np.full(L.padded_size + 7, 0xEE, np.uint8)
        for (l, e), b in blobs.items():
            smoe.smoe_vault_read_expert(v, l, e, out.ctypes.data, out.size, smoe.SMOE_MEM_HOST)
            assert np.array_equal(out[:L.padded_size], b)
            assert np.all(out[L.padded_size:] == 0xEE)
        desc = smoe.smoe_vault_layer_desc(v, 7)
        assert (desc.d_model, desc.ffn_dim, desc.num_experts, desc.bits, desc.group_size,
                desc.scale_dtype, desc.blob_stride, desc.shared_ffn_dim) == \
            (d, ffn, E, bits, 64, smoe.SMOE_SCALE_F16, L.padded_size, 0)
        bank = np.zeros(E * L.padded_size, np.uint8)
        smoe.smoe_vault_read_layer(v, 7, bank.ctypes.data, bank.size, smoe.SMOE_MEM_HOST)
        assert np.array_equal(bank, np.concatenate([blobs[(7, e)] for e in range(E)]))
        # errors
        for call, code in [
            (lambda: smoe.smoe_vault_find(v, 0, E), smoe.SMOE_E_NOT_FOUND),
            (lambda: smoe.smoe_vault_find(v, 1, 0), smoe.SMOE_E_NOT_FOUND),
            (lambda: smoe.smoe_vault_layer_desc(v, 3), smoe.SMOE_E_NOT_FOUND),
            (lambda: smoe.smoe_vault_read_layer(v, 7, bank.ctypes.data, bank.size - 1,
                                                smoe.SMOE_MEM_HOST), smoe.SMOE_E_ARG),
            (lambda: smoe.smoe_vault_read_expert(v, 0, 0, out.ctypes.data, L.padded_size - 1,
                                                 smoe.SMOE_MEM_HOST), smoe.SMOE_E_ARG),
            (lambda: smoe.smoe_vault_read_expert(v, 0, 0, out.ctypes.data, out.size, 5),
             smoe.SMOE_E_ARG),
        ]:
            with pytest.raises(smoe.SmoeError) as ex:
                call()
            assert ex.value.code == code
    finally:
        smoe.smoe_vault_close(v)


def test_layer_not_numbered_from_zero_is_valid_but_not_a_bank(tmp_path):
    _, blobs = _blobs(430, 128, 64, 4, [0], 2)
    buf = V.write_vault(1, 4, 128, 64, [0], 2, lambda l, e: blobs[(l, e)])
    buf = _patch(buf, V.ENTRY_FIELDS, 64 + 48, "expert_id", 5)   # experts 0, 5
    V.read_vault(buf)
    p = tmp_path / "gap.smoe"
    p.write_bytes(buf)
    v = smoe.smoe_vault_open(str(p))
    try:
        smoe.smoe_vault_find(v, 0, 5)
        with pytest.raises(smoe.SmoeError) as e:
            smoe.smoe_vault_layer_desc(v, 0)
        assert e.value.code == smoe.SMOE_E_UNSUPPORTED
    finally:
        smoe.smoe_vault_close(v)


def test_open_errors(tmp_path):
    with pytest.raises(smoe.SmoeError) as e:
        smoe.smoe_vault_open(str(tmp_path / "missing.smoe"))
    assert e.value.code == smoe.SMOE_E_IO


def test_writer_argument_checks(tmp_path):
    arch = smoe.smoe_arch_block_init()
    arch.moe_top_k, arch.num_heads, arch.num_kv_heads = 8, 8, 2
    bad_arch = smoe.smoe_arch_block_init()
    bad_arch.moe_top_k, bad_arch.num_heads, bad_arch.num_kv_heads = 8, 8, 2
    bad_arch.activation = 1
    cases = [
        dict(version=3), dict(bits=3), dict(d_model=100), dict(layer_ids=[2, 1]),
        dict(layer_ids=[]), dict(experts_per_layer=0), dict(arch=None),
        dict(version=1, arch=arch), dict(arch=bad_arch),
    ]
    for c in cases:
        kw = dict(version=2, bits=4, d_model=128, moe_ffn_dim=64, layer_ids=[0],
                  experts_per_layer=2, arch=arch)
        kw.update(c)
        spec = smoe.make_vault_spec(**kw)
        with pytest.raises(smoe.SmoeError) as e:
            smoe.smoe_vault_plan(spec)
        assert e.value.code == smoe.SMOE_E_ARG, c
        with pytest.raises(smoe.SmoeError):
            smoe.smoe_vault_create(str(tmp_path / "x.smoe"), spec)
    spec = smoe.make_vault_spec(2, 4, 128, 64, [0, 1], 2, arch)
    w = smoe.smoe_vault_create(str(tmp_path / "y.smoe"), spec)
    blob = np.zeros(O.expert_layout(128, 64, 4, "f16").raw_size, np.uint8)
    for args, code in [((2, 0, blob.size), smoe.SMOE_E_NOT_FOUND),
                       ((0, 2, blob.size), smoe.SMOE_E_NOT_FOUND),
                       ((0, 0, blob.size - 1), smoe.SMOE_E_ARG)]:
        with pytest.raises(smoe.SmoeError) as e:
            smoe.smoe_vault_put_expert(w, args[0], args[1], blob.ctypes.data, args[2],
                                       smoe.SMOE_MEM_HOST)
        assert e.value.code == code
    smoe.smoe_vault_put_expert(w, 0, 0, blob.ctypes.data, blob.size, smoe.SMOE_MEM_HOST)
    with pytest.raises(smoe.SmoeError) as e:
        smoe.smoe_vault_finish(w)   # three experts missing
    assert e.value.code == smoe.SMOE_E_ARG


def test_huge_descriptor_shape_is_refused_without_overflow(tmp_path):
    # rows * cols near 2^64 would wrap a 64-bit size computation
    bad = _patch(_valid(), V.DESC_FIELDS, 64 + 48 * 6, "rows", 0xFFFFFFFF)
    bad = _patch(bad, V.DESC_FIELDS, 64 + 48 * 6, "cols", 0xFFFFFFFF)
    with pytest.raises(V.VaultFormatError):
        V.read_vault(bad)
    p = tmp_path / "huge.smoe"
    p.write_bytes(bad)
    with pytest.raises(smoe.SmoeError) as e:
        smoe.smoe_vault_open(str(p))
    assert e.value.code == smoe.SMOE_E_FORMAT
