""".smoe vault writer and reader in plain Python (test infrastructure).

TEST INFRASTRUCTURE, like the rest of this package: the GPU library's own
vault code (C++) is checked against this module byte for byte; the two share
no code. Only the test suite may use it.

Source: ".smoe Binary Format" -- Immutable Encoding (little-endian, offsets
from the start of the file, 16,384-byte blob alignment), File Architecture
(header, then the expert table, then the tensor descriptors, then the arch
block in the gap before the 16 KB-aligned data), File Header, Version
acceptance, Arch Block "SARC", Expert Table Entry (sorted by layer, then
expert), Tensor Descriptor (gate, up, down per entry), Expert Blob
Architecture, C++ Struct Mirror (record sizes 64, 48 and 128 bytes).

Every record is written and read field by field at the offsets the pages'
tables give (FIELD tables below), not through a sequential struct format, so
that a wrong offset in either implementation shows up as a byte difference.

Readings where the pages leave a choice (each also listed in the design
notes): the arch block sits at the first multiple of 64 after the
descriptors and the data at the first multiple of 16,384 after the last
metadata byte; blobs follow in table order, padded_size apart; a reader
refuses, besides what the pages name (magic, version, arch block magic /
size / activation / top_k / head_dim / head divisibility), every field that
contradicts the layout (see ``validate``).
"""

from __future__ import annotations

import struct
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

from . import smoe_oracle as O

__all__ = [
    "MAGIC", "SARC_MAGIC", "HEADER_FIELDS", "ARCH_FIELDS", "ENTRY_FIELDS", "DESC_FIELDS",
    "HEADER_SIZE", "ARCH_SIZE", "ENTRY_SIZE", "DESC_SIZE", "VaultFormatError",
    "pack_record", "unpack_record", "default_arch", "vault_layout", "write_vault",
    "read_vault", "expert_blob",
]

MAGIC = bytes([0x53, 0x4D, 0x4F, 0x45, 0xDE, 0xEA, 0x00, 0x01])  # File Header, magic
SARC_MAGIC = b"SARC"                                               # Arch Block, magic

# (name, byte offset, struct code) -- the pages' tables, one row each.
HEADER_SIZE = 64
HEADER_FIELDS = [
    ("magic", 0, "8s"), ("version", 8, "I"), ("num_moe_layers", 12, "I"),
    ("max_experts_per_layer", 16, "I"), ("total_experts", 20, "I"),
    ("table_offset", 24, "Q"), ("data_offset", 32, "Q"), ("group_size", 40, "I"),
    ("bits", 44, "I"), ("d_model", 48, "I"), ("vocab_size", 52, "I"), ("ffn_dim", 56, "I"),
    ("reserved_ext", 60, "I"),
]
ARCH_SIZE = 128
ARCH_FIELDS = [
    ("magic", 0, "4s"), ("block_version", 4, "I"), ("block_size", 8, "I"), ("flags", 12, "I"),
    ("rope_theta", 16, "f"), ("num_heads", 20, "I"), ("num_kv_heads", 24, "I"),
    ("head_dim", 28, "I"), ("moe_top_k", 32, "I"), ("moe_ffn_dim", 36, "I"),
    ("dense_ffn_dim", 40, "I"), ("shared_expert_ffn_dim", 44, "I"), ("activation", 48, "I"),
    ("num_hidden_layers", 52, "I"), ("rms_norm_eps", 56, "f"), ("model_type", 60, "24s"),
    ("reserved", 84, "44s"),
]
ENTRY_SIZE = 48
ENTRY_FIELDS = [
    ("layer_id", 0, "I"), ("expert_id", 4, "I"), ("byte_offset", 8, "Q"), ("raw_size", 16, "Q"),
    ("padded_size", 24, "Q"), ("group_size", 32, "I"), ("num_groups", 36, "Q"),
    ("reserved", 44, "4s"),
]
DESC_SIZE = 44
DESC_FIELDS = [
    ("tensor_type", 0, "B"), ("ndim", 1, "B"), ("reserved_0", 2, "2s"), ("rows", 4, "I"),
    ("cols", 8, "I"), ("packed_offset", 12, "Q"), ("packed_size", 20, "Q"),
    ("scales_offset", 28, "Q"), ("scales_size", 36, "Q"),
]

PAGE = O.BLOB_ALIGN
TABLE_OFFSET = 64


class VaultFormatError(ValueError):
    """The bytes are not a valid .smoe vault."""


def pack_record(fields, size: int, values: Dict) -> bytes:
    """A record of `size` bytes with each field little-endian at its offset;
    missing fields are zero."""
    buf = bytearray(size)
    for name, off, code in fields:
        v = values.get(name, b"" if code.endswith("s") else 0)
        struct.pack_into("<" + code, buf, off, v)
    return bytes(buf)


def unpack_record(fields, buf, off: int = 0) -> Dict:
    return {name: struct.unpack_from("<" + code, buf, off + o)[0] for name, o, code in fields}


def default_arch(**kw) -> Dict:
    """A valid arch block (SiLU, top-k 8, 64 heads / 4 KV heads of 128)."""
    a = {"magic": SARC_MAGIC, "block_version": 1, "block_size": ARCH_SIZE, "flags": 1,
         "rope_theta": 1.0e6, "num_heads": 64, "num_kv_heads": 4, "head_dim": 128,
         "moe_top_k": 8, "moe_ffn_dim": 0, "dense_ffn_dim": 0, "shared_expert_ffn_dim": 0,
         "activation": 0, "num_hidden_layers": 0, "rms_norm_eps": 1e-6,
         "model_type": b"qwen3_moe", "reserved": b""}
    a.update(kw)
    return a


def _ceil(a: int, b: int) -> int:
    return -(-a // b)


def vault_layout(version: int, n_experts: int) -> Dict[str, int]:
    """Where the metadata goes for n_experts table entries."""
    desc_off = TABLE_OFFSET + n_experts * ENTRY_SIZE
    meta_end = desc_off + 3 * n_experts * DESC_SIZE
    arch_off = _ceil(meta_end, 64) * 64 if version == 2 else 0
    end = arch_off + ARCH_SIZE if version == 2 else meta_end
    return {"desc_offset": desc_off, "meta_end": meta_end, "arch_offset": arch_off,
            "data_offset": _ceil(end, PAGE) * PAGE}


def write_vault(version: int, bits: int, d_model: int, ffn: int, layer_ids: Sequence[int],
                experts_per_layer: int, blob_of: Callable[[int, int], np.ndarray],
                arch: Optional[Dict] = None, vocab_size: int = 0, ffn_dim: int = 0,
                tensor_order: Sequence[str] = ("gate", "up", "down")) -> bytes:
    """The bytes of a vault. blob_of(layer, expert) gives the expert's
    canonical blob (oracle layout, fp16 scales). tensor_order places the
    three tensors (codes then scales each) in another order inside the
    blobs, giving descriptors that differ from the canonical offsets."""
    L = O.expert_layout(d_model, ffn, bits, "f16")
    spans = L.spans()
    # blob-relative placement in the requested order
    place = {}
    pos = 0
    for name in tensor_order:
        sp = spans[name]
        place[name] = (pos, pos + sp.codes_bytes)
        pos += sp.codes_bytes + sp.scales_bytes
    raw = pos
    padded = _ceil(raw, PAGE) * PAGE
    keys = [(l, e) for l in layer_ids for e in range(experts_per_layer)]
    n = len(keys)
    lay = vault_layout(version, n)
    out = bytearray(lay["data_offset"] + n * padded)
    hdr = {"magic": MAGIC, "version": version, "num_moe_layers": len(layer_ids),
           "max_experts_per_layer": experts_per_layer, "total_experts": n,
           "table_offset": TABLE_OFFSET, "data_offset": lay["data_offset"],
           "group_size": O.GROUP_SIZE, "bits": bits, "d_model": d_model,
           "vocab_size": vocab_size, "ffn_dim": ffn_dim, "reserved_ext": lay["arch_offset"]}
    out[0:HEADER_SIZE] = pack_record(HEADER_FIELDS, HEADER_SIZE, hdr)
    groups = sum(_ceil(sp.rows * sp.cols, O.GROUP_SIZE) for sp in spans.values())
    for i, (l, e) in enumerate(keys):
        off = lay["data_offset"] + i * padded
        ent = {"layer_id": l, "expert_id": e, "byte_offset": off, "raw_size": raw,
               "padded_size": padded, "group_size": O.GROUP_SIZE, "num_groups": groups}
        p = TABLE_OFFSET + i * ENTRY_SIZE
        out[p:p + ENTRY_SIZE] = pack_record(ENTRY_FIELDS, ENTRY_SIZE, ent)
        blob = np.asarray(blob_of(l, e), dtype=np.uint8)
        for k, name in enumerate(("gate", "up", "down")):
            sp = spans[name]
            co, so = place[name]
            d = {"tensor_type": k, "ndim": 2, "rows": sp.rows, "cols": sp.cols,
                 "packed_offset": co, "packed_size": sp.codes_bytes, "scales_offset": so,
                 "scales_size": sp.scales_bytes}
            q = lay["desc_offset"] + (3 * i + k) * DESC_SIZE
            out[q:q + DESC_SIZE] = pack_record(DESC_FIELDS, DESC_SIZE, d)
            out[off + co:off + co + sp.codes_bytes] = \
                blob[sp.codes_offset:sp.codes_offset + sp.codes_bytes].tobytes()
            out[off + so:off + so + sp.scales_bytes] = \
                blob[sp.scales_offset:sp.scales_offset + sp.scales_bytes].tobytes()
    if version == 2:
        a = arch if arch is not None else default_arch()
        out[lay["arch_offset"]:lay["arch_offset"] + ARCH_SIZE] = \
            pack_record(ARCH_FIELDS, ARCH_SIZE, a)
    return bytes(out)


def _fail(msg: str):
    raise VaultFormatError(msg)


def _check_arch(a: Dict):
    if a["magic"] != SARC_MAGIC:
        _fail("arch magic")
    if a["block_version"] != 1:
        _fail("arch block_version")
    if a["block_size"] != ARCH_SIZE:
        _fail("arch block_size")
    if a["activation"] != 0:
        _fail("activation is not SiLU")
    if not 1 <= a["moe_top_k"] <= O.MAX_TOP_K:
        _fail("moe_top_k")
    if a["head_dim"] > 256:
        _fail("head_dim")
    if a["num_kv_heads"] == 0 or a["num_heads"] % a["num_kv_heads"]:
        _fail("head divisibility")
    if any(a["reserved"]):
        _fail("arch reserved")


def read_vault(buf: bytes) -> Dict:
    """Parse and validate; returns {"header", "arch" (None for v1),
    "entries", "descs" (lists of dicts; three descriptors per entry)}."""
    size = len(buf)
    if size < HEADER_SIZE:
        _fail("short file")
    h = unpack_record(HEADER_FIELDS, buf)
    if h["magic"] != MAGIC:
        _fail("magic")
    if h["version"] not in (1, 2):
        _fail("version")
    if h["table_offset"] != TABLE_OFFSET:
        _fail("table_offset")
    if h["group_size"] != O.GROUP_SIZE:
        _fail("group_size")
    if h["bits"] not in (2, 4):
        _fail("bits")
    n = h["total_experts"]
    if n < 1:
        _fail("empty table")
    if h["data_offset"] % PAGE:
        _fail("data_offset alignment")
    lay = vault_layout(1, n)
    if h["data_offset"] < lay["meta_end"]:
        _fail("data_offset inside the metadata")
    if h["data_offset"] > size:
        _fail("data_offset past the end")
    arch = None
    if h["version"] == 1:
        if h["reserved_ext"] != 0:
            _fail("v1 reserved_ext")
    else:
        a_off = h["reserved_ext"]
        if a_off % 64 or a_off < lay["meta_end"] or a_off + ARCH_SIZE > h["data_offset"]:
            _fail("arch block placement")
        arch = unpack_record(ARCH_FIELDS, buf, a_off)
        _check_arch(arch)
    entries = [unpack_record(ENTRY_FIELDS, buf, TABLE_OFFSET + i * ENTRY_SIZE) for i in range(n)]
    descs = [unpack_record(DESC_FIELDS, buf, lay["desc_offset"] + j * DESC_SIZE)
             for j in range(3 * n)]
    keys = [(e["layer_id"], e["expert_id"]) for e in entries]
    if any(keys[i] >= keys[i + 1] for i in range(n - 1)):
        _fail("table order")
    layer_sizes: Dict[int, int] = {}
    for l, _ in keys:
        layer_sizes[l] = layer_sizes.get(l, 0) + 1
    if h["num_moe_layers"] != len(layer_sizes):
        _fail("num_moe_layers")
    if h["max_experts_per_layer"] != max(layer_sizes.values()):
        _fail("max_experts_per_layer")
    blobs = []
    for i, e in enumerate(entries):
        if e["group_size"] != h["group_size"]:
            _fail("entry group_size")
        if any(e["reserved"]):
            _fail("entry reserved")
        if e["byte_offset"] % PAGE or e["byte_offset"] < h["data_offset"]:
            _fail("blob offset")
        if e["padded_size"] != _ceil(e["raw_size"], PAGE) * PAGE:
            _fail("padded_size")
        if e["byte_offset"] + e["padded_size"] > size:
            _fail("blob past the end")
        blobs.append((e["byte_offset"], e["byte_offset"] + e["padded_size"]))
        ds = descs[3 * i:3 * i + 3]
        ranges = []
        groups = 0
        for k, d in enumerate(ds):
            if d["tensor_type"] != k or d["ndim"] != 2 or any(d["reserved_0"]):
                _fail("descriptor kind")
            cnt = d["rows"] * d["cols"]
            if d["packed_size"] != _ceil(cnt * h["bits"], 8):
                _fail("packed_size")
            if d["scales_size"] != 2 * _ceil(cnt, O.GROUP_SIZE):
                _fail("scales_size")
            groups += _ceil(cnt, O.GROUP_SIZE)
            ranges += [(d["packed_offset"], d["packed_size"]), (d["scales_offset"], d["scales_size"])]
        g, u, dn = ds
        ffn = g["rows"]
        if not (ffn >= 1 and u["rows"] == ffn and dn["cols"] == ffn and
                g["cols"] == h["d_model"] and u["cols"] == h["d_model"] and
                dn["rows"] == h["d_model"]):
            _fail("shapes")
        if e["num_groups"] != groups:
            _fail("num_groups")
        ranges.sort()
        for j, (o, s) in enumerate(ranges):
            if o + s > e["raw_size"]:
                _fail("tensor range past raw_size")
            if j and o < ranges[j - 1][0] + ranges[j - 1][1]:
                _fail("tensor ranges overlap")
    blobs.sort()
    if any(blobs[i][0] < blobs[i - 1][1] for i in range(1, len(blobs))):
        _fail("blobs overlap")
    return {"header": h, "arch": arch, "entries": entries, "descs": descs}


def expert_blob(vault: Dict, buf: bytes, layer: int, expert: int) -> np.ndarray:
    """One expert's blob in canonical layout (oracle expert_layout, fp16
    scales), zero-padded to its padded size, taken through its descriptors."""
    h = vault["header"]
    for i, e in enumerate(vault["entries"]):
        if (e["layer_id"], e["expert_id"]) == (layer, expert):
            break
    else:
        raise KeyError((layer, expert))
    ds = vault["descs"][3 * i:3 * i + 3]
    L = O.expert_layout(h["d_model"], ds[0]["rows"], h["bits"], "f16")
    out = np.zeros(L.padded_size, dtype=np.uint8)
    base = e["byte_offset"]
    for name, d in zip(("gate", "up", "down"), ds):
        sp = L.spans()[name]
        out[sp.codes_offset:sp.codes_offset + sp.codes_bytes] = np.frombuffer(
            buf, np.uint8, sp.codes_bytes, base + d["packed_offset"])
        out[sp.scales_offset:sp.scales_offset + sp.scales_bytes] = np.frombuffer(
            buf, np.uint8, sp.scales_bytes, base + d["scales_offset"])
    return out
