"""Pins for the CPU oracle: checks against what the pages print and what the
mathematics fixes, never against the oracle's own formulas retyped.

Each test names the page section it follows. Every check here runs on CPU.
"""

import math

import numpy as np
import pytest
import scipy.special

import oracle as O
import synth
from conftest import read_golden


# ---------------------------------------------------------------- levels ---

def test_q2_levels_match_printed_values():
    # "SMOE Quantisation", Quantisation Levels: -1.0, -0.333, +0.333, +1.0
    rows = read_golden("q2_levels.txt")
    printed = {int(r[0].split()[0]): float(r[0].split()[1]) for r in rows}
    packed = O.pack_codes(np.array([0, 1, 2, 3]), 2)
    W = O.dequantise(packed, np.array([1.0]), 1, 4, 2)[0]
    for c in range(4):
        assert abs(W[c] - printed[c]) < 5e-4
    # exact closed form: +-1 and +-1/3
    assert W[0] == -1.0 and W[3] == 1.0
    assert abs(W[1] + 1.0 / 3.0) < 1e-15 and abs(W[2] - 1.0 / 3.0) < 1e-15


def test_q4_levels_closed_form():
    # "SMOE Quantisation", Quantisation Levels (16 symmetric levels) and the
    # Metal decode: (code - 7.5) / 7.5 * scale
    packed = O.pack_codes(np.arange(16), 4)
    W = O.dequantise(packed, np.array([1.0]), 1, 16, 4)[0]
    assert W[0] == -1.0 and W[15] == 1.0
    for c in range(16):
        assert W[15 - c] == -W[c]           # symmetric, exactly
    assert np.all(W != 0.0)                  # no zero level
    d = np.diff(W)
    assert np.allclose(d, 2.0 / 15.0, rtol=0, atol=1e-15)  # uniform spacing


def test_scale_multiplies_level():
    packed = O.pack_codes(np.array([0, 5, 15, 9]), 4)
    a = O.dequantise(packed, np.array([1.0]), 1, 4, 4)
    b = O.dequantise(packed, np.array([0.37]), 1, 4, 4)
    assert np.allclose(b, 0.37 * a, rtol=1e-15, atol=0)


# --------------------------------------------------------------- packing ---

def test_packing_worked_bytes():
    # "SMOE Quantisation", Bit Packing (LSB-first); bytes derived by hand
    for bits, codes, hexbytes in read_golden("packing_worked_bytes.txt"):
        bits = int(bits)
        codes = [int(c) for c in codes.split()]
        want = bytes(int(h, 16) for h in hexbytes.split())
        got = O.pack_codes(np.array(codes), bits).tobytes()
        assert got == want, (bits, codes)
        assert O.unpack_codes_scalar(want, len(codes), bits) == codes
        assert list(O.unpack_codes(np.frombuffer(want, np.uint8), len(codes), bits)) == codes


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_unpack_roundtrip_and_vector_matches_scalar(bits):
    r = np.random.default_rng(11)
    for n in (1, 3, 7, 64, 129, 1000):
        c = r.integers(0, 1 << bits, n)
        p = O.pack_codes(c, bits)
        assert p.size == O.packed_size(n, bits)
        assert np.array_equal(O.unpack_codes(p, n, bits), c)
        assert O.unpack_codes_scalar(p.tolist(), n, bits) == c.tolist()


def test_pack_rejects_out_of_range():
    with pytest.raises(ValueError):
        O.pack_codes(np.array([4]), 2)
    with pytest.raises(ValueError):
        O.pack_codes(np.array([16]), 4)


def test_flattened_groups_straddle_rows():
    # ".smoe Binary Format", Expert Blob Architecture: ceil(rows*cols/64)
    # scales over the flattened tensor; worked case written out by hand
    packed = O.pack_codes(np.full(2 * 96, 15), 4)
    W = O.dequantise(packed, np.array([1.0, 2.0, 3.0]), 2, 96, 4)
    for row, rng_, value in read_golden("flat_group_dequant.txt"):
        lo, hi = (int(v) for v in rng_.split())
        assert np.all(W[int(row), lo:hi + 1] == float(value))


# ----------------------------------------------------------------- sizes ---

def test_blob_size_formula_reproduces_printed_table():
    # "SMOE Quantisation", Why Quantise: ~38 MB -> ~195/s, ~10 MB -> ~740/s,
    # ~5 MB (Q2) at ~7.4 GB/s; .smoe scales are fp16
    rows = {r[0]: r[1:] for r in read_golden("blob_size_table.txt")}
    ssd = float(rows["ssd_GBps"][0]) * 1e9
    bf16_size = 3 * 4096 * 1536 * 2
    q4 = O.expert_layout(4096, 1536, 4, "f16").raw_size
    q2 = O.expert_layout(4096, 1536, 2, "f16").raw_size
    for name, size in (("bf16", bf16_size), ("q4", q4), ("q2", q2)):
        mb, rate, use_rate = rows[name]
        assert abs(size / 1e6 - float(mb)) / float(mb) < 0.07, name
        if use_rate == "yes":
            assert abs(ssd / size - float(rate)) / float(rate) < 0.01, name
    assert q4 == 10_027_008 and q2 == 5_308_416


def test_layout_offsets_worked_by_hand():
    for head, vals in read_golden("qwen_q4_f32_layout.txt"):
        d, ffn, bits, sbytes = (int(v) for v in head.split())
        want = [int(v) for v in vals.split()]
        L = O.expert_layout(d, ffn, bits, "f32" if sbytes == 4 else "f16")
        got = [L.gate.codes_offset, L.gate.scales_offset, L.up.codes_offset,
               L.up.scales_offset, L.down.codes_offset, L.down.scales_offset,
               L.raw_size, L.padded_size]
        assert got == want
        assert L.padded_size % 16384 == 0


def test_blob_build_and_read_back():
    r = synth.rng(5)
    L = O.expert_layout(128, 64, 4, "f32")
    tensors = {}
    for name, span in L.spans().items():
        tensors[name] = (synth.uniform_bytes(r, span.codes_bytes),
                         synth.lognormal_f32(r, span.n_scales))
    blob = O.build_expert_blob(L, tensors)
    assert blob.size == L.padded_size
    assert np.all(blob[L.raw_size:] == 0)
    W = O.read_expert_tensors(blob, L)
    assert W["gate"].shape == (64, 128) and W["down"].shape == (128, 64)
    for name in ("gate", "up", "down"):
        codes, scales = tensors[name]
        span = L.spans()[name]
        ref = O.dequantise(codes, scales, span.rows, span.cols, 4)
        assert np.array_equal(W[name], ref)


# ------------------------------------------------------------- quantiser ---

def test_candidate_grid():
    # "SMOE Quantisation", L2-MSE Scale Optimiser: 64 candidates, 0.1 .. 1.0
    c = O.candidate_fractions()
    assert c.size == 64 and c[0] == 0.1 and c[-1] == 1.0
    assert np.allclose(np.diff(c), 0.9 / 63, rtol=0, atol=1e-15)


def _mse_with_table(w, s, codes, bits):
    # independent decode through the pinned level table
    lv = O.level_table(bits)
    return float(np.sum((np.asarray(w, np.float64) - lv[codes] * s) ** 2))


def _brute_force_best(w, bits):
    # every candidate, every code chosen by nearest level (ties to even code
    # index are resolved by exhaustive search over the 2^bits levels)
    lv = O.level_table(bits)
    a = float(np.max(np.abs(w)))
    best = None
    for i, f in enumerate(O.candidate_fractions()):
        s = float(np.float32(f * a))
        # nearest level for each weight, exhaustive over codes
        err_per_code = (np.asarray(w)[:, None] - lv[None, :] * s) ** 2
        codes = np.argmin(err_per_code, axis=1)
        mse = float(np.sum((np.asarray(w) - lv[codes] * s) ** 2))
        if best is None or mse < best[0] - 1e-18:
            best = (mse, i, s)
    return best


@pytest.mark.parametrize("bits", [2, 4])
def test_mse_grid_never_worse_than_absmax_and_in_range(bits):
    r = np.random.default_rng(3)
    for _ in range(40):
        w = r.standard_normal(64) * 0.02
        s, codes, i = O.mse_grid_scale(w, bits)
        a = float(np.max(np.abs(w)))
        assert 0.1 * a * (1 - 1e-6) <= s <= a * (1 + 1e-6)
        err = _mse_with_table(w, s, codes, bits)
        s_abs = float(np.float32(a))
        c_abs = O.encode_codes(w, s_abs, bits)
        assert err <= _mse_with_table(w, s_abs, c_abs, bits) + 1e-18


@pytest.mark.parametrize("bits", [2, 4])
def test_mse_grid_matches_brute_force(bits):
    # the nearest-level encoder and the chosen candidate agree with an
    # exhaustive search over (candidate, code) pairs
    r = np.random.default_rng(17)
    for _ in range(25):
        w = r.standard_normal(64) * 0.02
        w[r.integers(0, 64)] *= 10
        s, codes, i = O.mse_grid_scale(w, bits)
        mse = _mse_with_table(w, s, codes, bits)
        bmse, bi, bs = _brute_force_best(w, bits)
        assert abs(mse - bmse) <= 1e-15 * max(1.0, bmse) + 1e-20
        assert i == bi and s == bs


def test_f16_candidate_roundings_worked_by_hand(golden):
    # the fixture's fp16 values are derived by hand from the fp16 format
    # (11-bit significand, subnormal step 2^-24, ties to even)
    for row in golden("f16_scale_candidates.txt"):
        absmax, i, prod, want = float(row[0]), int(row[1]), float(row[2]), float(row[3])
        assert O.candidate_fractions()[i] * absmax == prod
        assert float(np.float16(prod)) == want


def test_f16_scale_is_the_rounded_candidate():
    # "SMOE Quantisation", L2-MSE Scale Optimiser, with fp16 storage: a group
    # lying on the level grid of the fp16 value of its absmax candidate (and
    # whose absmax element is 1 + 2^-11 or 1 + 3 * 2^-11, halfway between two
    # fp16 values) is stored with the tie-to-even fp16 scale: 1.0 and
    # 1 + 2^-9, not the fp32 values of the candidates
    r = np.random.default_rng(9)
    for absmax, want in ((1.00048828125, 1.0), (1.00146484375, 1.001953125)):
        for bits in (2, 4):
            lv = O.level_table(bits)
            # codes below the top level, so no element but the first reaches
            # the scale; the first is the absmax, just off the grid
            codes = r.integers(1, (1 << bits) - 1, 64)
            w = lv[codes] * want
            w[0] = absmax
            s16, c16, i16 = O.mse_grid_scale(w, bits, "f16")
            assert i16 == 63 and s16 == want
            s32, _, i32 = O.mse_grid_scale(w, bits, "f32")
            assert s32 != want


@pytest.mark.parametrize("bits", [2, 4])
def test_mse_grid_f16_matches_brute_force(bits):
    # exhaustive search over (candidate, code) pairs with every candidate
    # stored as fp16 (the rounding pinned by the fixture above)
    lv = O.level_table(bits)
    r = np.random.default_rng(23)
    for _ in range(25):
        w = r.standard_normal(64) * 0.02
        w[r.integers(0, 64)] *= 10
        a = float(np.max(np.abs(w)))
        best = None
        for i, f in enumerate(O.candidate_fractions()):
            sc = float(np.float16(f * a))
            err = np.min((w[:, None] - lv[None, :] * sc) ** 2, axis=1).sum()
            if best is None or err < best[0] - 1e-18:
                best = (err, i, sc)
        s, codes, i = O.mse_grid_scale(w, bits, "f16")
        assert i == best[1] and s == best[2]
        assert abs(_mse_with_table(w, s, codes, bits) - best[0]) <= 1e-15 * max(1.0, best[0])


def test_outlier_group_picks_smaller_scale():
    # "SMOE Quantisation", L2-MSE Scale Optimiser: one loud outlier among
    # near-zero weights pulls the scale below absmax
    r = np.random.default_rng(1)
    w = r.standard_normal(64) * 0.01
    w[5] = 1.0
    for bits in (2, 4):
        s, codes, _ = O.mse_grid_scale(w, bits)
        assert s < 0.99
        # the small weights are better preserved than with the absmax scale
        small = np.arange(64) != 5
        lv = O.level_table(bits)
        e_grid = np.sum((w[small] - lv[codes[small]] * s) ** 2)
        c_abs = O.encode_codes(w, 1.0, bits)
        e_abs = np.sum((w[small] - lv[c_abs[small]] * 1.0) ** 2)
        assert e_grid < e_abs


@pytest.mark.parametrize("bits", [2, 4])
def test_exact_recovery_on_a_candidate_grid(bits):
    # weights that lie exactly on the level grid of candidate i0 (with the
    # absmax equal to the scale's level-1 weight) are reproduced exactly
    lv = O.level_table(bits)
    r = np.random.default_rng(2)
    codes = r.integers(0, 1 << bits, 64)
    codes[0] = (1 << bits) - 1          # a +1 level so absmax == scale
    w = lv[codes] * 0.75
    s, got, i = O.mse_grid_scale(w, bits)
    assert i == 63 and s == 0.75
    assert np.array_equal(got, codes)


def test_zero_group_and_rounding_mode():
    s, codes, _ = O.mse_grid_scale(np.zeros(64), 4)
    assert s == 0.0 and np.all(codes == 8)      # rint(7.5) -> 8 (half-even)
    s, codes, _ = O.mse_grid_scale(np.zeros(64), 2)
    assert s == 0.0 and np.all(codes == 2)      # rint(1.5) -> 2
    # half-even at an exact tie: w/s*7.5 + 7.5 = 8.5 -> 8, 9.5 -> 10
    assert O.encode_codes(np.array([1 / 7.5]), 1.0, 4)[0] == 8
    assert O.encode_codes(np.array([2 / 7.5]), 1.0, 4)[0] == 10
    # clamping
    assert O.encode_codes(np.array([5.0, -5.0]), 1.0, 4).tolist() == [15, 0]


def test_quantise_tensor_groups_and_snr():
    # Q4 on N(0,1) beats Q2 by a wide margin; Q2 SNR on a 128 x 64 Gaussian
    # is in a loose band around the page's "~6 dB" remark (the printed
    # numbers of the page's smoke test are not reproducible).
    r = np.random.default_rng(0)
    W = r.standard_normal((128, 64))
    snr = {}
    for bits in (2, 4):
        p, s = O.quantise_tensor(W, bits)
        assert s.size == 128 and s.dtype == np.float32
        R = O.dequantise(p, s, 128, 64, bits)
        snr[bits] = 10 * math.log10(np.sum(W ** 2) / np.sum((W - R) ** 2))
    assert 4.0 < snr[2] < 12.0
    assert snr[4] > snr[2] + 8.0


# ---------------------------------------------------------------- routing ---

def test_route_matches_stable_argsort_and_softmax():
    # "CMF v2 Format Specification", 2.2: softmax over all logits, top-k with
    # ties to the lower index, optional renormalisation
    r = np.random.default_rng(4)
    for E, k in ((128, 8), (64, 6), (8, 8), (1, 1), (16, 16)):
        for _ in range(20):
            l = r.standard_normal(E).astype(np.float32)
            ids, w = O.route(l, k, False)
            assert ids == list(np.argsort(-l, kind="stable")[:k])
            p = scipy.special.softmax(l.astype(np.float64))
            assert np.allclose(w, p[ids], rtol=1e-13, atol=0)
            ids2, w2 = O.route(l, k, True)
            assert ids2 == ids
            assert np.allclose(w2, p[ids] / p[ids].sum(), rtol=1e-13, atol=0)
            assert abs(w2.sum() - 1.0) < 1e-14


def test_route_ties_go_to_lower_index():
    l = np.zeros(16, dtype=np.float32)
    l[[3, 9, 12]] = 2.0
    ids, _ = O.route(l, 5, True)
    assert ids == [3, 9, 12, 0, 1]
    # fp32 ties that differ in fp64 do not exist; equal fp32 values tie
    l = np.array([1.0, 1.0 + 2 ** -23, 1.0], dtype=np.float32)
    assert O.route(l, 2, True)[0] == [1, 0]


def test_route_special_cases():
    l = np.full(32, 0.5, dtype=np.float32)
    ids, w = O.route(l, 4, True)
    assert ids == [0, 1, 2, 3] and np.allclose(w, 0.25, rtol=0, atol=1e-16)
    r = np.random.default_rng(8).standard_normal(16).astype(np.float32)
    ids, w = O.route(r, 16, True)
    assert abs(w.sum() - 1.0) < 1e-15
    ids, w = O.route(r, 1, True)
    assert w[0] == 1.0
    ids, w = O.route(r, 3, False)
    assert w.sum() < 1.0
    for bad in (0, 17):
        with pytest.raises(ValueError):
            O.route(np.zeros(64, np.float32), bad, True)
    with pytest.raises(ValueError):
        O.route(np.zeros(4, np.float32), 5, True)


# ------------------------------------------------------------ expert FFN ---

def _scalar_expert(blob, L, x):
    """Brute force straight from the packed bytes: scalar unpack, explicit
    loops, named gate/up/down tensors."""
    def mat(span):
        codes = O.unpack_codes_scalar(
            blob[span.codes_offset: span.codes_offset + span.codes_bytes].tolist(),
            span.rows * span.cols, L.bits)
        sc = blob[span.scales_offset: span.scales_offset + span.scales_bytes
                  ].copy().view(np.float32).astype(np.float64).tolist()
        lv = O.level_table(L.bits).tolist()
        return [[lv[codes[r * span.cols + c]] * sc[(r * span.cols + c) // 64]
                 for c in range(span.cols)] for r in range(span.rows)]
    G, U, D = mat(L.gate), mat(L.up), mat(L.down)
    xs = [float(v) for v in x]
    g = [sum(G[i][j] * xs[j] for j in range(L.d_model)) for i in range(L.ffn_dim)]
    u = [sum(U[i][j] * xs[j] for j in range(L.d_model)) for i in range(L.ffn_dim)]
    h = [g[i] / (1.0 + math.exp(-g[i])) * u[i] for i in range(L.ffn_dim)]
    return [sum(D[o][i] * h[i] for i in range(L.ffn_dim)) for o in range(L.d_model)]


def _random_expert_blob(seed, d, ffn, bits):
    r = synth.rng(seed)
    L = O.expert_layout(d, ffn, bits, "f32")
    tensors = {n: (synth.uniform_bytes(r, s.codes_bytes), synth.lognormal_f32(r, s.n_scales))
               for n, s in L.spans().items()}
    return L, O.build_expert_blob(L, tensors)


@pytest.mark.parametrize("bits", [2, 4])
def test_expert_matches_scalar_brute_force(bits):
    # non-square shapes so a transposed operand cannot pass
    L, blob = _random_expert_blob(21 + bits, 128, 64, bits)
    x = synth.normal_f32(synth.rng(7), 128)
    W = O.read_expert_tensors(blob, L)
    y = O.swiglu_expert(W["gate"], W["up"], W["down"], x)
    ref = _scalar_expert(blob, L, x)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_expert_constant_code_closed_form():
    # constant codes: every gate row gives lg*sg*sum(x), every up row
    # lu*su*sum(x), every down row ld*sd*ffn*silu(g)*u
    d, ffn = 128, 64
    L = O.expert_layout(d, ffn, 4, "f32")
    cg, cu, cd = 12, 3, 9
    sg, su, sd = 0.05, 0.07, 0.011
    lv = O.level_table(4)
    tensors = {}
    for name, c, s in (("gate", cg, sg), ("up", cu, su), ("down", cd, sd)):
        span = L.spans()[name]
        tensors[name] = (O.pack_codes(np.full(span.rows * span.cols, c), 4),
                         np.full(span.n_scales, s, np.float32))
    blob = O.build_expert_blob(L, tensors)
    x = synth.normal_f32(synth.rng(3), d)
    W = O.read_expert_tensors(blob, L)
    y = O.swiglu_expert(W["gate"], W["up"], W["down"], x)
    sx = float(np.sum(x.astype(np.float64)))
    g = lv[cg] * float(np.float32(sg)) * sx
    u = lv[cu] * float(np.float32(su)) * sx
    h = g / (1 + math.exp(-g)) * u
    want = lv[cd] * float(np.float32(sd)) * ffn * h
    assert np.allclose(y, want, rtol=1e-12, atol=0)


def test_silu_values():
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert abs(O.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    v = O.silu(np.array([-1000.0, 1000.0]))
    assert v[0] == 0.0 and v[1] == 1000.0
    assert abs(O.silu(np.array([2.0]))[0] - 2.0 * scipy.special.expit(2.0)) < 1e-15


# ------------------------------------------------------------------ layer ---

def _layer(seed, d, ffn, E, bits, shared=0, zero_routed=False):
    r = synth.rng(seed)
    L = O.expert_layout(d, ffn, bits, "f32")
    blobs = []
    for e in range(E):
        t = {}
        for n, s in L.spans().items():
            sc = synth.lognormal_f32(r, s.n_scales)
            if zero_routed:
                sc[:] = 0
            t[n] = (synth.uniform_bytes(r, s.codes_bytes), sc)
        blobs.append(O.build_expert_blob(L, t))
    sblob = None
    if shared:
        SL = O.expert_layout(d, shared, bits, "f32")
        sblob = O.build_expert_blob(SL, {n: (synth.uniform_bytes(r, s.codes_bytes),
                                              synth.lognormal_f32(r, s.n_scales))
                                          for n, s in SL.spans().items()})
    return O.OracleLayer(d, ffn, E, bits, np.concatenate(blobs), shared_ffn_dim=shared,
                         shared_blob=sblob)


def test_single_expert_top1_layer_is_plain_swiglu():
    layer = _layer(1, 128, 64, 1, 4)
    x = synth.normal_f32(synth.rng(2), (1, 128))
    out, ids, w = O.moe_forward(layer, x, np.zeros((1, 1), np.float32), 1, True)
    W = layer.expert_weights(0)
    assert ids.tolist() == [[0]] and w[0, 0] == 1.0
    assert np.array_equal(out[0], O.swiglu_expert(W["gate"], W["up"], W["down"], x[0]))


def test_layer_is_weighted_sum_of_selected_experts():
    layer = _layer(2, 128, 64, 8, 4)
    r = synth.rng(9)
    x = synth.normal_f32(r, (3, 128))
    lg = synth.normal_f32(r, (3, 8))
    out, ids, w = O.moe_forward(layer, x, lg, 3, False)
    for t in range(3):
        acc = np.zeros(128)
        for j, e in enumerate(ids[t]):
            W = layer.expert_weights(int(e))
            acc += w[t, j] * O.swiglu_expert(W["gate"], W["up"], W["down"], x[t])
        assert np.allclose(out[t], acc, rtol=1e-14, atol=1e-16)
        # unselected experts do not matter
        assert set(ids[t].tolist()) == set(np.argsort(-lg[t], kind="stable")[:3].tolist())


def test_zero_scales_give_zero_and_shared_expert_weight_one():
    layer = _layer(3, 128, 64, 4, 4, shared=192, zero_routed=True)
    x = synth.normal_f32(synth.rng(4), (2, 128))
    lg = synth.normal_f32(synth.rng(5), (2, 4))
    out, _, _ = O.moe_forward(layer, x, lg, 2, True)
    S = layer.shared_weights()
    for t in range(2):
        assert np.allclose(out[t], O.swiglu_expert(S["gate"], S["up"], S["down"], x[t]),
                           rtol=1e-14, atol=0)
    layer0 = _layer(3, 128, 64, 4, 4, zero_routed=True)
    out0, _, _ = O.moe_forward(layer0, x, lg, 2, True)
    assert np.all(out0 == 0.0)


# ------------------------------------------------------------------ stack ---

def test_rms_norm_closed_forms():
    c = 3.0
    v = O.rms_norm(np.full((1, 16), c))
    assert np.allclose(v, c / math.sqrt(c * c + 1e-6), rtol=1e-15, atol=0)
    h = np.random.default_rng(1).standard_normal((2, 64))
    n = O.rms_norm(h)
    assert np.allclose(np.mean(n * n, axis=-1), 1.0 / (1.0 + 1e-6 / np.mean(h * h, axis=-1)),
                       rtol=1e-12)
    # scale invariance up to the eps term: norm(a h) / norm(h) is the ratio
    # sqrt(ms + eps) / sqrt(ms + eps / a^2) for every element
    ms = np.mean(h * h, axis=-1, keepdims=True)
    ratio = np.sqrt(ms + 1e-6) / np.sqrt(ms + 1e-6 / 1e6)
    assert np.allclose(O.rms_norm(h * 1e3), O.rms_norm(h) * ratio, rtol=1e-12)
    assert not np.allclose(O.rms_norm(h * 1e3), O.rms_norm(h), rtol=1e-9)


def test_decode_step_norm_placement_closed_form():
    # ".smoe Binary Format", Arch Block (rms eps 1e-6): each layer adds
    # MoE(rms_norm(h)) to h. One expert with every code 12 (level 4.5 / 7.5 =
    # 0.6) and every scale 2^-7, on a constant h = a: rms_norm(h) is the
    # constant nu = a / sqrt(a^2 + eps), gate = up = 0.6 * 2^-7 * d * nu on
    # every row, and the down output is 0.6 * 2^-7 * ffn * silu(g) * g on
    # every element. Dropping the norm, applying it after the layer, or
    # taking eps outside the root gives a different value.
    d, ffn, L, s = 64, 64, 0.6, 2.0 ** -7
    lay = O.expert_layout(d, ffn, 4, "f32")
    blob = np.zeros(lay.padded_size, np.uint8)
    for span in lay.spans().values():
        blob[span.codes_offset: span.codes_offset + span.codes_bytes] = 0xCC  # codes 12, 12
        blob[span.scales_offset: span.scales_offset + span.scales_bytes] = \
            np.full(span.n_scales, s, np.float32).view(np.uint8)
    layer = O.OracleLayer(d, ffn, 1, 4, blob)
    lg = [np.zeros((1, 1), np.float32)] * 2

    def silu(v):
        return v / (1.0 + math.exp(-v))

    for a in (0.5, 1e-3):
        x = np.full((1, d), a)
        h = O.decode_step([layer, layer], x, lg, 1, True)
        want = a
        for _ in range(2):
            nu = want / math.sqrt(want * want + 1e-6)
            g = L * s * d * nu
            want = want + L * s * ffn * silu(g) * g
        assert np.allclose(h, want, rtol=1e-13, atol=0)
        # the same layer without the norm, or with eps outside the root
        g_raw = L * s * d * a
        assert abs((a + L * s * ffn * silu(g_raw) * g_raw) - h[0, 0]) > 1e-9
        nu_bad = a / (math.sqrt(a * a) + 1e-6)
        g_bad = L * s * d * nu_bad
        one_bad = a + L * s * ffn * silu(g_bad) * g_bad
        nu1 = a / math.sqrt(a * a + 1e-6)
        one = a + L * s * ffn * silu(L * s * d * nu1) * (L * s * d * nu1)
        assert abs(one_bad - one) > 1e-12 or a == 0.5


def test_decode_step_zero_layers_keep_residual_and_chain():
    layers = [_layer(10 + i, 128, 64, 4, 4, zero_routed=True) for i in range(5)]
    x = synth.normal_f32(synth.rng(0), (1, 128))
    lgs = [synth.normal_f32(synth.rng(20 + i), (1, 4)) for i in range(5)]
    h = O.decode_step(layers, x, lgs, 2, True)
    assert np.array_equal(h, x.astype(np.float64))
    # two real layers: equals the explicit chain
    L2 = [_layer(30 + i, 128, 64, 4, 4) for i in range(2)]
    h = O.decode_step(L2, x, lgs[:2], 2, True)
    ref = x.astype(np.float64)
    for layer, lg in zip(L2, lgs[:2]):
        n = ref / np.sqrt(np.mean(ref * ref) + 1e-6)
        y, _, _ = O.moe_forward(layer, n, lg, 2, True)
        ref = ref + y
    assert np.allclose(h, ref, rtol=1e-14, atol=0)
