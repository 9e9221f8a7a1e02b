"""Pins for the oracle's routing variants ("CMF v2 Format Specification",
2.2 MoE; 5. Masks section): checks against closed forms and hand-worked
cases, not against the oracle's formulas retyped. CPU only.
"""

import math

import numpy as np
import pytest
import scipy.special

import oracle as O
from helpers import random_layer

LN3 = math.log(3.0)


def test_default_options_are_plain_routing():
    r = np.random.default_rng(11)
    for _ in range(20):
        lg = r.standard_normal(32).astype(np.float32)
        for norm in (False, True):
            a = O.route(lg, 6, norm)
            b = O.route_ex(lg, 6, norm, O.RouteOpts())
            assert a[0] == b[0]
            assert np.array_equal(a[1], b[1])


def test_sigmoid_scores_are_independent_per_expert():
    # 2.2 MoE: router_sigmoid scores each expert with sigmoid; sigmoid(ln 3)
    # = 3/4, sigmoid(0) = 1/2, sigmoid(-ln 3) = 1/4 exactly
    lg = np.array([-LN3, 0.0, LN3, -5.0], dtype=np.float32)
    ids, w = O.route_ex(lg, 3, False, O.RouteOpts(sigmoid=True))
    assert ids == [2, 1, 0]
    assert np.allclose(w, [0.75, 0.5, 0.25], rtol=0, atol=1e-7)
    # unlike softmax, the weights do not sum to 1 and do not depend on the
    # other experts' logits
    lg2 = lg.copy()
    lg2[3] = 4.0
    ids2, w2 = O.route_ex(lg2, 4, False, O.RouteOpts(sigmoid=True))
    assert ids2 == [3, 2, 1, 0]
    assert np.allclose(w2[1:], [0.75, 0.5, 0.25], rtol=0, atol=1e-7)
    # renormalised: 3:2:1
    _, wn = O.route_ex(lg, 3, True, O.RouteOpts(sigmoid=True))
    assert np.allclose(wn, [0.5, 1 / 3, 1 / 6], rtol=0, atol=1e-7)


def test_bias_changes_selection_not_weights():
    # 2.2 MoE: expert_bias affects the top-k selection only
    lg = np.zeros(4, dtype=np.float32)
    bias = np.array([0.0, 0.0, 1.0, 0.0], dtype=np.float32)
    ids, w = O.route_ex(lg, 1, False, O.RouteOpts(expert_bias=bias))
    assert ids == [2] and w[0] == 0.25           # softmax over 4 equal logits
    ids, w = O.route_ex(lg, 2, False, O.RouteOpts(expert_bias=bias))
    assert ids == [2, 0]                         # then the tie goes to the lower id
    assert np.allclose(w, [0.25, 0.25], rtol=0, atol=1e-15)
    # with sigmoid scoring the gathered weight is sigmoid(logit), not + bias
    ids, w = O.route_ex(np.array([LN3, 0.0], np.float32), 1, False,
                        O.RouteOpts(sigmoid=True, expert_bias=np.array([0.0, 0.3], np.float32)))
    assert ids == [1] and abs(w[0] - 0.5) < 1e-7  # 0.5 + 0.3 > 0.75
    # a bias that does not change the order changes nothing
    lg = np.array([3.0, 2.0, 1.0, 0.0], dtype=np.float32)
    a = O.route_ex(lg, 2, True, O.RouteOpts())
    b = O.route_ex(lg, 2, True, O.RouteOpts(expert_bias=np.array([0.01, 0, 0, 0], np.float32)))
    assert a[0] == b[0] and np.allclose(a[1], b[1], rtol=0, atol=1e-15)


def test_scaling_applies_after_renormalisation():
    # 2.2 MoE: optionally renormalise, then apply routed_scaling_factor
    r = np.random.default_rng(5)
    lg = r.standard_normal(64).astype(np.float32)
    _, w = O.route_ex(lg, 8, True, O.RouteOpts(scaling=2.5))
    assert abs(np.sum(w) - 2.5) < 1e-12
    _, w1 = O.route_ex(lg, 8, False, O.RouteOpts())
    _, w2 = O.route_ex(lg, 8, False, O.RouteOpts(scaling=2.5))
    assert np.allclose(w2, 2.5 * w1, rtol=1e-15, atol=0)


def test_mask_restricts_selection_and_renormalises_softmax():
    # 5. Masks section: selection over the routable set only, the router
    # softmax renormalising over it
    lg = np.array([5.0, 0.0, 0.0, 9.0], dtype=np.float32)
    mask = np.array([False, True, True, False])
    ids, w = O.route_ex(lg, 2, False, O.RouteOpts(mask=mask))
    assert ids == [1, 2]
    assert np.allclose(w, [0.5, 0.5], rtol=0, atol=1e-15)
    # an all-true mask restricts nothing
    a = O.route_ex(lg, 2, False, O.RouteOpts())
    b = O.route_ex(lg, 2, False, O.RouteOpts(mask=np.ones(4, bool)))
    assert a[0] == b[0] and np.allclose(a[1], b[1], rtol=1e-15, atol=0)
    # the softmax over the routable set equals scipy's on that subset
    r = np.random.default_rng(3)
    lg = r.standard_normal(16).astype(np.float32)
    m = r.random(16) < 0.5
    m[:4] = True
    ids, w = O.route_ex(lg, 4, False, O.RouteOpts(mask=m))
    sub = np.flatnonzero(m)
    p = scipy.special.softmax(lg[sub].astype(np.float64))
    want = sub[np.argsort(-lg[sub], kind="stable")][:4]
    assert ids == [int(e) for e in want]
    assert np.allclose(w, [p[list(sub).index(e)] for e in ids], rtol=1e-12)
    with pytest.raises(ValueError):
        O.route_ex(lg, 5, False, O.RouteOpts(mask=np.arange(16) < 4))


def test_shared_gate_weights_the_shared_expert():
    # 2.2 MoE: the shared expert is added with weight
    # sigmoid(shared_expert_gate . x) when that tensor is present
    hl = random_layer(21, 128, 64, 4, 4, "f32", 128)
    ol = hl.oracle()
    r = np.random.default_rng(22)
    x = r.standard_normal((3, 128)).astype(np.float32)
    lg = r.standard_normal((3, 4)).astype(np.float32)
    plain, _, _ = O.moe_forward(ol, x, lg, 2, True)
    zero_gate, _, _ = O.moe_forward(ol, x, lg, 2, True,
                                    opts=O.RouteOpts(shared_gate=np.zeros(3, np.float32)))
    ln3_gate, _, _ = O.moe_forward(ol, x, lg, 2, True,
                                   opts=O.RouteOpts(shared_gate=np.full(3, LN3, np.float32)))
    # plain = routed + S, zero gate = routed + S/2, ln 3 gate = routed + 3S/4
    S = 2.0 * (plain - zero_gate)
    assert np.allclose(ln3_gate, plain - S / 4.0, rtol=1e-6, atol=1e-9)
    assert np.max(np.abs(S)) > 0.0


def test_biased_selection_is_decided_in_float64():
    # 2.2 MoE: the bias is added to the score for the selection. Two equal
    # logits but for 2^-20: softmax scores 1/2 -+ tanh(2^-21) (closed form),
    # and a bias on expert 0 of 2^-21 - 2^-30 (exact in fp32). The exact keys
    # differ by 2^-30 - (tanh(2^-21) - 2^-21), i.e. expert 1 is ahead by
    # about 2^-30; an fp32 sum would round both keys to 1/2 + 2^-22 and the
    # tie would go to expert 0.
    d = 2.0 ** -20
    lg = np.array([0.0, d], dtype=np.float32)
    assert float(lg[1]) == d
    bias = np.array([2.0 ** -21 - 2.0 ** -30, 0.0], dtype=np.float32)
    assert float(bias[0]) == 2.0 ** -21 - 2.0 ** -30
    p0, p1 = 0.5 - math.tanh(d / 2) / 2, 0.5 + math.tanh(d / 2) / 2
    assert (p0 + float(bias[0])) < p1                      # exact order: 1 first
    assert np.float32(np.float32(p0) + bias[0]) == np.float32(p1)  # fp32 ties
    ids, w = O.route_ex(lg, 1, False, O.RouteOpts(expert_bias=bias))
    assert ids == [1]
    assert abs(w[0] - p1) < 1e-15
    ids, _ = O.route_ex(lg, 2, False, O.RouteOpts(expert_bias=bias))
    assert ids == [1, 0]
    # the same with sigmoid scoring: sigmoid(0) = 1/2, sigmoid(2^-20) =
    # 1/2 + tanh(2^-21)/2 in closed form
    s1 = 0.5 + math.tanh(d / 2) / 2
    b2 = np.array([2.0 ** -22 - 2.0 ** -31, 0.0], dtype=np.float32)
    assert (0.5 + float(b2[0])) < s1
    ids, w = O.route_ex(lg, 1, False, O.RouteOpts(sigmoid=True, expert_bias=b2))
    assert ids == [1] and abs(w[0] - s1) < 1e-15
