"""Pins of the fp64 CPU oracle against what the pages and mathematics fix.

Each test ties one oracle function to something other than itself: values
worked by hand (tests/golden/), closed forms, invariants, special cases that
reduce to a library routine, or brute force on tiny inputs.  The cases are
chosen so that a dropped term, a wrong sign or index, or a transposed operand
fails at least one of them.
"""
import itertools
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle
import synthetic as syn

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLD, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def _bf16(bits_hex):
    return float(syn.bf16_bits_to_f32(np.array([int(bits_hex, 16)], np.uint16))[0])


# --------------------------------------------------------------------------- #
# dequantisation and the FMA identity (hand-worked, golden)
# --------------------------------------------------------------------------- #
def test_dequant_hand_worked():
    for q, sh, bh, x, w, qsx, bx, prod in _rows("dequant_worked.txt"):
        q, x = int(q), float(x)
        s, b = _bf16(sh), _bf16(bh)
        assert oracle.dequant(q, int(sh, 16), int(bh, 16)) == float(w)
        # the page's rewrite: (q*s + b)*x == q*(s*x) + b*x, exactly on dyadic values
        assert q * (s * x) == float(qsx) and b * x == float(bx)
        assert float(qsx) + float(bx) == float(prod) == float(w) * x
        # the same product through the quantised GEMV: one row of 64 columns,
        # x placed at a column that is not the first, other columns zero
        for col in (0, 37):
            codes = np.zeros((1, 64), np.uint8)
            codes[0, col] = q
            v = np.zeros(64)
            v[col] = x
            out = oracle.qgemv(codes, np.array([[int(sh, 16)]], np.uint16),
                               np.array([[int(bh, 16)]], np.uint16), v)
            assert out[0] == float(prod)


def test_code_zero_gives_bias():
    for bias in (-0.1, -0.05078125, 0.0):
        bb = int(syn.f32_to_bf16_bits(np.array([bias], np.float32))[0])
        assert oracle.dequant(0, 0x3C00, bb) == _bf16(f"{bb:04X}")


def _dyadic_case(rng, rows, cols, group=64):
    codes = rng.integers(0, 16, size=(rows, cols), dtype=np.uint8)
    # scales/biases with 4-bit mantissas and small exponents: exact in bf16
    s = rng.integers(1, 16, size=(rows, cols // group)) * 2.0 ** rng.integers(-9, -5, size=(rows, cols // group))
    b = -rng.integers(0, 16, size=(rows, cols // group)) * 2.0 ** rng.integers(-8, -4, size=(rows, cols // group))
    v = rng.integers(-64, 64, size=cols) * 2.0 ** -5
    sb = syn.f32_to_bf16_bits(s.astype(np.float32))
    bb = syn.f32_to_bf16_bits(b.astype(np.float32))
    assert np.array_equal(syn.bf16_bits_to_f32(sb), s.astype(np.float32))
    return codes, sb, bb, s, b, v


def test_group_fold_closed_form():
    """sum_c (q s_g + b_g) v_c == sum_g (s_g sum_{c in g} q_c v_c + b_g sum_{c in g} v_c):
    the regrouping the GPU kernels use, exact on dyadic inputs.  Non-square,
    row- and group-dependent scales catch a wrong group index or a transposition."""
    rng = np.random.default_rng(11)
    for rows, cols in ((3, 256), (5, 128), (2, 64)):
        codes, sb, bb, s, b, v = _dyadic_case(rng, rows, cols)
        out = oracle.qgemv(codes, sb, bb, v)
        ng = cols // 64
        qv = (codes.astype(np.float64) * v).reshape(rows, ng, 64).sum(-1)
        vs = v.reshape(ng, 64).sum(-1)
        fold = (s * qv + b * vs).sum(-1)
        assert np.array_equal(out, fold)


def test_qgemv_brute_force_fractions():
    rng = np.random.default_rng(5)
    codes, sb, bb, s, b, v = _dyadic_case(rng, 2, 128)
    out = oracle.qgemv(codes, sb, bb, v)
    for r in range(2):
        acc = Fraction(0)
        for c in range(128):
            acc += (int(codes[r, c]) * Fraction(float(s[r, c // 64])) + Fraction(float(b[r, c // 64]))) * Fraction(float(v[c]))
        assert Fraction(out[r]) == acc


# --------------------------------------------------------------------------- #
# RMSNorm
# --------------------------------------------------------------------------- #
def test_rmsnorm_constant_vector_closed_form():
    H, eps = 256, 1e-6
    gamma = syn.layer_dense(0, 0, syn.Dims(H, 128, 8, 2, 4))["norm_weight"]
    g = syn.bf16_bits_to_f32(gamma).astype(np.float64)
    for c in (2.0, -0.5, 1e-3):
        h = oracle.rmsnorm(np.full(H, c, np.float32), gamma, eps)
        c64 = float(np.float32(c))
        expect = np.sign(c64) * g * abs(c64) / np.sqrt(c64 * c64 + eps)
        np.testing.assert_allclose(h, expect, rtol=1e-14, atol=0)


def test_rmsnorm_textbook():
    rng = np.random.default_rng(3)
    H = 4096
    x = rng.standard_normal(H).astype(np.float32)
    gamma = syn.f32_to_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    g = syn.bf16_bits_to_f32(gamma).astype(np.float64)
    h = oracle.rmsnorm(x, gamma, 1e-6)
    x64 = x.astype(np.float64)
    ref = x64 / np.sqrt(np.mean(x64 ** 2) + 1e-6) * g
    np.testing.assert_allclose(h, ref, rtol=1e-13)
    # eps matters for tiny inputs: x = 0 gives h = 0, not NaN
    assert np.all(oracle.rmsnorm(np.zeros(8, np.float32), gamma[:8], 1e-6) == 0)


# --------------------------------------------------------------------------- #
# router GEMV
# --------------------------------------------------------------------------- #
def test_router_gemv_matches_matmul_nonsquare():
    rng = np.random.default_rng(4)
    W = syn.f32_to_bf16_bits(rng.normal(0, 0.02, size=(24, 512)).astype(np.float32))
    h = rng.standard_normal(512)
    z = oracle.gemv_bf16(W, h)
    ref = syn.bf16_bits_to_f32(W).astype(np.float64) @ h
    np.testing.assert_allclose(z, ref, rtol=1e-12, atol=1e-15)
    # a one-hot h picks a column, not a row
    e = np.zeros(512)
    e[7] = 1.0
    np.testing.assert_array_equal(oracle.gemv_bf16(W, e), syn.bf16_bits_to_f32(W)[:, 7].astype(np.float64))


# --------------------------------------------------------------------------- #
# softmax -> top-K -> renormalise
# --------------------------------------------------------------------------- #
def test_topk_brute_force_tiny():
    rng = np.random.default_rng(8)
    E = 8
    for trial in range(200):
        z = rng.standard_normal(E)
        if trial % 3 == 0:  # constructed ties
            z = rng.integers(-2, 3, size=E).astype(np.float64)
        for K in (1, 2, 3, 5, 8):
            idx, w = oracle.route(z, K)
            # brute force: the K-subset whose key sequence (logit desc, index asc) is largest
            best = max(itertools.combinations(range(E), K),
                       key=lambda sub: sorted(((z[e], -e) for e in sub), reverse=True))
            expect = sorted(best, key=lambda e: (-z[e], e))
            assert list(idx) == expect
            p = np.exp(z - z.max()) / np.exp(z - z.max()).sum()
            np.testing.assert_allclose(w, p[expect] / p[expect].sum(), rtol=1e-14)
            assert abs(w.sum() - 1.0) < 1e-15


def test_topk_constructed_ties():
    z = np.array([1.0, 3.0, 3.0, 2.0, 3.0, 0.0, -0.0, 0.0])
    assert list(oracle.route(z, 2)[0]) == [1, 2]
    assert list(oracle.route(z, 4)[0]) == [1, 2, 4, 3]
    # -0.0 and +0.0 are the same key: index order decides
    assert list(oracle.route(z, 7)[0]) == [1, 2, 4, 3, 0, 5, 6]


def test_route_special_cases():
    # router of zeros: every logit 0 -> the first K experts, equal weights
    z = oracle.gemv_bf16(np.zeros((16, 64), np.uint16), np.ones(64))
    idx, w = oracle.route(z, 4)
    assert list(idx) == [0, 1, 2, 3] and np.all(w == 0.25)
    rng = np.random.default_rng(9)
    z = rng.standard_normal(16)
    # K = E: the weights are the full softmax, in key order
    idx, w = oracle.route(z, 16)
    np.testing.assert_allclose(w, sp_softmax(z)[idx], rtol=1e-14)
    # K = 1: weight exactly one
    idx, w = oracle.route(z, 1)
    assert w[0] == 1.0 and idx[0] == int(np.argmax(z))
    # shifting every logit by a constant changes nothing
    for c in (-30.0, 7.5, 100.0):
        i2, w2 = oracle.route(z + c, 5)
        i1, w1 = oracle.route(z, 5)
        assert list(i1) == list(i2)
        np.testing.assert_allclose(w1, w2, rtol=1e-12)
    with pytest.raises(ValueError):
        oracle.route(z, 17)


def test_near_tie_rule():
    z = np.array([3.0, 2.0, 2.0 - 1e-7, 0.0])
    assert oracle.near_tie(z, 2)
    assert not oracle.near_tie(z, 1)
    assert not oracle.near_tie(np.array([3.0, 2.0, 1.0]), 2)


# --------------------------------------------------------------------------- #
# one expert: SwiGLU FFN
# --------------------------------------------------------------------------- #
def _dense(codes, s, b, G=64):
    sd = syn.bf16_bits_to_f32(s).astype(np.float64)
    bd = syn.bf16_bits_to_f32(b).astype(np.float64)
    return codes * np.repeat(sd, G, axis=1) + np.repeat(bd, G, axis=1)


def test_expert_reduces_to_dense_swiglu_ffn():
    dims = syn.Dims(256, 128, 8, 2, 4)
    ex = syn.expert_canonical(0, 0, 3, dims)
    rng = np.random.default_rng(1)
    h = rng.standard_normal(256)
    y = oracle.expert(ex, h)
    Wg, Wu, Wd = (_dense(ex["codes"][m], ex["scale"][m], ex["bias"][m]) for m in range(3))
    g, u = Wg @ h, Wu @ h
    ref = Wd @ (g / (1.0 + np.exp(-g)) * u)
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)
    # gate and up are not interchangeable: silu(u)*g differs
    swapped = Wd @ (u / (1.0 + np.exp(-u)) * g)
    assert np.max(np.abs(swapped - y)) > 1e-3


def test_expert_constant_weights_closed_form():
    H, F = 128, 64
    ex = {"codes": [], "scale": [], "bias": []}
    consts = [(5, 0x3C00, 0xBC00), (3, 0x3C80, 0x0000), (7, 0x3B80, 0xBB00)]  # (q, s, b)
    for m, (q, sbits, bbits) in enumerate(consts):
        rows, cols = (F, H) if m < 2 else (H, F)
        ex["codes"].append(np.full((rows, cols), q, np.uint8))
        ex["scale"].append(np.full((rows, cols // 64), sbits, np.uint16))
        ex["bias"].append(np.full((rows, cols // 64), bbits, np.uint16))
    c = [q * _bf16(f"{s:04X}") + _bf16(f"{b:04X}") for q, s, b in consts]
    h = np.random.default_rng(2).standard_normal(H)
    S = h.sum()
    g, u = c[0] * S, c[1] * S
    a = g / (1 + np.exp(-g)) * u
    expect = np.full(H, c[2] * F * a)
    np.testing.assert_allclose(oracle.expert(ex, h), expect, rtol=1e-12)


# --------------------------------------------------------------------------- #
# whole layer: combine, sigmoid gate, residual
# --------------------------------------------------------------------------- #
def _tiny_layer(seed=0):
    w = syn.WORKLOADS["tiny"]
    d = w.dims
    dense = syn.layer_dense(seed, 0, d)
    experts = [syn.expert_canonical(seed, 0, e, d) for e in range(d.n_experts + 1)]
    x = syn.tokens(seed, 4, d.hidden)
    return d, dense, experts, x


def test_layer_c_and_orchestrated_agree_bitwise():
    d, dense, experts, x = _tiny_layer()
    for t in range(4):
        a = oracle.layer_all(d, x[t], dense, experts)
        b = oracle.layer(d, x[t], dense, lambda e: experts[e])
        assert list(a["idx"]) == list(b["idx"])
        assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["w"], b["w"])
        # only the selected experts and the shared expert are needed
        sparse = [experts[e] if (e in a["idx"] or e == d.n_experts) else None for e in range(d.n_experts + 1)]
        assert np.array_equal(oracle.layer_all(d, x[t], dense, sparse)["out"], a["out"])


def test_layer_zero_shared_gate_gives_half():
    d, dense, experts, x = _tiny_layer()
    dense = dict(dense, shared_gate=np.zeros(d.hidden, np.uint16))
    r = oracle.layer_all(d, x[0], dense, experts)
    assert r["gs"] == 0.0
    h = oracle.rmsnorm(x[0], dense["norm_weight"], d.rms_eps)
    expect = x[0].astype(np.float64)
    for k in range(d.top_k):
        expect = expect + r["w"][k] * oracle.expert(experts[r["idx"][k]], h)
    expect = expect + 0.5 * oracle.expert(experts[d.n_experts], h)
    np.testing.assert_allclose(r["out"], expect, rtol=1e-13, atol=1e-13)


def test_layer_zero_down_gives_residual_exactly():
    d, dense, experts, x = _tiny_layer()
    z = []
    for ex in experts:
        ex = {k: list(v) for k, v in ex.items()}
        ex["codes"][2] = np.zeros_like(ex["codes"][2])
        ex["bias"][2] = np.zeros_like(ex["bias"][2])
        z.append(ex)
    r = oracle.layer_all(d, x[1], dense, z)
    assert np.array_equal(r["out"], x[1].astype(np.float64))


def test_layer_doubling_down_doubles_update():
    d, dense, experts, x = _tiny_layer()
    two = []
    for ex in experts:
        ex = {k: list(v) for k, v in ex.items()}
        for key in ("scale", "bias"):
            f = syn.bf16_bits_to_f32(ex[key][2]) * np.float32(2.0)
            ex[key][2] = syn.f32_to_bf16_bits(f)
        two.append(ex)
    r1 = oracle.layer_all(d, x[2], dense, experts)
    r2 = oracle.layer_all(d, x[2], dense, two)
    x64 = x[2].astype(np.float64)
    np.testing.assert_allclose(r2["out"] - x64, 2.0 * (r1["out"] - x64), rtol=1e-12, atol=1e-12)


def test_layer_expert_permutation_invariance():
    d, dense, experts, x = _tiny_layer()
    E = d.n_experts
    perm = np.random.default_rng(6).permutation(E)  # new expert i is old expert perm[i]
    dense_p = dict(dense, router_weight=dense["router_weight"][perm])
    experts_p = [experts[perm[i]] for i in range(E)] + [experts[E]]
    inv = np.argsort(perm)
    for t in range(4):
        a = oracle.layer_all(d, x[t], dense, experts)
        b = oracle.layer_all(d, x[t], dense_p, experts_p)
        assert list(inv[a["idx"]]) == list(b["idx"])
        np.testing.assert_allclose(b["out"], a["out"], rtol=1e-14, atol=1e-14)


def test_layer_update_is_linear_in_weights_sum():
    """The routed weights sum to one, so giving every routed expert the same
    output y makes the routed part equal y itself."""
    d, dense, experts, x = _tiny_layer()
    same = [experts[0]] * d.n_experts + [experts[d.n_experts]]
    r = oracle.layer_all(d, x[3], dense, same)
    h = oracle.rmsnorm(x[3], dense["norm_weight"], d.rms_eps)
    y0 = oracle.expert(experts[0], h)
    yS = oracle.expert(experts[d.n_experts], h)
    expect = x[3].astype(np.float64) + y0 + oracle.sigmoid(r["gs"]) * yS
    np.testing.assert_allclose(r["out"], expect, rtol=1e-12, atol=1e-11)


def test_sigmoid_values():
    assert oracle.sigmoid(0.0) == 0.5
    assert abs(oracle.sigmoid(np.log(3.0)) - 0.75) < 1e-15
    assert abs(oracle.sigmoid(-np.log(3.0)) - 0.25) < 1e-15


def test_layer_forced_equals_layer_on_its_own_selection_and_renormalises():
    """With the oracle's own selection, the forced layer is the layer; with
    another selection its weights are that selection's renormalised softmax
    (they sum to 1 and follow the logits' order) and its output is the same
    combine with those experts."""
    d = syn.WORKLOADS["tiny"].dims
    dense = syn.layer_dense(0, 0, d)
    experts = [syn.expert_canonical(0, 0, e, d) for e in range(d.n_experts + 1)]
    x = syn.tokens(0, 2, d.hidden)
    for t in range(2):
        a = oracle.layer(d, x[t], dense, lambda e: experts[e])
        b = oracle.layer_forced(d, x[t], dense, lambda e: experts[e], a["idx"])
        np.testing.assert_allclose(b["out"], a["out"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(b["w"], a["w"], rtol=0, atol=1e-15)
        other = [int(a["idx"][0]), [e for e in range(d.n_experts) if e not in a["idx"]][0]]
        c = oracle.layer_forced(d, x[t], dense, lambda e: experts[e], other)
        assert abs(float(np.sum(c["w"])) - 1.0) < 1e-15
        z = c["z"][other]
        assert (c["w"][0] > c["w"][1]) == (z[0] > z[1])
        ref = np.asarray(x[t], np.float64) + sum(c["w"][k] * oracle.expert(experts[other[k]], c["h"])
                                                 for k in range(2)) + \
            oracle.sigmoid(c["gs"]) * oracle.expert(experts[d.n_experts], c["h"])
        np.testing.assert_allclose(c["out"], ref, rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.layer_forced(d, x[0], dense, lambda e: experts[e], [1, 1])
