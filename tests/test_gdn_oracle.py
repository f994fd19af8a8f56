"""Pins of the GatedDeltaNet state-update oracle (CPU only).

Each pin fixes the oracle against something other than itself: hand-worked
steps (tests/golden/gdn_worked.txt), the matrix form of the recurrence, the
delta rule's exact recall at a unit key, decay alone, brute-force element
loops, and the state as an associative memory of orthonormal keys.  A dropped
decay, a sign error in v - u, a transposed outer product, the recall taken on
the undecayed state or the output taken from the old state each fail one."""
import os

import numpy as np
import pytest

from oracle import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _cases():
    cases, cur = {}, None
    with open(os.path.join(ROOT, "tests", "golden", "gdn_worked.txt")) as f:
        for ln in f:
            ln = ln.strip()
            if not ln or ln.startswith("#"):
                continue
            key, *vals = ln.split()
            if key == "case":
                cur = cases.setdefault(vals[0], {})
            else:
                cur[key] = np.array([float(v) for v in vals])
    for c in cases.values():
        d = int(c["d"][0])
        c["S0"] = c["S0"].reshape(d, d)
        c["S1"] = c["S1"].reshape(d, d)
    return cases


@pytest.mark.parametrize("name,tol", [("A", 0.0), ("B", 1e-12), ("C", 0.0)])
def test_hand_worked_steps(name, tol):
    c = _cases()[name]
    S1, o = gdn.gdn_step(c["S0"], c["q"], c["k"], c["v"], c["alpha"][0], c["beta"][0])
    assert np.max(np.abs(S1 - c["S1"])) <= tol
    assert np.max(np.abs(o - c["o"])) <= tol


def _rand(rng, d_v, d_k):
    S = rng.normal(0, 1, (d_v, d_k))
    q, k = rng.normal(0, 1, d_k), rng.normal(0, 1, d_k)
    v = rng.normal(0, 1, d_v)
    return S, q, k, v


@pytest.mark.parametrize("d_v,d_k", [(3, 3), (5, 7), (128, 128)])
def test_matrix_form(d_v, d_k):
    """S' = alpha S (I - beta k k^T) + beta v k^T, o = S' q (the recurrence as
    its authors write it, as one dense product)."""
    rng = np.random.default_rng(1)
    S, q, k, v = _rand(rng, d_v, d_k)
    alpha, beta = 0.8125, 0.375
    S1, o = gdn.gdn_step(S, q, k, v, alpha, beta)
    ref = alpha * S @ (np.eye(d_k) - beta * np.outer(k, k)) + beta * np.outer(v, k)
    np.testing.assert_allclose(S1, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))
    np.testing.assert_allclose(o, ref @ q, rtol=0, atol=1e-11 * max(1.0, np.abs(ref @ q).max()))


def test_delta_rule_recalls_v_at_a_unit_key():
    rng = np.random.default_rng(2)
    for d in (2, 16, 128):
        S, q, k, v = _rand(rng, d, d)
        k /= np.linalg.norm(k)
        S1, _ = gdn.gdn_step(S, q, k, v, 1.0, 1.0)
        np.testing.assert_allclose(S1 @ k, v, rtol=0, atol=1e-12 * max(1.0, np.abs(S).max() * d))


def test_beta_zero_is_decay_alone():
    rng = np.random.default_rng(3)
    S, q, k, v = _rand(rng, 6, 4)
    S1, o = gdn.gdn_step(S, q, k, v, 0.5, 0.0)
    assert np.array_equal(S1, 0.5 * S) and np.allclose(o, 0.5 * S @ q, rtol=0, atol=1e-14)


def test_orthonormal_keys_store_independent_values():
    """With alpha = beta = 1, writing v1 at k1 and then v2 at k2 (orthonormal)
    leaves S k1 = v1 and S k2 = v2, whatever the state held."""
    rng = np.random.default_rng(4)
    d = 8
    Q, _ = np.linalg.qr(rng.normal(0, 1, (d, d)))
    k1, k2 = Q[:, 0], Q[:, 1]
    S = rng.normal(0, 1, (d, d))
    v1, v2 = rng.normal(0, 1, d), rng.normal(0, 1, d)
    S, _ = gdn.gdn_step(S, k1, k1, v1, 1.0, 1.0)
    S, _ = gdn.gdn_step(S, k2, k2, v2, 1.0, 1.0)
    np.testing.assert_allclose(S @ k1, v1, atol=1e-12)
    np.testing.assert_allclose(S @ k2, v2, atol=1e-12)


def test_brute_force_element_loops():
    """Every element written out with Python loops, on small random states."""
    rng = np.random.default_rng(5)
    for d_v, d_k in ((1, 1), (2, 3), (4, 4)):
        S, q, k, v = _rand(rng, d_v, d_k)
        alpha, beta = float(rng.uniform(0.5, 1)), float(rng.uniform(0, 1))
        ref = [[0.0] * d_k for _ in range(d_v)]
        for i in range(d_v):
            recall = sum(alpha * S[i][j] * k[j] for j in range(d_k))
            for j in range(d_k):
                ref[i][j] = alpha * S[i][j] + beta * (v[i] - recall) * k[j]
        out = [sum(ref[i][j] * q[j] for j in range(d_k)) for i in range(d_v)]
        S1, o = gdn.gdn_step(S, q, k, v, alpha, beta)
        np.testing.assert_allclose(S1, np.array(ref), rtol=0, atol=1e-13)
        np.testing.assert_allclose(o, np.array(out), rtol=0, atol=1e-13)


def test_layer_is_tokens_in_order_and_keeps_the_input_state():
    rng = np.random.default_rng(6)
    T, Hh, d = 3, 2, 4
    S0 = rng.normal(0, 1, (Hh, d, d))
    q, k, v = (rng.normal(0, 1, (T, Hh, d)) for _ in range(3))
    alpha, beta = rng.uniform(0.5, 1, (T, Hh)), rng.uniform(0, 1, (T, Hh))
    keep = S0.copy()
    S, out = gdn.gdn_layer(S0, q, k, v, alpha, beta)
    assert np.array_equal(S0, keep)
    for h in range(Hh):
        s = S0[h]
        for t in range(T):
            s, o = gdn.gdn_step(s, q[t, h], k[t, h], v[t, h], alpha[t, h], beta[t, h])
            assert np.array_equal(o, out[t, h])
        assert np.array_equal(s, S[h])
