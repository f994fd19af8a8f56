"""GPU parity of the GatedDeltaNet state update (moe_gdn_update) against the
fp64 oracle (oracle/gdn.py): the hand-worked steps of tests/golden/gdn_worked.txt
embedded in a 128 x 128 state (exact), and the pages' 64 heads x 128 x 128 on
synthetic inputs for 1 and 8 tokens (rel-L2 <= 1e-4, max-abs <= 1e-3, the
layer's output tolerance)."""
import os

import numpy as np
import pytest

import synthetic as syn
from oracle import gdn

from _parity import log, rel_l2

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
D = 128


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_dequant_expert_router_amd as m
    return m


def _run(moe, state, q, k, v, alpha, beta):
    T, Hh = alpha.shape
    dev = [torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda() for a in (state, q, k, v, alpha, beta)]
    out = torch.full((T, Hh, D), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_gdn_update(Hh, D, D, T, dev[0], *dev[1:], out)
    torch.cuda.synchronize()
    return dev[0].cpu().numpy(), out.cpu().numpy()


def _golden():
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
                cur[key] = np.array([float(x) for x in vals])
    return cases


@pytest.mark.parametrize("name", ["A", "C"])
def test_worked_step_embedded(moe, name):
    """The hand-worked d x d step in the top-left corner of a zero 128 x 128
    state (q, k, v zero beyond d): the corner follows the worked values exactly
    (all dyadic), the rest of the state and the outputs stay zero."""
    c = _golden()[name]
    d = int(c["d"][0])
    state = np.zeros((2, D, D), np.float32)
    state[1, :d, :d] = c["S0"].reshape(d, d)  # head 1; head 0 stays zero
    q, k, v = (np.zeros((1, 2, D), np.float32) for _ in range(3))
    q[0, 1, :d], k[0, 1, :d], v[0, 1, :d] = c["q"], c["k"], c["v"]
    alpha = np.array([[0.5, c["alpha"][0]]], np.float32)
    beta = np.array([[0.5, c["beta"][0]]], np.float32)
    S, out = _run(moe, state, q, k, v, alpha, beta)
    assert np.array_equal(S[1, :d, :d], c["S1"].reshape(d, d).astype(np.float32))
    assert np.array_equal(out[0, 1, :d], c["o"].astype(np.float32))
    S[1, :d, :d] = 0
    assert not np.any(S) and not np.any(out[0, 1, d:]) and not np.any(out[0, 0])


@pytest.mark.parametrize("T", [1, 8])
def test_full_layer(moe, T):
    """64 heads x 128 x 128 (the pages' shape) on synthetic inputs."""
    x = syn.gdn_inputs(0, 64, D, T)
    S, out = _run(moe, x["state"], x["q"], x["k"], x["v"], x["alpha"], x["beta"])
    Sr, outr = gdn.gdn_layer(x["state"], x["q"], x["k"], x["v"], x["alpha"], x["beta"])
    es, eo = rel_l2(S, Sr), rel_l2(out, outr)
    ms, mo = float(np.max(np.abs(S - Sr))), float(np.max(np.abs(out - outr)))
    log(f"gdn 64 heads, {T} tokens: state rel-L2 {es:.2e} max-abs {ms:.2e}; out rel-L2 {eo:.2e} max-abs {mo:.2e}")
    assert es <= 1e-4 and eo <= 1e-4 and ms <= 1e-3 and mo <= 1e-3


def test_tokens_in_one_call_equal_single_token_calls(moe):
    """Eight tokens in one call give the same state and outputs as eight calls
    of one token (the same fp32 operations in the same order)."""
    x = syn.gdn_inputs(1, 4, D, 8)
    S8, out8 = _run(moe, x["state"], x["q"], x["k"], x["v"], x["alpha"], x["beta"])
    S = x["state"]
    for t in range(8):
        S, o = _run(moe, S, x["q"][t:t + 1], x["k"][t:t + 1], x["v"][t:t + 1], x["alpha"][t:t + 1],
                    x["beta"][t:t + 1])
        assert np.array_equal(o[0], out8[t])
    assert np.array_equal(S, S8)


def test_beta_zero_decays_the_state(moe):
    """beta = 0: the state becomes alpha S, rounded once per entry as fp32."""
    x = syn.gdn_inputs(2, 3, D, 1)
    beta = np.zeros_like(x["beta"])
    S, out = _run(moe, x["state"], x["q"], x["k"], x["v"], x["alpha"], beta)
    ref = (x["alpha"][0][:, None, None] * x["state"]).astype(np.float32)
    assert np.array_equal(S, ref)
