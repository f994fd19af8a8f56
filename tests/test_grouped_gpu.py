"""GPU tests of the batched (grouped-by-expert) path's work distribution.

The streaming kernels run a persistent grid whose blocks claim runs of work
from counters in the workspace's control block; the last block of each group
resets its counters.  These tests check that every output row is computed in
every call (a workspace filled with NaN bytes between calls), that the counters
are zero after each call and across repeated or re-run stages, and that a
token's result does not depend on the batch it is in (up to the largest batch
the grouped path takes), with sampled tokens against the fp64 oracle.
"""
import numpy as np
import pytest

import synthetic as syn

from _parity import check_token, dense_layer, log, oracle_layer_canonical, oracle_layer_generated, run_layer

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CTRL_BYTES = 8192  # the control block: the first 8 KiB of a workspace (include/moe.h)


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_dequant_expert_router_amd as m
    return m


def _layer(dims, seed, layer):
    from bit_dequant_expert_router_amd.weights import layer_generated
    return layer_generated(dims, dense_layer(seed, layer, dims), seed, layer)


def _call(moe, dims, lw, x, ws, poison=True):
    T = x.shape[0]
    if poison:
        ws[CTRL_BYTES:].fill_(0xFF)  # NaN in every float buffer, -1 in every int one
    xt = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    yt = torch.empty_like(xt)
    ridx = torch.empty((T, dims.top_k), dtype=torch.int32, device="cuda")
    rw = torch.empty((T, dims.top_k), dtype=torch.float32, device="cuda")
    moe.moe_layer_forward(dims, lw.descriptor(), xt, yt, T, ridx, rw, ws)
    torch.cuda.synchronize()
    return yt.cpu().numpy(), ridx.cpu().numpy(), rw.cpu().numpy()


def _ctrl_zero(ws):
    return bool(torch.count_nonzero(ws[:CTRL_BYTES]).item() == 0)


@pytest.mark.parametrize("name,T", [("tiny", 50), ("batch32", 32)])
def test_reused_poisoned_workspace(moe, name, T):
    """One workspace, three calls (inputs A, B, A), NaN bytes written over it
    before each: every call equals a call on a fresh workspace, bit for bit,
    and leaves the control block at zero."""
    w = syn.WORKLOADS[name]
    dims = w.dims
    log(f"{name}: reused poisoned workspace, {T} tokens")
    lw = _layer(dims, w.seed, 1)
    xa = syn.tokens(11, T, dims.hidden)
    xb = syn.tokens(12, T, dims.hidden)
    ref_a, _, _ = run_layer(dims, lw, xa)
    ref_b, _, _ = run_layer(dims, lw, xb)
    ws = torch.empty(moe.moe_workspace_bytes(dims, T), dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws)
    for x, ref in ((xa, ref_a), (xb, ref_b), (xa, ref_a)):
        out, _, _ = _call(moe, dims, lw, x, ws)
        assert np.array_equal(out, ref)
        assert _ctrl_zero(ws)


def test_stages_rerun(moe):
    """Stages of the grouped path enqueued again (gate/up and down twice, then
    the rest) give the one-call result; the counters stay at zero."""
    w = syn.WORKLOADS["batch32"]
    dims = w.dims
    T = 10
    lw = _layer(dims, w.seed, 2)
    x = syn.tokens(13, T, dims.hidden)
    ref, _, _ = run_layer(dims, lw, x)
    ws = torch.empty(moe.moe_workspace_bytes(dims, T), dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws)
    xt = torch.from_numpy(x).cuda()
    yt = torch.empty_like(xt)
    assert moe.moe_forward_stage_count(dims, T) == 7
    for stage in (0, 1, 2, 3, 3, 4, 5, 5, 6, 3, 4, 5, 6):
        moe.moe_layer_forward_stage(dims, lw.descriptor(), xt, yt, T, None, None, ws, None, stage)
    torch.cuda.synchronize()
    assert np.array_equal(yt.cpu().numpy(), ref)
    assert _ctrl_zero(ws)


def test_batch_independence_up_to_largest_batch(moe):
    """384 tokens with top-10 (3840 assignments, near the grouped path's limit
    of 4096): each token's output equals the one it gets in 32-token batches,
    bit for bit; sampled tokens match the oracle.  (Batches of 32 tokens or
    more run the shared expert on the matrix cores, smaller ones in limb
    passes: equal within rounding, not bit for bit.)"""
    w = syn.WORKLOADS["batch32"]
    dims = w.dims
    T = 384
    log(f"batch of {T}: {dims}")
    lw = _layer(dims, w.seed, 0)
    x = syn.tokens(14, T, dims.hidden)
    ws = torch.empty(moe.moe_workspace_bytes(dims, T), dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws)
    big, idx, wt = _call(moe, dims, lw, x, ws)
    assert _ctrl_zero(ws)
    for t0 in range(0, T, 32):
        part, _, _ = run_layer(dims, lw, x[t0:t0 + 32])
        assert np.array_equal(big[t0:t0 + 32], part), f"tokens {t0}..{t0 + len(part) - 1}"
    for t in (0, 31, 32, 200, 383):
        ref = oracle_layer_generated(dims, w.seed, 0, x[t])
        check_token(big[t], idx[t], wt[t], ref, dims.top_k, f"batch {T} token {t}")


def test_many_experts_grouped(moe):
    """1024 experts (four logits per lane in each routing wave): 25 tokens
    (100 assignments) on the grouped path, and tokens 0-1 on the per-token
    path."""
    from bit_dequant_expert_router_amd.weights import layer_from_canonical
    import oracle
    dims = syn.Dims(256, 128, 1024, 8, 4)
    dense = syn.layer_dense(5, 0, dims)
    experts = [syn.expert_canonical(5, 0, e, dims) for e in range(dims.n_experts + 1)]
    lw = layer_from_canonical(dims, dense, experts)
    x = syn.tokens(15, 25, dims.hidden)
    assert moe.moe_forward_stage_count(dims, 25) == 7
    out, idx, wt = run_layer(dims, lw, x)
    refs = [oracle_layer_canonical(dims, x[t], dense, experts) for t in range(x.shape[0])]
    for t in range(x.shape[0]):
        check_token(out[t], idx[t], wt[t], refs[t], dims.top_k, f"1024 experts token {t}")
    out, idx, wt = run_layer(dims, lw, x[:2])
    for t in range(2):
        check_token(out[t], idx[t], wt[t], refs[t], dims.top_k, f"1024 experts per-token path, token {t}")


def test_ragged_token_tile_full_size(moe):
    """45 tokens at the batched shape: the shared expert's second 32-token
    matrix-core tile holds 13 tokens; sampled tokens of both tiles against the
    oracle."""
    w = syn.WORKLOADS["batch32"]
    dims = w.dims
    T = 45
    log(f"batch of {T}: {dims}")
    lw = _layer(dims, w.seed, 3)
    x = syn.tokens(16, T, dims.hidden)
    out, idx, wt = run_layer(dims, lw, x)
    for t in (0, 31, 32, 40, 44):
        ref = oracle_layer_generated(dims, w.seed, 3, x[t])
        check_token(out[t], idx[t], wt[t], ref, dims.top_k, f"batch {T} token {t}")


def test_batch_past_grouping_limit(moe):
    """2049 tiny tokens with top-2 (4098 assignments, past the grouped path's
    4096) run the per-token kernels, one row of blocks per token; sampled
    tokens against the oracle, and the first 2048 tokens as one grouped call
    give the same routing."""
    import oracle
    w = syn.WORKLOADS["tiny"]
    dims = w.dims
    T = 2049
    assert moe.moe_forward_stage_count(dims, T) == 3
    assert moe.moe_forward_stage_count(dims, T - 1) == 7
    from bit_dequant_expert_router_amd.weights import layer_from_canonical
    dense = syn.layer_dense(w.seed, 0, dims)
    experts = [syn.expert_canonical(w.seed, 0, e, dims) for e in range(dims.n_experts + 1)]
    lw = layer_from_canonical(dims, dense, experts)
    x = syn.tokens(17, T, dims.hidden)
    out, idx, wt = run_layer(dims, lw, x)
    for t in (0, 1, 1000, 2047, 2048):
        check_token(out[t], idx[t], wt[t], oracle_layer_canonical(dims, x[t], dense, experts), dims.top_k,
                    f"token {t} of {T}")
    og, ig, wg = run_layer(dims, lw, x[:T - 1])
    assert np.array_equal(ig, idx[:T - 1])
    np.testing.assert_allclose(og, out[:T - 1], rtol=1e-5, atol=1e-4)
