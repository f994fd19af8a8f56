"""GPU: tiered expert residency through the C ABI.

The experts live in pinned host memory; the device holds an LRU cache of
n_slots expert slots.  Every output, routing index and routing weight must
equal, bit for bit, those of moe_layer_forward's per-token kernels with every
expert resident (so the oracle parity of that path carries over).  Every layer
of every call is also checked against the oracle directly: up to four tokens
of the first call, and the first token of each later call, whose experts come
from slots that were filled, hit or refilled by the calls before.  The cache's lookups,
hits, misses and copied bytes, and the set of experts it holds at the end,
must equal the LRU oracle's on the same access sequence.
"""
import numpy as np
import pytest

import synthetic as syn
from oracle.lru import layer_accesses, lru_run

from _parity import check_token, log, oracle_layer_generated

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_dequant_expert_router_amd as m
    return m


def _layers(dims, n_layers, seed, pinned=True):
    from bit_dequant_expert_router_amd.weights import layer_generated
    lws = [layer_generated(dims, syn.layer_dense(seed, l, dims), seed, l) for l in range(n_layers)]
    hosts = []
    for lw in lws:
        n = lw.experts.numel()
        raw = torch.empty(n + 256, dtype=torch.uint8, pin_memory=pinned)
        off = (-raw.data_ptr()) % 256  # the store must be 256-byte aligned
        h = raw[off:off + n]
        h.copy_(lw.experts)
        hosts.append(h)
    torch.cuda.synchronize()
    return lws, hosts


def _same(a, b):
    """Bitwise equality, NaN positions included."""
    return torch.equal(torch.isnan(a), torch.isnan(b)) and torch.equal(torch.nan_to_num(a, nan=7.0),
                                                                       torch.nan_to_num(b, nan=7.0))


def _run(moe, dims, n_layers, n_slots, max_tokens, calls, seed=0, nan_token=None, pinned_store=True):
    K, E = dims.top_k, dims.n_experts
    log(f"tier: {dims}, {n_layers} layers, {n_slots} slots, calls {calls}")
    lws, hosts = _layers(dims, n_layers, seed, pinned_store)
    eb = moe.moe_expert_bytes(dims)
    state = torch.zeros(moe.moe_tier_state_bytes(dims, n_layers, n_slots, max_tokens), dtype=torch.uint8,
                        pin_memory=True)
    dev = torch.empty(moe.moe_tier_device_bytes(dims, n_slots, max_tokens), dtype=torch.uint8, device="cuda")
    moe.moe_tier_init(dims, n_layers, n_slots, max_tokens, state, dev)
    ws = torch.empty(moe.moe_workspace_bytes(dims, max_tokens), dtype=torch.uint8, device="cuda")
    ws_ref = torch.empty_like(ws)
    moe.moe_workspace_init(ws)
    moe.moe_workspace_init(ws_ref)
    x_all = syn.tokens(seed + 1, sum(calls), dims.hidden)
    if nan_token is not None:
        x_all[nan_token, 17] = np.nan
    accesses, off = [], 0
    for c, T in enumerate(calls):
        xt = torch.from_numpy(x_all[off:off + T]).cuda()
        xr = xt.clone()
        off += T
        for l in range(n_layers):
            lw = lws[l]
            tier_layer = moe.make_layer(lw.norm_weight, lw.router_weight, lw.shared_gate, hosts[l], lw.shared)
            yt, yr = torch.empty_like(xt), torch.empty_like(xr)
            it = torch.full((T, K), -1, dtype=torch.int32, device="cuda")
            ir = torch.full_like(it, -2)
            wt = torch.full((T, K), -1.0, dtype=torch.float32, device="cuda")
            wr = torch.full_like(wt, -2.0)
            xin = xt.cpu().numpy()
            moe.moe_tier_layer_forward(state, l, tier_layer, xt, yt, T, it, wt, ws)
            moe.moe_layer_forward(dims, lw.descriptor(), xr, yr, T, ir, wr, ws_ref)
            torch.cuda.synchronize()
            assert torch.equal(it, ir), (c, l)
            assert _same(wt, wr), (c, l)
            assert _same(yt, yr), (c, l)
            # against the oracle, fed the layer's input as the GPU saw it
            # (teacher forcing): up to four tokens of the first call, the first
            # token of every later one
            yh, ih, wh = yt.cpu().numpy(), it.cpu().numpy(), wt.cpu().numpy()
            for t in range(min(T, 4) if c == 0 else 1):
                if not np.all(np.isfinite(xin[t])):
                    continue
                ref = oracle_layer_generated(dims, seed, l, xin[t])
                check_token(yh[t], ih[t], wh[t], ref, K, f"tier call {c} layer {l} token {t}", unit_scale=l > 0)
            accesses += layer_accesses(l, ir.cpu().numpy(), E)
            xt, xr = yt, yr
    hits, cache = lru_run(accesses, n_slots)
    st = moe.moe_tier_get_stats(state)
    misses = hits.count(False)
    log(f"tier: {len(accesses)} lookups, {misses} misses")
    assert st.calls == len(calls) * n_layers
    assert (st.lookups, st.hits, st.misses) == (len(accesses), len(accesses) - misses, misses)
    assert st.bytes_copied == misses * eb
    slots = {}
    for l in range(n_layers):
        for e in range(E):
            s = moe.moe_tier_lookup(state, l, e)
            if s >= 0:
                assert 0 <= s < n_slots
                slots[l * E + e] = s
    assert set(slots) == set(cache)
    assert len(set(slots.values())) == len(slots)  # one expert per slot
    return st


def test_tiny_three_layers(moe):
    dims = syn.WORKLOADS["tiny"].dims  # 8 experts, top-2
    st = _run(moe, dims, 3, 5, 2, [1, 2, 1, 1, 2, 2, 1, 2, 1, 1, 2, 1])
    assert 0 < st.hits < st.lookups


def test_tiny_2bit(moe):
    dims = syn.Dims(256, 128, 8, 2, 2)
    _run(moe, dims, 2, 4, 2, [2, 1, 2, 2, 1, 1, 2])


def test_cache_holds_everything(moe):
    # every expert of both layers fits: only cold misses, then hits only
    dims = syn.WORKLOADS["tiny"].dims
    st = _run(moe, dims, 2, 16, 3, [3] * 10)
    assert st.misses <= 16


def test_many_experts_and_four_tokens(moe):
    # more than 512 experts (the routing's wide variant) and calls of four
    # tokens (the router's multi-token kernel)
    dims = syn.Dims(256, 128, 1024, 4, 4)
    _run(moe, dims, 1, 16, 4, [4, 1, 3, 4, 2])


def test_full_size_layers(moe):
    # two 4096/1024 layers of 512 experts (7.1 GB of pinned host memory)
    dims = syn.WORKLOADS["layer4"].dims
    _run(moe, dims, 2, 20, 4, [1, 4, 2, 1, 3, 1])


def test_sixty_four_assignments(moe):
    # the most a call carries (64 slots in the kernel arguments): 16 tokens x
    # top-4, and 4 tokens x top-16
    _run(moe, syn.Dims(256, 128, 64, 4, 4), 1, 80, 16, [16, 5, 16, 1, 16])
    _run(moe, syn.Dims(256, 128, 64, 16, 4), 2, 64, 4, [4, 1, 4, 3])


def test_nan_token(moe):
    # a NaN in one token's x: its routing still selects valid experts, its
    # outputs are NaN, the other tokens' are finite, all as on the resident path
    dims = syn.WORKLOADS["tiny"].dims
    _run(moe, dims, 2, 6, 3, [3, 1, 3], nan_token=1)


def test_state_not_pinned_is_rejected(moe):
    # the routing kernel writes into the state, so pageable memory is refused
    # before anything is launched
    dims = syn.WORKLOADS["tiny"].dims
    lws, hosts = _layers(dims, 1, 0)
    state = torch.zeros(moe.moe_tier_state_bytes(dims, 1, 4, 1), dtype=torch.uint8)  # pageable
    dev = torch.empty(moe.moe_tier_device_bytes(dims, 4, 1), dtype=torch.uint8, device="cuda")
    moe.moe_tier_init(dims, 1, 4, 1, state, dev)
    ws = torch.empty(moe.moe_workspace_bytes(dims, 1), dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws)
    x = torch.from_numpy(syn.tokens(0, 1, dims.hidden)).cuda()
    y = torch.empty_like(x)
    lw = lws[0]
    layer = moe.make_layer(lw.norm_weight, lw.router_weight, lw.shared_gate, hosts[0], lw.shared)
    with pytest.raises(moe.MoeError) as err:
        moe.moe_tier_layer_forward(state, 0, layer, x, y, 1, None, None, ws)
    assert err.value.status == moe.MOE_ERR_INVALID_ARG
    assert moe.moe_tier_get_stats(state).calls == 0
    torch.cuda.synchronize()


def test_pageable_store(moe):
    # a host store that is not pinned: the misses are copied by DMA instead of
    # the copy kernel, with the same results
    dims = syn.WORKLOADS["tiny"].dims
    st = _run(moe, dims, 2, 5, 2, [2, 1, 2, 2, 1], pinned_store=False)
    assert st.misses > 0


def test_stack_equals_resident_stack(moe):
    # three chained layers through the cache in one call == moe_stack_forward
    # with every expert resident, bit for bit, including the routing records
    dims = syn.WORKLOADS["tiny"].dims
    L, T, K = 3, 2, dims.top_k
    lws, hosts = _layers(dims, L, 0)
    state = torch.zeros(moe.moe_tier_state_bytes(dims, L, 6, T), dtype=torch.uint8, pin_memory=True)
    dev = torch.empty(moe.moe_tier_device_bytes(dims, 6, T), dtype=torch.uint8, device="cuda")
    moe.moe_tier_init(dims, L, 6, T, state, dev)
    ws = torch.empty(moe.moe_workspace_bytes(dims, T), dtype=torch.uint8, device="cuda")
    ws_ref = torch.empty_like(ws)
    moe.moe_workspace_init(ws)
    moe.moe_workspace_init(ws_ref)
    tier_layers = [moe.make_layer(lw.norm_weight, lw.router_weight, lw.shared_gate, h, lw.shared)
                   for lw, h in zip(lws, hosts)]
    for c in range(4):
        x = torch.from_numpy(syn.tokens(40 + c, T, dims.hidden)).cuda()
        yt, yr = torch.empty_like(x), torch.empty_like(x)
        it = torch.full((L, T, K), -1, dtype=torch.int32, device="cuda")
        ir = torch.full_like(it, -2)
        wt = torch.full((L, T, K), -1.0, dtype=torch.float32, device="cuda")
        wr = torch.full_like(wt, -2.0)
        moe.moe_tier_stack_forward(state, tier_layers, x, yt, T, it, wt, ws)
        moe.moe_stack_forward(dims, [lw.descriptor() for lw in lws], x, yr, T, ir, wr, ws_ref)
        torch.cuda.synchronize()
        assert torch.equal(it, ir) and _same(wt, wr) and _same(yt, yr), c
    assert moe.moe_tier_get_stats(state).calls == 4 * L
