"""moe_layer_forward_noalloc (the library's own fixed workspace) against
moe_layer_forward: bit-identical outputs and routing on two calls in a row,
the second with a smaller batch, on the per-token and the grouped paths."""
import numpy as np
import pytest

import synthetic as syn

from _parity import canon_expert, dense_layer, log, run_layer

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_dequant_expert_router_amd as m
    return m


def _noalloc(moe, dims, lw, x):
    T = x.shape[0]
    xt = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    yt = torch.full_like(xt, float("nan"))
    ridx = torch.full((T, dims.top_k), -1, dtype=torch.int32, device="cuda")
    rw = torch.full((T, dims.top_k), -1.0, dtype=torch.float32, device="cuda")
    moe.moe_layer_forward_noalloc(dims, lw.descriptor(), xt, yt, T, ridx, rw)
    torch.cuda.synchronize()
    return yt.cpu().numpy(), ridx.cpu().numpy(), rw.cpu().numpy()


def _same(a, b, what):
    for u, v, name in zip(a, b, ("y", "route_idx", "route_w")):
        assert np.array_equal(u, v), f"{what}: {name} differs"


def _canonical_layer(dims, seed=0, layer=0):
    from bit_dequant_expert_router_amd.weights import layer_from_canonical
    dense = dense_layer(seed, layer, dims)
    experts = [canon_expert(seed, layer, e, dims) for e in range(dims.n_experts + 1)]
    return layer_from_canonical(dims, dense, experts)


@pytest.mark.parametrize("name,first,second", [
    ("tiny", 50, 3),     # grouped (100 assignments), then per-token
    ("layer4", 6, 1),    # per-token, six tokens then the single-token call
    ("batch32", 32, 2),  # grouped 32 x top-10 (13.5 MB of the 16 MiB), then per-token
])
def test_noalloc_equals_workspace_call(moe, name, first, second):
    from bit_dequant_expert_router_amd.weights import layer_generated
    w = syn.WORKLOADS[name]
    dims = w.dims
    if name == "tiny":
        lw = _canonical_layer(dims)
    else:
        lw = layer_generated(dims, dense_layer(w.seed, 0, dims), w.seed, 0)
    x = syn.tokens(w.seed + 11, first, dims.hidden)
    for T in (first, second):
        log(f"no-alloc {name}: {T} tokens ({moe.moe_workspace_bytes(dims, T)} workspace bytes)")
        assert moe.moe_workspace_bytes(dims, T) <= moe.MOE_NOALLOC_SCRATCH_BYTES
        ref = run_layer(dims, lw, x[:T])
        got = _noalloc(moe, dims, lw, x[:T])
        _same(got, ref, f"{name} {T} tokens")

