"""Host-side contract of the C ABI (no GPU needed): the library loads, exports
every entry point the header declares, sizes match the closed forms, and every
invalid argument is rejected with its documented status before anything is
enqueued."""
import ctypes
import os
import re
import subprocess

import pytest

import bit_dequant_expert_router_amd as moe
import synthetic as syn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", n) for n in sorted(os.listdir(os.path.join(ROOT, "include")))
           if n.endswith(".h")]


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    assert set(moe.EXPORTED) == set(names)
    assert moe.moe_abi_version() == 1


def d(**kw):
    base = dict(hidden=4096, ffn=1024, n_experts=512, top_k=4, bits=4)
    base.update(kw)
    return moe.make_dims(**base)


def _gold(name):
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        return {ln.split()[0]: float(ln.split()[1]) for ln in f if ln.strip() and not ln.startswith("#")}


def test_expert_bytes_closed_form_and_pages():
    for H, F, bits in ((4096, 1024, 4), (4096, 1024, 2), (256, 128, 4), (1024, 4096, 4), (128, 128, 2)):
        closed = 3 * H * F * bits // 8 + 3 * (H * F // 64) * 4
        assert moe.moe_expert_bytes(d(hidden=H, ffn=F, bits=bits)) == closed
    assert moe.moe_expert_bytes(d()) == 7_077_888
    assert moe.moe_expert_bytes(d(bits=2)) == 3_932_160
    assert moe.moe_expert_bytes(syn.WORKLOADS["tiny"].dims) == 55_296
    g = _gold("page_sizes.txt")
    mib = 1 << 20
    assert moe.moe_expert_bytes(d()) == g["expert_4bit"] * mib
    assert 4 * moe.moe_expert_bytes(d()) == g["layer_k4_4bit"] * mib
    assert abs(moe.moe_expert_bytes(d()) / 1e6 - g["blit_4x"]) < 0.1


@pytest.mark.parametrize("kw,status", [
    (dict(bits=3), moe.MOE_ERR_UNSUPPORTED),
    (dict(bits=8), moe.MOE_ERR_UNSUPPORTED),
    (dict(bits=0), moe.MOE_ERR_INVALID_ARG),
    (dict(bits=9), moe.MOE_ERR_INVALID_ARG),
    (dict(group_size=32), moe.MOE_ERR_UNSUPPORTED),
    (dict(group_size=0), moe.MOE_ERR_INVALID_ARG),
    (dict(hidden=4000), moe.MOE_ERR_INVALID_ARG),
    (dict(ffn=1000), moe.MOE_ERR_INVALID_ARG),
    (dict(hidden=3072), moe.MOE_ERR_UNSUPPORTED),
    (dict(hidden=8192), moe.MOE_ERR_UNSUPPORTED),
    (dict(hidden=64), moe.MOE_ERR_UNSUPPORTED),
    (dict(top_k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(top_k=513), moe.MOE_ERR_INVALID_ARG),
    (dict(top_k=17), moe.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=2048), moe.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=0), moe.MOE_ERR_INVALID_ARG),
    (dict(rms_eps=-1.0), moe.MOE_ERR_INVALID_ARG),
    (dict(rms_eps=float("nan")), moe.MOE_ERR_INVALID_ARG),
    (dict(rms_eps=float("inf")), moe.MOE_ERR_INVALID_ARG),
])
def test_check_dims_errors(kw, status):
    assert moe.moe_check_dims(d(**kw)) == status
    assert moe.moe_expert_bytes(d(**kw)) == 0
    assert moe.moe_workspace_bytes(d(**kw), 1) == 0


def test_valid_dims():
    for w in syn.WORKLOADS.values():
        assert moe.moe_check_dims(w.dims) == moe.MOE_OK
    assert moe.moe_check_dims(d(top_k=16, n_experts=16, hidden=128, ffn=4096, bits=2)) == moe.MOE_OK
    assert moe._lib.moe_check_dims(None) == moe.MOE_ERR_INVALID_ARG


def test_workspace_bytes_monotone():
    prev = 0
    for T in (1, 2, 3, 8, 32, 100):
        b = moe.moe_workspace_bytes(d(), T)
        assert b > prev and b % 256 == 0
        prev = b
    assert moe.moe_workspace_bytes(d(), 0) == 0


# fake, never-dereferenced device addresses: every call below must fail validation
A = 1 << 40


def _layer(**kw):
    f = dict(norm_weight=A, router_weight=A + 0x10000, shared_gate=A + 0x20000, experts=A + 0x100000,
             shared_expert=A + 0x200000)
    f.update(kw)
    return moe.moe_layer_t(*[f[k] for k in ("norm_weight", "router_weight", "shared_gate", "experts",
                                            "shared_expert")])


def _fwd(dims=None, layer=None, x=A + 0x300000, y=A + 0x400000, T=1, ridx=None, rw=None, ws=A + 0x500000,
         wsb=None):
    dims = dims or d()
    layer = layer if layer is not None else _layer()
    if wsb is None:
        wsb = moe.moe_workspace_bytes(dims, max(T, 1))
    return moe._lib.moe_layer_forward(ctypes.byref(dims), ctypes.byref(layer) if layer else None, x, y, T, ridx,
                                      rw, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dims=d(bits=3)), moe.MOE_ERR_UNSUPPORTED),
    (dict(x=None), moe.MOE_ERR_INVALID_ARG),
    (dict(y=None), moe.MOE_ERR_INVALID_ARG),
    (dict(ws=None), moe.MOE_ERR_INVALID_ARG),
    (dict(T=0), moe.MOE_ERR_INVALID_ARG),
    (dict(T=-3), moe.MOE_ERR_INVALID_ARG),
    (dict(T=70000), moe.MOE_ERR_INVALID_ARG),
    (dict(x=A + 0x300004), moe.MOE_ERR_ALIGNMENT),
    (dict(y=A + 0x400008), moe.MOE_ERR_ALIGNMENT),
    (dict(ws=A + 0x500010), moe.MOE_ERR_ALIGNMENT),
    (dict(ridx=A + 0x600002), moe.MOE_ERR_ALIGNMENT),
    (dict(wsb=1024), moe.MOE_ERR_WORKSPACE),
    (dict(y=A + 0x300000 + 4096), moe.MOE_ERR_INVALID_ARG),  # partial overlap of x and y
    (dict(layer=False), moe.MOE_ERR_INVALID_ARG),
    (dict(layer=_layer(experts=None)), moe.MOE_ERR_INVALID_ARG),
    (dict(layer=_layer(norm_weight=None)), moe.MOE_ERR_INVALID_ARG),
    (dict(layer=_layer(shared_expert=A + 0x200040)), moe.MOE_ERR_ALIGNMENT),
    (dict(layer=_layer(router_weight=A + 0x10002)), moe.MOE_ERR_ALIGNMENT),
])
def test_forward_rejects(kw, status):
    if kw.get("layer") is False:
        kw = dict(kw, layer=None)
        dims = d()
        rc = moe._lib.moe_layer_forward(ctypes.byref(dims), None, A + 0x300000, A + 0x400000, 1, None, None,
                                        A + 0x500000, moe.moe_workspace_bytes(dims, 1), None)
        assert rc == status
        return
    assert _fwd(**kw) == status


def test_noalloc_rejects_before_any_launch():
    """The no-alloc variant checks its arguments like moe_layer_forward and
    refuses a batch whose workspace exceeds its fixed array, all on the host."""
    f = moe._lib.moe_layer_forward_noalloc
    lay = _layer()
    big = d(top_k=10)
    assert moe.moe_workspace_bytes(big, 32) <= moe.MOE_NOALLOC_SCRATCH_BYTES < moe.moe_workspace_bytes(big, 64)
    assert f(ctypes.byref(big), ctypes.byref(lay), A + 0x300000, A + 0x300000, 64, None, None,
             None) == moe.MOE_ERR_WORKSPACE
    dims = d()
    assert f(ctypes.byref(dims), None, A + 0x300000, A + 0x400000, 1, None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert f(ctypes.byref(dims), ctypes.byref(lay), A + 0x300004, A + 0x400000, 1, None, None,
             None) == moe.MOE_ERR_ALIGNMENT
    assert f(ctypes.byref(dims), ctypes.byref(lay), A + 0x300000, A + 0x400000, 0, None, None,
             None) == moe.MOE_ERR_INVALID_ARG
    assert f(ctypes.byref(d(bits=3)), ctypes.byref(lay), A + 0x300000, A + 0x400000, 1, None, None,
             None) == moe.MOE_ERR_UNSUPPORTED


def test_microbench_rejects():
    """Argument checks of the measurement kernels (host only)."""
    assert moe._lib.moe_mb_stream_read(None, 1024, 4, 2, A, None) == moe.MOE_ERR_INVALID_ARG
    assert moe._lib.moe_mb_stream_read(A, 1000, 4, 2, A, None) == moe.MOE_ERR_INVALID_ARG
    assert moe._lib.moe_mb_stream_read(A, 1024, 4, 3, A, None) == moe.MOE_ERR_INVALID_ARG
    assert moe._lib.moe_mb_stream_read(A, 1024, 0, 2, A, None) == moe.MOE_ERR_INVALID_ARG
    assert moe._lib.moe_mb_stream_read(A + 8, 1024, 4, 2, A, None) == moe.MOE_ERR_ALIGNMENT
    g = moe._lib.moe_mb_dependent_read
    assert g(None, 1024, 4, 2, A, A, A, None) == moe.MOE_ERR_INVALID_ARG
    assert g(A, 1024, 4, 2, A, None, A, None) == moe.MOE_ERR_INVALID_ARG  # no output vector
    assert g(A, 1024, 4, 8, A, A + 8, A, None) == moe.MOE_ERR_ALIGNMENT
    assert g(A, 1024, 4, 3, A, A, A, None) == moe.MOE_ERR_INVALID_ARG
    assert moe._lib.moe_mb_empty(0, None) == moe.MOE_ERR_INVALID_ARG
    assert moe.moe_mb_exchange_bytes(256, 8) > 256 * 8
    assert moe.moe_mb_exchange_bytes(256, 7) == 0  # blocks not a multiple of groups
    assert moe.moe_mb_exchange_bytes(4096, 8) == 0
    n = moe.moe_mb_exchange_bytes(256, 8)
    f = moe._lib.moe_mb_exchange
    assert f(5, 256, 8, A, n, None) == moe.MOE_ERR_INVALID_ARG
    assert f(4, 256, 128, A, moe.moe_mb_exchange_bytes(256, 128), None) == moe.MOE_ERR_INVALID_ARG  # > 64 counters
    assert f(4, 3, 1, A, moe.moe_mb_exchange_bytes(3, 1), None) == moe.MOE_ERR_INVALID_ARG  # odd grid
    assert f(1, 256, 8, A + 64, n, None) == moe.MOE_ERR_ALIGNMENT
    assert f(1, 256, 8, A, n - 4, None) == moe.MOE_ERR_WORKSPACE
    assert f(1, 256, 8, None, n, None) == moe.MOE_ERR_INVALID_ARG


def test_gdn_rejects():
    """Argument checks of the GatedDeltaNet update, all on the host."""
    f = moe._lib.moe_gdn_update
    P = [A + 0x1000 * i for i in range(7)]
    assert f(0, 128, 128, 1, *P, None) == moe.MOE_ERR_INVALID_ARG
    assert f(4097, 128, 128, 1, *P, None) == moe.MOE_ERR_INVALID_ARG
    assert f(64, 128, 128, 0, *P, None) == moe.MOE_ERR_INVALID_ARG
    assert f(64, 64, 128, 1, *P, None) == moe.MOE_ERR_UNSUPPORTED
    assert f(64, 128, 256, 1, *P, None) == moe.MOE_ERR_UNSUPPORTED
    assert f(64, 128, 128, 1, None, *P[1:], None) == moe.MOE_ERR_INVALID_ARG
    assert f(64, 128, 128, 1, P[0] + 8, *P[1:], None) == moe.MOE_ERR_ALIGNMENT
    assert f(64, 128, 128, 1, P[0], P[1] + 4, *P[2:], None) == moe.MOE_ERR_ALIGNMENT


def test_stage_rejects():
    dims = d()
    wsb = moe.moe_workspace_bytes(dims, 1)
    f = moe._lib.moe_layer_forward_stage
    lay = _layer()
    for stage in (-1, 3, 100):
        assert f(ctypes.byref(dims), ctypes.byref(lay), A + 0x300000, A + 0x400000, 1, None, None, A + 0x500000,
                 wsb, stage, None) == moe.MOE_ERR_INVALID_ARG
    assert f(ctypes.byref(dims), ctypes.byref(lay), A + 0x300000, A + 0x400000, 1, None, None, A + 0x500000,
             16, 0, None) == moe.MOE_ERR_WORKSPACE
    assert f(ctypes.byref(dims), None, A + 0x300000, A + 0x400000, 1, None, None, A + 0x500000,
             wsb, 0, None) == moe.MOE_ERR_INVALID_ARG


def test_stage_count():
    dims = d()
    K = dims.top_k
    assert moe.moe_forward_stage_count(dims, 1) == 3
    assert moe.moe_forward_stage_count(dims, 17) == 3  # 68 assignments: per-token kernels
    assert moe.moe_forward_stage_count(dims, 18) == 7  # 72: grouped by expert
    assert moe.moe_forward_stage_count(dims, 4096 // K) == 7
    assert moe.moe_forward_stage_count(dims, 4096 // K + 1) == 3
    f = moe._lib.moe_forward_stage_count
    assert f(ctypes.byref(dims), 0) == moe.MOE_ERR_INVALID_ARG
    assert f(ctypes.byref(dims), 65536) == moe.MOE_ERR_INVALID_ARG
    bad = d()
    bad.bits = 3
    assert f(ctypes.byref(bad), 1) == moe.MOE_ERR_UNSUPPORTED


def test_grouped_stage_rejects():
    dims = d()
    T = 25
    wsb = moe.moe_workspace_bytes(dims, T)
    f = moe._lib.moe_layer_forward_stage
    lay = _layer()
    for stage in (-1, 7, 100):
        assert f(ctypes.byref(dims), ctypes.byref(lay), A + 0x300000, A + 0x400000, T, None, None, A + 0x500000,
                 wsb, stage, None) == moe.MOE_ERR_INVALID_ARG


def test_stack_rejects():
    dims = d()
    lay = (moe.moe_layer_t * 2)(_layer(), _layer(experts=None))
    wsb = moe.moe_workspace_bytes(dims, 1)
    f = moe._lib.moe_stack_forward
    assert f(ctypes.byref(dims), lay, 2, A, A + 0x400000, 1, None, None, A + 0x500000, wsb, None) == moe.MOE_ERR_INVALID_ARG
    assert f(ctypes.byref(dims), lay, 0, A, A + 0x400000, 1, None, None, A + 0x500000, wsb, None) == moe.MOE_ERR_INVALID_ARG
    assert f(ctypes.byref(dims), None, 1, A, A + 0x400000, 1, None, None, A + 0x500000, wsb, None) == moe.MOE_ERR_INVALID_ARG
    assert f(ctypes.byref(dims), lay, 1, A, A + 0x400000, 1, None, None, A + 0x500000, 16, None) == moe.MOE_ERR_WORKSPACE


def test_pack_generate_init_reject():
    dims = d()
    P = moe._vp * 3
    ok3 = P(A, A + 0x1000, A + 0x2000)
    bad3 = P(A, None, A + 0x2000)
    f = moe._lib.moe_pack_expert
    assert f(ctypes.byref(dims), bad3, ok3, ok3, A + 0x100000, None) == moe.MOE_ERR_INVALID_ARG
    assert f(ctypes.byref(dims), ok3, ok3, ok3, A + 0x100010, None) == moe.MOE_ERR_ALIGNMENT
    assert f(ctypes.byref(d(bits=3)), ok3, ok3, ok3, A + 0x100000, None) == moe.MOE_ERR_UNSUPPORTED
    g = moe._lib.moe_generate_layer
    assert g(ctypes.byref(dims), 0, 0, None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert g(ctypes.byref(dims), 0, 0, A + 0x80, None, None) == moe.MOE_ERR_ALIGNMENT
    i = moe._lib.moe_workspace_init
    assert i(None, 16384, None) == moe.MOE_ERR_INVALID_ARG
    assert i(A, 16, None) == moe.MOE_ERR_WORKSPACE
    assert i(A, 4096, None) == moe.MOE_ERR_WORKSPACE  # the control block is 8 KiB
    assert i(A + 8, 16384, None) == moe.MOE_ERR_ALIGNMENT


def test_status_strings():
    for s in range(0, -6, -1):
        assert moe.moe_status_string(s) not in ("", "unknown status")
    assert moe.moe_status_string(-99) == "unknown status"


# --------------------------------------------------------------------------- #
# tiered expert residency: sizes, initialisation and argument checks (host only)
# --------------------------------------------------------------------------- #
def test_tier_sizes():
    dims = d()
    eb = moe.moe_expert_bytes(dims)
    for ns, T in ((4, 1), (64, 16), (4096, 3)):
        assert moe.moe_tier_device_bytes(dims, ns, T) == ns * eb
    base = moe.moe_tier_state_bytes(dims, 1, 4, 1)
    assert base > 0
    # int32 bookkeeping (3 per slot, 1 per (layer, expert)) padded to 8 bytes, then one
    # 8-byte tagged entry per assignment of one call
    assert moe.moe_tier_state_bytes(dims, 1, 5, 1) - base == 16  # 12 + 512 ints, then 15 + 512 -> 528
    assert moe.moe_tier_state_bytes(dims, 1, 6, 1) - base == 24
    assert moe.moe_tier_state_bytes(dims, 3, 4, 1) - base == 2 * 512 * 4
    assert moe.moe_tier_state_bytes(dims, 1, 8, 2) - moe.moe_tier_state_bytes(dims, 1, 8, 1) == dims.top_k * 8
    # at most 64 assignments per call (the slots travel as kernel arguments)
    assert moe.moe_tier_state_bytes(dims, 1, 64, 16) > 0
    assert moe.moe_tier_state_bytes(dims, 1, 68, 17) == 0
    for args in ((0, 4, 1), (1, 3, 1), (1, 7, 2), (1, 4, 0), (1, 70000 * 4, 70000), (1 << 22, 4, 1)):
        assert moe.moe_tier_state_bytes(dims, *args) == 0, args
    assert moe.moe_tier_device_bytes(dims, 3, 1) == 0
    assert moe.moe_tier_device_bytes(dims, 68, 17) == 0
    assert moe.moe_tier_state_bytes(d(bits=3), 1, 4, 1) == 0


def _tier_state(dims, n_layers, n_slots, max_tokens):
    import numpy as np
    buf = np.zeros(moe.moe_tier_state_bytes(dims, n_layers, n_slots, max_tokens) + 8, np.uint8)
    addr = buf.ctypes.data
    addr += (-addr) % 8
    return buf, addr


def test_tier_init_lookup_and_rejects():
    dims = d()
    n_layers, n_slots, max_tokens = 2, 16, 2
    buf, st = _tier_state(dims, n_layers, n_slots, max_tokens)
    sb = moe.moe_tier_state_bytes(dims, n_layers, n_slots, max_tokens)
    db = moe.moe_tier_device_bytes(dims, n_slots, max_tokens)
    f = moe._lib.moe_tier_init
    # the device memory is never touched by init: a fake address is enough
    assert f(ctypes.byref(dims), n_layers, n_slots, max_tokens, st, sb - 4, A, db) == moe.MOE_ERR_WORKSPACE
    assert f(ctypes.byref(dims), n_layers, n_slots, max_tokens, st, sb, A, db - 1) == moe.MOE_ERR_WORKSPACE
    assert f(ctypes.byref(dims), n_layers, n_slots, max_tokens, st + 4, sb, A, db) == moe.MOE_ERR_ALIGNMENT
    assert f(ctypes.byref(dims), n_layers, n_slots, max_tokens, st, sb, A + 64, db) == moe.MOE_ERR_ALIGNMENT
    assert f(ctypes.byref(dims), n_layers, n_slots, max_tokens, None, sb, A, db) == moe.MOE_ERR_INVALID_ARG
    assert f(ctypes.byref(dims), n_layers, 7, max_tokens, st, sb, A, db) == moe.MOE_ERR_INVALID_ARG
    assert f(ctypes.byref(dims), n_layers, 68, 17, st, sb, A, db) == moe.MOE_ERR_UNSUPPORTED
    # not initialised yet: no entry point accepts the state
    assert moe._lib.moe_tier_get_stats(st, ctypes.byref(moe.moe_tier_stats_t())) == moe.MOE_ERR_INVALID_ARG
    assert f(ctypes.byref(dims), n_layers, n_slots, max_tokens, st, sb, A, db) == moe.MOE_OK
    s = moe.moe_tier_get_stats(st)
    assert (s.calls, s.lookups, s.hits, s.misses, s.bytes_copied) == (0, 0, 0, 0, 0)
    for layer in range(n_layers):
        for e in (0, 7, 511):
            assert moe.moe_tier_lookup(st, layer, e) == -1
    slot = ctypes.c_int32()
    lk = moe._lib.moe_tier_lookup
    assert lk(st, 2, 0, ctypes.byref(slot)) == moe.MOE_ERR_INVALID_ARG
    assert lk(st, 0, 512, ctypes.byref(slot)) == moe.MOE_ERR_INVALID_ARG
    assert lk(st, 0, 0, None) == moe.MOE_ERR_INVALID_ARG
    # forward: every check precedes the first HIP call
    fw = moe._lib.moe_tier_layer_forward
    wsb = moe.moe_workspace_bytes(dims, max_tokens + 1)
    lay = _layer()

    def call(state=st, li=0, layer=lay, T=1, ws=A + 0x500000):
        return fw(state, li, ctypes.byref(layer) if layer else None, A + 0x300000, A + 0x400000, T, None, None,
                  ws, wsb, None)

    assert call(state=st + 8) == moe.MOE_ERR_INVALID_ARG  # not a state
    assert call(li=-1) == moe.MOE_ERR_INVALID_ARG
    assert call(li=n_layers) == moe.MOE_ERR_INVALID_ARG
    assert call(T=max_tokens + 1) == moe.MOE_ERR_INVALID_ARG
    assert call(layer=_layer(experts=None)) == moe.MOE_ERR_INVALID_ARG
    assert call(ws=A + 0x500010) == moe.MOE_ERR_ALIGNMENT
    sf = moe._lib.moe_tier_stack_forward
    lays = (moe.moe_layer_t * 3)(lay, lay, lay)
    assert sf(st, lays, 3, A + 0x300000, A + 0x400000, 1, None, None, A + 0x500000, wsb, None) == \
        moe.MOE_ERR_INVALID_ARG  # more layers than the state holds
    assert sf(st, lays, 0, A + 0x300000, A + 0x400000, 1, None, None, A + 0x500000, wsb, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert sf(st + 8, lays, 1, A + 0x300000, A + 0x400000, 1, None, None, A + 0x500000, wsb, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert moe.moe_tier_get_stats(st).calls == 0
