"""Python binding of libmoe, the MI355X (gfx950) Flash-MoE expert layer.

Argument marshalling only: every function here forwards to the entry point of
the same name in ``include/moe.h``.  Tensors are PyTorch tensors on the GPU
(used for device memory and streams) or raw device addresses given as ints.
There is no fallback: importing this package raises if ``libmoe.so`` has not
been built (``python bit_dequant_expert_router_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# MOE_LIBRARY names another build of the same library (the host-sanitizer
# build of tests/sanitize_host.py); it is loaded in its place, never as a fallback
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(PKG_DIR, "libmoe.so")

# torch first: its bundled HIP runtime (soname libamdhip64.so.7) must be the
# one libmoe.so binds to.  Loading libmoe.so first would bring in a second HIP
# runtime from /opt/rocm, and the two cannot share the device.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python bit_dequant_expert_router_amd/build.py` "
        "(there is no CPU fallback)")

_lib = ctypes.CDLL(LIB_PATH)

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_ALIGNMENT = -4
MOE_ERR_HIP = -5


class moe_dims_t(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("ffn", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("bits", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("rms_eps", ctypes.c_float)]


class moe_layer_t(ctypes.Structure):
    _fields_ = [("norm_weight", ctypes.c_void_p), ("router_weight", ctypes.c_void_p),
                ("shared_gate", ctypes.c_void_p), ("experts", ctypes.c_void_p),
                ("shared_expert", ctypes.c_void_p)]


class moe_tier_stats_t(ctypes.Structure):
    _fields_ = [("calls", ctypes.c_uint64), ("lookups", ctypes.c_uint64), ("hits", ctypes.c_uint64),
                ("misses", ctypes.c_uint64), ("bytes_copied", ctypes.c_uint64)]


_vp = ctypes.c_void_p
_dimsp = ctypes.POINTER(moe_dims_t)
_layerp = ctypes.POINTER(moe_layer_t)
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t

_SIGS = {
    "moe_abi_version": (ctypes.c_int, []),
    "moe_check_dims": (ctypes.c_int, [_dimsp]),
    "moe_expert_bytes": (_sz, [_dimsp]),
    "moe_workspace_bytes": (_sz, [_dimsp, _i32]),
    "moe_workspace_init": (ctypes.c_int, [_vp, _sz, _vp]),
    "moe_pack_expert": (ctypes.c_int, [_dimsp, _vp * 3, _vp * 3, _vp * 3, _vp, _vp]),
    "moe_generate_layer": (ctypes.c_int, [_dimsp, ctypes.c_uint64, ctypes.c_uint32, _vp, _vp, _vp]),
    "moe_layer_forward": (ctypes.c_int, [_dimsp, _layerp, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "moe_layer_forward_noalloc": (ctypes.c_int, [_dimsp, _layerp, _vp, _vp, _i32, _vp, _vp, _vp]),
    "moe_layer_forward_stage": (ctypes.c_int, [_dimsp, _layerp, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _i32, _vp]),
    "moe_forward_stage_count": (ctypes.c_int, [_dimsp, _i32]),
    "moe_stack_forward": (ctypes.c_int, [_dimsp, _layerp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "moe_tier_state_bytes": (_sz, [_dimsp, _i32, _i32, _i32]),
    "moe_tier_device_bytes": (_sz, [_dimsp, _i32, _i32]),
    "moe_tier_init": (ctypes.c_int, [_dimsp, _i32, _i32, _i32, _vp, _sz, _vp, _sz]),
    "moe_tier_layer_forward": (ctypes.c_int, [_vp, _i32, _layerp, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "moe_tier_stack_forward": (ctypes.c_int, [_vp, _layerp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "moe_tier_get_stats": (ctypes.c_int, [_vp, ctypes.POINTER(moe_tier_stats_t)]),
    "moe_tier_lookup": (ctypes.c_int, [_vp, _i32, _i32, ctypes.POINTER(ctypes.c_int32)]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    # GatedDeltaNet state update (include/moe_gdn.h)
    "moe_gdn_update": (ctypes.c_int, [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    # measurement kernels (include/moe_microbench.h)
    "moe_mb_stream_read": (ctypes.c_int, [_vp, _sz, _i32, _i32, _vp, _vp]),
    "moe_mb_dependent_read": (ctypes.c_int, [_vp, _sz, _i32, _i32, _vp, _vp, _vp, _vp]),
    "moe_mb_empty": (ctypes.c_int, [_i32, _vp]),
    "moe_mb_exchange": (ctypes.c_int, [_i32, _i32, _i32, _vp, _sz, _vp]),
    "moe_mb_exchange_bytes": (_sz, [_i32, _i32]),
    "moe_mb_exchange_failures": (ctypes.c_int, [_vp, ctypes.POINTER(ctypes.c_uint32)]),
    "moe_last_error": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        detail = f" [{moe_last_error()}]" if status == MOE_ERR_HIP else ""
        super().__init__(f"{fn}: {moe_status_string(status)} ({status}){detail}")
        self.status = status


def _addr(t) -> Optional[int]:
    """Device address of a tensor, an int address, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        # the current stream's handle without building a Stream object (2.6 us a call)
        return torch._C._cuda_getCurrentRawStream(torch.cuda.current_device()) or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def _check(fn: str, rc: int) -> int:
    if rc != MOE_OK:
        raise MoeError(fn, rc)
    return rc


def make_dims(hidden: int, ffn: int, n_experts: int, top_k: int, bits: int, group_size: int = 64,
              rms_eps: float = 1e-6) -> moe_dims_t:
    return moe_dims_t(hidden, ffn, n_experts, top_k, bits, group_size, rms_eps)


def dims_of(d) -> moe_dims_t:
    """moe_dims_t from any object with hidden/ffn/n_experts/top_k/bits fields."""
    if isinstance(d, moe_dims_t):
        return d
    return make_dims(d.hidden, d.ffn, d.n_experts, d.top_k, d.bits, getattr(d, "group_size", 64),
                     getattr(d, "rms_eps", 1e-6))


def make_layer(norm_weight, router_weight, shared_gate, experts, shared_expert) -> moe_layer_t:
    return moe_layer_t(_addr(norm_weight), _addr(router_weight), _addr(shared_gate), _addr(experts),
                       _addr(shared_expert))


# --------------------------------------------------------------------------- #
# entry points (same names as the C ABI)
# --------------------------------------------------------------------------- #
def moe_abi_version() -> int:
    return int(_lib.moe_abi_version())


def moe_status_string(status: int) -> str:
    return _lib.moe_status_string(int(status)).decode()


def moe_last_error() -> str:
    return _lib.moe_last_error().decode()


def moe_check_dims(dims) -> int:
    return int(_lib.moe_check_dims(ctypes.byref(dims_of(dims))))


def moe_expert_bytes(dims) -> int:
    return int(_lib.moe_expert_bytes(ctypes.byref(dims_of(dims))))


def moe_workspace_bytes(dims, n_tokens: int) -> int:
    return int(_lib.moe_workspace_bytes(ctypes.byref(dims_of(dims)), int(n_tokens)))


def moe_workspace_init(workspace, workspace_bytes: Optional[int] = None, stream=None) -> int:
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    return _check("moe_workspace_init", _lib.moe_workspace_init(_addr(workspace), nbytes, _stream(stream)))


def moe_pack_expert(dims, codes: Sequence, scale: Sequence, bias: Sequence, dst, stream=None) -> int:
    c = (_vp * 3)(*[_addr(t) for t in codes])
    s = (_vp * 3)(*[_addr(t) for t in scale])
    b = (_vp * 3)(*[_addr(t) for t in bias])
    return _check("moe_pack_expert",
                  _lib.moe_pack_expert(ctypes.byref(dims_of(dims)), c, s, b, _addr(dst), _stream(stream)))


def moe_generate_layer(dims, seed: int, layer: int, experts, shared_expert, stream=None) -> int:
    return _check("moe_generate_layer",
                  _lib.moe_generate_layer(ctypes.byref(dims_of(dims)), int(seed), int(layer), _addr(experts),
                                          _addr(shared_expert), _stream(stream)))


def moe_layer_forward(dims, layer: moe_layer_t, x, y, n_tokens: int, route_idx, route_w, workspace,
                      workspace_bytes: Optional[int] = None, stream=None) -> int:
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    return _check("moe_layer_forward",
                  _lib.moe_layer_forward(ctypes.byref(dims_of(dims)), ctypes.byref(layer), _addr(x), _addr(y),
                                         int(n_tokens), _addr(route_idx), _addr(route_w), _addr(workspace),
                                         nbytes, _stream(stream)))


def layer_forward_call(dims, layer: moe_layer_t, x, y, n_tokens: int, route_idx, route_w, workspace,
                       workspace_bytes: Optional[int] = None, stream=None):
    """moe_layer_forward with its arguments marshalled once: returns a function of
    no arguments that makes the call (and raises on an error code), for loops that
    repeat one call.  The tensors must outlive the returned function."""
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    d = dims_of(dims)
    args = (ctypes.byref(d), ctypes.byref(layer), _addr(x), _addr(y), int(n_tokens), _addr(route_idx),
            _addr(route_w), _addr(workspace), nbytes, _stream(stream))
    f = _lib.moe_layer_forward

    def call():
        rc = f(*args)
        if rc != MOE_OK:
            raise MoeError("moe_layer_forward", rc)

    call.keep = (d, layer)  # the structures the byref pointers refer to
    return call


MOE_NOALLOC_SCRATCH_BYTES = 16 << 20  # include/moe.h


def moe_layer_forward_noalloc(dims, layer: moe_layer_t, x, y, n_tokens: int, route_idx, route_w,
                              stream=None) -> int:
    return _check("moe_layer_forward_noalloc",
                  _lib.moe_layer_forward_noalloc(ctypes.byref(dims_of(dims)), ctypes.byref(layer), _addr(x),
                                                 _addr(y), int(n_tokens), _addr(route_idx), _addr(route_w),
                                                 _stream(stream)))


def moe_layer_forward_stage(dims, layer: moe_layer_t, x, y, n_tokens: int, route_idx, route_w, workspace,
                            workspace_bytes: Optional[int], stage: int, stream=None) -> int:
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    return _check("moe_layer_forward_stage",
                  _lib.moe_layer_forward_stage(ctypes.byref(dims_of(dims)), ctypes.byref(layer), _addr(x),
                                               _addr(y), int(n_tokens), _addr(route_idx), _addr(route_w),
                                               _addr(workspace), nbytes, int(stage), _stream(stream)))


def moe_forward_stage_count(dims, n_tokens: int) -> int:
    rc = int(_lib.moe_forward_stage_count(ctypes.byref(dims_of(dims)), int(n_tokens)))
    if rc < 0:
        raise MoeError("moe_forward_stage_count", rc)
    return rc


def moe_stack_forward(dims, layers: Sequence[moe_layer_t], x, y, n_tokens: int, route_idx, route_w,
                      workspace, workspace_bytes: Optional[int] = None, stream=None) -> int:
    arr = (moe_layer_t * len(layers))(*layers)
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    return _check("moe_stack_forward",
                  _lib.moe_stack_forward(ctypes.byref(dims_of(dims)), arr, len(layers), _addr(x), _addr(y),
                                         int(n_tokens), _addr(route_idx), _addr(route_w), _addr(workspace),
                                         nbytes, _stream(stream)))


# tiered expert residency: `state` is pinned host memory (for example a uint8
# tensor made with pin_memory=True), `device` device memory; layer.experts of
# moe_tier_layer_forward is the host copy of the layer's packed experts
def _nbytes(t, given: Optional[int]) -> int:
    return given if given is not None else t.numel() * t.element_size()


def moe_tier_state_bytes(dims, n_layers: int, n_slots: int, max_tokens: int) -> int:
    return int(_lib.moe_tier_state_bytes(ctypes.byref(dims_of(dims)), int(n_layers), int(n_slots),
                                         int(max_tokens)))


def moe_tier_device_bytes(dims, n_slots: int, max_tokens: int) -> int:
    return int(_lib.moe_tier_device_bytes(ctypes.byref(dims_of(dims)), int(n_slots), int(max_tokens)))


def moe_tier_init(dims, n_layers: int, n_slots: int, max_tokens: int, state, device,
                  state_bytes: Optional[int] = None, device_bytes: Optional[int] = None) -> int:
    return _check("moe_tier_init",
                  _lib.moe_tier_init(ctypes.byref(dims_of(dims)), int(n_layers), int(n_slots), int(max_tokens),
                                     _addr(state), _nbytes(state, state_bytes), _addr(device),
                                     _nbytes(device, device_bytes)))


def moe_tier_layer_forward(state, layer_index: int, layer: moe_layer_t, x, y, n_tokens: int, route_idx, route_w,
                           workspace, workspace_bytes: Optional[int] = None, stream=None) -> int:
    return _check("moe_tier_layer_forward",
                  _lib.moe_tier_layer_forward(_addr(state), int(layer_index), ctypes.byref(layer), _addr(x),
                                              _addr(y), int(n_tokens), _addr(route_idx), _addr(route_w),
                                              _addr(workspace), _nbytes(workspace, workspace_bytes),
                                              _stream(stream)))


def moe_tier_stack_forward(state, layers: Sequence[moe_layer_t], x, y, n_tokens: int, route_idx, route_w,
                           workspace, workspace_bytes: Optional[int] = None, stream=None) -> int:
    arr = (moe_layer_t * len(layers))(*layers)
    return _check("moe_tier_stack_forward",
                  _lib.moe_tier_stack_forward(_addr(state), arr, len(layers), _addr(x), _addr(y), int(n_tokens),
                                              _addr(route_idx), _addr(route_w), _addr(workspace),
                                              _nbytes(workspace, workspace_bytes), _stream(stream)))


def moe_tier_get_stats(state) -> moe_tier_stats_t:
    out = moe_tier_stats_t()
    _check("moe_tier_get_stats", _lib.moe_tier_get_stats(_addr(state), ctypes.byref(out)))
    return out


def moe_tier_lookup(state, layer_index: int, expert: int) -> int:
    slot = ctypes.c_int32()
    _check("moe_tier_lookup", _lib.moe_tier_lookup(_addr(state), int(layer_index), int(expert), ctypes.byref(slot)))
    return slot.value


# GatedDeltaNet recurrent-state update (include/moe_gdn.h)
def moe_gdn_update(n_heads: int, d_k: int, d_v: int, n_tokens: int, state, q, k, v, alpha, beta, out,
                   stream=None) -> int:
    return _check("moe_gdn_update",
                  _lib.moe_gdn_update(int(n_heads), int(d_k), int(d_v), int(n_tokens), _addr(state), _addr(q),
                                      _addr(k), _addr(v), _addr(alpha), _addr(beta), _addr(out), _stream(stream)))


# measurement kernels (include/moe_microbench.h): no part of the layer
def moe_mb_stream_read(src, nbytes: int, blocks: int, in_flight: int, sink, stream=None) -> int:
    return _check("moe_mb_stream_read", _lib.moe_mb_stream_read(_addr(src), int(nbytes), int(blocks),
                                                                int(in_flight), _addr(sink), _stream(stream)))


def moe_mb_dependent_read(src, nbytes: int, blocks: int, in_flight: int, dep, out, sink, stream=None) -> int:
    return _check("moe_mb_dependent_read",
                  _lib.moe_mb_dependent_read(_addr(src), int(nbytes), int(blocks), int(in_flight), _addr(dep),
                                             _addr(out), _addr(sink), _stream(stream)))


def moe_mb_empty(blocks: int, stream=None) -> int:
    return _check("moe_mb_empty", _lib.moe_mb_empty(int(blocks), _stream(stream)))


def moe_mb_exchange_bytes(blocks: int, groups: int) -> int:
    return int(_lib.moe_mb_exchange_bytes(int(blocks), int(groups)))


def moe_mb_exchange(kind: int, blocks: int, groups: int, buf, buf_bytes: Optional[int] = None, stream=None) -> int:
    return _check("moe_mb_exchange", _lib.moe_mb_exchange(int(kind), int(blocks), int(groups), _addr(buf),
                                                          _nbytes(buf, buf_bytes), _stream(stream)))


def moe_mb_exchange_failures(buf) -> int:
    out = ctypes.c_uint32()
    _check("moe_mb_exchange_failures", _lib.moe_mb_exchange_failures(_addr(buf), ctypes.byref(out)))
    return int(out.value)
