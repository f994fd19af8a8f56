"""fp64 CPU oracle of the Flash-MoE expert layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It never imports the GPU library and
shares no code with it; both sides receive their inputs from ``synthetic``.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp64, serial sums); this
module loads it with ctypes and strings the steps together in the pages' order
(RMSNorm -> router GEMV -> softmax/top-K/renormalise -> the K selected experts
and the shared expert, each gate/up -> SwiGLU -> down -> weighted combine with
the sigmoid-gated shared expert and the residual).  Steps are cited in
``moe_oracle.c``.

Parity status of each function (what pins it is listed in
``tests/test_oracle_pins.py``): all pinned except absolute end-to-end values of
the original trained model, which the pages do not print (parity unpinned).

``oracle/lru.py`` (pure Python) holds the expert-cache policy of tiered
residency, a plain least-recently-used cache, pinned in
``tests/test_tier_oracle.py``.  ``oracle/gdn.py`` (numpy, fp64) holds the
GatedDeltaNet recurrent-state update of the linear-attention layers, pinned in
``tests/test_gdn_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "moe_oracle.c")
# ORACLE_LIBRARY: another build of moe_oracle.c to load (the host-sanitizer
# build of tests/sanitize_host.py)
_LOAD_PATH = os.environ.get("ORACLE_LIBRARY") or LIB_PATH


def build(force: bool = False) -> str:
    """Compile moe_oracle.c with gcc (fp64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-shared", "-fPIC", "-std=c11", SRC_PATH, "-o", tmp, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        if _LOAD_PATH == LIB_PATH and not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(_LOAD_PATH)
        L.oracle_threads.restype = ctypes.c_int
        L.oracle_dequant.restype = ctypes.c_double
        L.oracle_dequant.argtypes = [ctypes.c_uint8, ctypes.c_uint16, ctypes.c_uint16]
        L.oracle_rmsnorm.argtypes = [_i64, _fp, _u16p, ctypes.c_double, _dp]
        L.oracle_gemv_bf16.argtypes = [_i64, _i64, _u16p, _dp, _dp]
        L.oracle_qgemv.argtypes = [_i64, _i64, _i64, _u8p, _u16p, _u16p, _dp, _dp]
        L.oracle_route.restype = ctypes.c_int
        L.oracle_route.argtypes = [_i64, _i64, _dp, _i32p, _dp]
        L.oracle_expert.argtypes = [_i64, _i64, _i64, ctypes.POINTER(_u8p), ctypes.POINTER(_u16p),
                                    ctypes.POINTER(_u16p), _dp, _dp]
        L.oracle_layer.restype = ctypes.c_int
        L.oracle_layer.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.c_double, _fp, _u16p, _u16p,
                                   _u16p, ctypes.POINTER(_u8p), ctypes.POINTER(_u16p),
                                   ctypes.POINTER(_u16p), _dp, _i32p, _dp, _dp, _dp]
        _lib = L
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def threads() -> int:
    return int(lib().oracle_threads())


# --------------------------------------------------------------------------- #
# single steps
# --------------------------------------------------------------------------- #
def dequant(code: int, scale_bits: int, bias_bits: int) -> float:
    return float(lib().oracle_dequant(code, scale_bits, bias_bits))


def rmsnorm(x: np.ndarray, gamma_bits: np.ndarray, eps: float) -> np.ndarray:
    x = _c(x, np.float32)
    g = _c(gamma_bits, np.uint16)
    h = np.empty(x.size, np.float64)
    lib().oracle_rmsnorm(x.size, _ptr(x, ctypes.c_float), _ptr(g, ctypes.c_uint16), eps,
                         _ptr(h, ctypes.c_double))
    return h


def gemv_bf16(W_bits: np.ndarray, v: np.ndarray) -> np.ndarray:
    W = _c(W_bits, np.uint16)
    rows, cols = W.shape
    v = _c(v, np.float64)
    out = np.empty(rows, np.float64)
    lib().oracle_gemv_bf16(rows, cols, _ptr(W, ctypes.c_uint16), _ptr(v, ctypes.c_double),
                           _ptr(out, ctypes.c_double))
    return out


def qgemv(codes: np.ndarray, scale_bits: np.ndarray, bias_bits: np.ndarray, v: np.ndarray,
          group: int = 64) -> np.ndarray:
    q = _c(codes, np.uint8)
    rows, cols = q.shape
    s = _c(scale_bits, np.uint16)
    b = _c(bias_bits, np.uint16)
    assert s.shape == (rows, cols // group) and b.shape == s.shape
    v = _c(v, np.float64)
    out = np.empty(rows, np.float64)
    lib().oracle_qgemv(rows, cols, group, _ptr(q, ctypes.c_uint8), _ptr(s, ctypes.c_uint16),
                       _ptr(b, ctypes.c_uint16), _ptr(v, ctypes.c_double), _ptr(out, ctypes.c_double))
    return out


def route(z: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    z = _c(z, np.float64)
    idx = np.empty(k, np.int32)
    w = np.empty(k, np.float64)
    rc = lib().oracle_route(z.size, k, _ptr(z, ctypes.c_double), _ptr(idx, ctypes.c_int32),
                            _ptr(w, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_route: bad arguments")
    return idx, w


def _expert_ptrs(exp: Dict[str, List[np.ndarray]]):
    keep = [[_c(a, np.uint8) for a in exp["codes"]],
            [_c(a, np.uint16) for a in exp["scale"]],
            [_c(a, np.uint16) for a in exp["bias"]]]
    cp = (_u8p * 3)(*[_ptr(a, ctypes.c_uint8) for a in keep[0]])
    sp = (_u16p * 3)(*[_ptr(a, ctypes.c_uint16) for a in keep[1]])
    bp = (_u16p * 3)(*[_ptr(a, ctypes.c_uint16) for a in keep[2]])
    return keep, cp, sp, bp


def expert(exp: Dict[str, List[np.ndarray]], h: np.ndarray, group: int = 64) -> np.ndarray:
    F, H = exp["codes"][0].shape
    keep, cp, sp, bp = _expert_ptrs(exp)
    h = _c(h, np.float64)
    y = np.empty(H, np.float64)
    lib().oracle_expert(H, F, group, cp, sp, bp, _ptr(h, ctypes.c_double), _ptr(y, ctypes.c_double))
    return y


def sigmoid(t: float) -> float:
    return float(1.0 / (1.0 + np.exp(-np.float64(t))))


# --------------------------------------------------------------------------- #
# whole layer / stack
# --------------------------------------------------------------------------- #
def layer_all(dims, x: np.ndarray, dense: Dict[str, np.ndarray],
              experts: Sequence[Optional[Dict[str, List[np.ndarray]]]]):
    """Whole layer in C (oracle_layer) for one token; ``experts`` has E+1
    entries (the last is the shared expert), unselected ones may be None."""
    H, F, E, K = dims.hidden, dims.ffn, dims.n_experts, dims.top_k
    keep = []
    cp = (_u8p * (3 * (E + 1)))()
    sp = (_u16p * (3 * (E + 1)))()
    bp = (_u16p * (3 * (E + 1)))()
    for e, ex in enumerate(experts):
        if ex is None:
            continue
        k, c3, s3, b3 = _expert_ptrs(ex)
        keep.append(k)
        for m in range(3):
            cp[3 * e + m], sp[3 * e + m], bp[3 * e + m] = c3[m], s3[m], b3[m]
    x = _c(x, np.float32)
    g = _c(dense["norm_weight"], np.uint16)
    r = _c(dense["router_weight"], np.uint16)
    sg = _c(dense["shared_gate"], np.uint16)
    out = np.empty(H, np.float64)
    idx = np.empty(K, np.int32)
    w = np.empty(K, np.float64)
    z = np.empty(E, np.float64)
    gs = np.empty(1, np.float64)
    rc = lib().oracle_layer(H, F, E, K, dims.group_size, dims.rms_eps, _ptr(x, ctypes.c_float),
                            _ptr(g, ctypes.c_uint16), _ptr(r, ctypes.c_uint16), _ptr(sg, ctypes.c_uint16),
                            cp, sp, bp, _ptr(out, ctypes.c_double), _ptr(idx, ctypes.c_int32),
                            _ptr(w, ctypes.c_double), _ptr(z, ctypes.c_double), _ptr(gs, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"oracle_layer failed ({rc})")
    return {"out": out, "idx": idx, "w": w, "z": z, "gs": float(gs[0])}


def layer(dims, x: np.ndarray, dense: Dict[str, np.ndarray],
          fetch_expert: Callable[[int], Dict[str, List[np.ndarray]]]):
    """The layer for one token, fetching only the experts the routing selects
    (``fetch_expert(e)``; e == E is the shared expert)."""
    E, K = dims.n_experts, dims.top_k
    h = rmsnorm(x, dense["norm_weight"], dims.rms_eps)
    z = gemv_bf16(dense["router_weight"], h)
    gs = float(gemv_bf16(np.asarray(dense["shared_gate"]).reshape(1, -1), h)[0])
    idx, w = route(z, K)
    out = np.asarray(x, np.float32).astype(np.float64)
    for k in range(K + 1):
        e = int(idx[k]) if k < K else E
        coef = float(w[k]) if k < K else sigmoid(gs)
        y = expert(fetch_expert(e), h, dims.group_size)
        out = out + coef * y
    return {"out": out, "idx": idx, "w": w, "z": z, "gs": gs, "h": h}


def layer_forced(dims, x: np.ndarray, dense: Dict[str, np.ndarray],
                 fetch_expert: Callable[[int], Dict[str, List[np.ndarray]]], idx: Sequence[int]):
    """The layer for one token with the selection given (K distinct experts, in
    the order given): for a near tie, where either selection is correct, the
    outputs the other selection defines.  The weights are the softmax restricted
    to the selection, exp(z_k - m) / sum_j exp(z_j - m) with m the largest
    selected logit, which equals the full softmax renormalised over it."""
    E, K = dims.n_experts, dims.top_k
    idx = [int(e) for e in idx]
    if len(idx) != K or len(set(idx)) != K or min(idx) < 0 or max(idx) >= E:
        raise ValueError("layer_forced: K distinct experts expected")
    h = rmsnorm(x, dense["norm_weight"], dims.rms_eps)
    z = gemv_bf16(dense["router_weight"], h)
    gs = float(gemv_bf16(np.asarray(dense["shared_gate"]).reshape(1, -1), h)[0])
    zs = z[idx]
    p = np.exp(zs - np.max(zs))
    w = p / np.sum(p)
    out = np.asarray(x, np.float32).astype(np.float64)
    for k in range(K + 1):
        e = idx[k] if k < K else E
        coef = float(w[k]) if k < K else sigmoid(gs)
        out = out + coef * expert(fetch_expert(e), h, dims.group_size)
    return {"out": out, "idx": np.array(idx, np.int32), "w": w, "z": z, "gs": gs, "h": h}


def near_tie(z: np.ndarray, k: int, rel: float = 1e-5) -> bool:
    """True when the K-th and (K+1)-th largest logits are closer than
    rel * max(1, max|z|): then either selection is a correct routing."""
    if k >= z.size:
        return False
    s = np.sort(np.asarray(z, np.float64))[::-1]
    return bool(s[k - 1] - s[k] < rel * max(1.0, float(np.max(np.abs(z)))))
