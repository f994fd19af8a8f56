"""Seeded synthetic inputs for the Flash-MoE expert layer.

This module is shared by the CPU oracle (``oracle/``) and by the GPU path's
tests and benchmark.  It builds inputs only: it holds none of the layer's
arithmetic (no normalisation, routing, dequantisation or products).

Shapes and value distributions follow the model the pages describe
(hidden 4096, 512 experts per layer, K=4 active experts plus one shared expert,
60 layers: "48GB内存运行397B模型", section "MoE稀疏架构"; the native 10+1
routing: juejin post, "为什么 397B 的模型能塞进 48GB").  The trained weights
are not available, so every tensor is synthetic:

* expert codes: uniform integers in [0, 2**bits), from a counter-based
  SplitMix64 stream (Steele, Lea & Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014).  One 64-bit output supplies 64/bits consecutive
  codes, lowest bits first;
* group scales: uniform in [0.005, 0.02), group biases: uniform in [-0.1, 0),
  one 64-bit output each, rounded fp64 -> fp32 -> bf16 (round to nearest even);
* router rows and the shared-expert gate vector: N(0, 0.02) rounded to bf16;
* RMSNorm weights: U(0.5, 1.5) rounded to bf16;
* activations x: N(0, 1) in fp32.

The expert-weight stream is defined exactly so that a device-side generator
can reproduce it bit for bit (the library's ``moe_generate_layer``):

    mix64(z):   z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9
                z = (z ^ (z >> 27)) * 0x94D049BB133111EB
                return z ^ (z >> 31)                 (all mod 2**64)
    tag       = (layer << 32) | (expert << 16) | (matrix << 8) | kind
    base      = mix64(mix64(seed + GAMMA) ^ tag),     GAMMA = 0x9E3779B97F4A7C15
    word[i]   = mix64(base + (i + 1) * GAMMA)         (SplitMix64 seeded with base)

matrix: 0 = gate [F][H], 1 = up [F][H], 2 = down [H][F] (row = output,
column = reduction index); kind: 0 = codes, 1 = scales, 2 = biases;
expert: 0..E-1 routed, E = the shared expert.  Code i of a matrix (row-major)
is bits [bits*(i mod 64/bits), +bits) of word[i div (64/bits)].  Scale and bias
of group g (row-major over [rows][cols/64]) use u = (word[g] >> 40) * 2**-24 and
s = fl64(fl64(0.015 * u) + 0.005), b = fl64(fl64(0.1 * u) - 0.1), each product
and sum rounded separately in fp64 (no fused multiply-add), then converted to
fp32 and to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
M64 = (1 << 64) - 1
GROUP = 64

GATE, UP, DOWN = 0, 1, 2
KIND_CODES, KIND_SCALE, KIND_BIAS = 0, 1, 2


# --------------------------------------------------------------------------- #
# SplitMix64
# --------------------------------------------------------------------------- #
def mix64_int(z: int) -> int:
    """SplitMix64 finaliser on a Python int (mod 2**64)."""
    z &= M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser, vectorised over a uint64 array (wraps mod 2**64)."""
    z = z.astype(np.uint64, copy=True)
    z ^= z >> np.uint64(30)
    z *= np.uint64(0xBF58476D1CE4E5B9)
    z ^= z >> np.uint64(27)
    z *= np.uint64(0x94D049BB133111EB)
    z ^= z >> np.uint64(31)
    return z


def splitmix64(base: int, n: int, start: int = 0) -> np.ndarray:
    """Outputs start .. start+n-1 of SplitMix64 seeded with ``base``."""
    i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(base & M64) + i * np.uint64(GAMMA)
    return mix64(z)


def stream_base(seed: int, layer: int, expert: int, matrix: int, kind: int) -> int:
    if not (0 <= expert < (1 << 16) and 0 <= layer < (1 << 32)):
        raise ValueError("expert or layer index out of range")
    tag = (layer << 32) | (expert << 16) | (matrix << 8) | kind
    return mix64_int(mix64_int((seed + GAMMA) & M64) ^ tag)


# --------------------------------------------------------------------------- #
# rounding helpers (input construction only)
# --------------------------------------------------------------------------- #
def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------- #
# configurations (shapes from the pages; value distributions as stated above)
# --------------------------------------------------------------------------- #
@dataclasses.dataclass(frozen=True)
class Dims:
    hidden: int
    ffn: int
    n_experts: int
    top_k: int
    bits: int
    group_size: int = GROUP
    rms_eps: float = 1e-6

    def matrix_shape(self, m: int):
        return (self.ffn, self.hidden) if m in (GATE, UP) else (self.hidden, self.ffn)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dims: Dims
    n_tokens: int = 1
    n_layers: int = 1
    seed: int = 0
    description: str = ""


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", Dims(256, 128, 8, 2, 4), 1, 1, 0,
                     "hidden 256, FFN 128, 8 experts + shared, top-2, 4-bit"),
    "layer4": Workload("layer4", Dims(4096, 1024, 512, 4, 4), 1, 1, 0,
                       "hidden 4096, FFN 1024, 512 experts + shared, top-4, 4-bit, 1 token"),
    "layer2": Workload("layer2", Dims(4096, 1024, 512, 4, 2), 1, 1, 0,
                       "hidden 4096, FFN 1024, 512 experts + shared, top-4, 2-bit, 1 token"),
    "stack60": Workload("stack60", Dims(4096, 1024, 512, 4, 4), 1, 60, 0,
                        "60 chained 4-bit layers of hidden 4096 / FFN 1024 / 512 experts, top-4, 1 token"),
    "batch32": Workload("batch32", Dims(4096, 1024, 512, 10, 4), 32, 1, 0,
                        "32 tokens, hidden 4096, FFN 1024, 512 4-bit experts, top-10 + shared"),
    "tier4": Workload("tier4", Dims(4096, 1024, 512, 4, 4), 1, 4, 0,
                      "4 chained 4-bit layers of hidden 4096 / FFN 1024 / 512 experts, top-4, 1 token, "
                      "experts in pinned host memory behind an LRU cache of device slots"),
}


# --------------------------------------------------------------------------- #
# expert weights (canonical form: one code per byte, bf16 scale/bias bits)
# --------------------------------------------------------------------------- #
def matrix_codes(seed: int, layer: int, expert: int, matrix: int, rows: int, cols: int,
                 bits: int) -> np.ndarray:
    n = rows * cols
    per_word = 64 // bits
    nwords = (n + per_word - 1) // per_word
    words = splitmix64(stream_base(seed, layer, expert, matrix, KIND_CODES), nwords)
    by = words.astype("<u8").view(np.uint8)
    if bits == 4:
        codes = np.empty(2 * by.size, dtype=np.uint8)
        codes[0::2] = by & 0x0F
        codes[1::2] = by >> 4
    elif bits == 2:
        codes = np.empty(4 * by.size, dtype=np.uint8)
        for c in range(4):
            codes[c::4] = (by >> (2 * c)) & 0x03
    else:
        raise ValueError("bits must be 2 or 4")
    return codes[:n].reshape(rows, cols)


def _uniform24(words: np.ndarray) -> np.ndarray:
    return (words >> np.uint64(40)).astype(np.float64) * (2.0 ** -24)


def matrix_scale_bias(seed: int, layer: int, expert: int, matrix: int, rows: int, cols: int,
                      group: int = GROUP):
    ng = rows * (cols // group)
    us = _uniform24(splitmix64(stream_base(seed, layer, expert, matrix, KIND_SCALE), ng))
    ub = _uniform24(splitmix64(stream_base(seed, layer, expert, matrix, KIND_BIAS), ng))
    s64 = np.multiply(0.015, us)
    s64 = np.add(s64, 0.005)
    b64 = np.multiply(0.1, ub)
    b64 = np.subtract(b64, 0.1)
    s = f32_to_bf16_bits(s64.astype(np.float32)).reshape(rows, cols // group)
    b = f32_to_bf16_bits(b64.astype(np.float32)).reshape(rows, cols // group)
    return s, b


def expert_canonical(seed: int, layer: int, expert: int, dims: Dims) -> Dict[str, List[np.ndarray]]:
    """Canonical tensors of one expert: codes u8[rows][cols], scale/bias bf16 bits
    u16[rows][cols/64] for gate, up and down."""
    out = {"codes": [], "scale": [], "bias": []}
    for m in (GATE, UP, DOWN):
        rows, cols = dims.matrix_shape(m)
        out["codes"].append(matrix_codes(seed, layer, expert, m, rows, cols, dims.bits))
        s, b = matrix_scale_bias(seed, layer, expert, m, rows, cols, dims.group_size)
        out["scale"].append(s)
        out["bias"].append(b)
    return out


# --------------------------------------------------------------------------- #
# dense per-layer tensors and activations (host numpy generators)
# --------------------------------------------------------------------------- #
def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def layer_dense(seed: int, layer: int, dims: Dims) -> Dict[str, np.ndarray]:
    """RMSNorm weight, router matrix and shared-expert gate vector of one layer,
    as bf16 bit patterns (uint16)."""
    H, E = dims.hidden, dims.n_experts
    gamma = _rng(seed, layer, 1).uniform(0.5, 1.5, size=H).astype(np.float32)
    router = _rng(seed, layer, 2).normal(0.0, 0.02, size=(E, H)).astype(np.float32)
    sgate = _rng(seed, layer, 3).normal(0.0, 0.02, size=H).astype(np.float32)
    return {
        "norm_weight": f32_to_bf16_bits(gamma),
        "router_weight": f32_to_bf16_bits(router).reshape(E, H),
        "shared_gate": f32_to_bf16_bits(sgate),
    }


def tokens(seed: int, n: int, hidden: int, pool: int = 0) -> np.ndarray:
    """n activation vectors x ~ N(0, 1), fp32 [n][hidden]."""
    return _rng(seed, 7, pool).standard_normal(size=(n, hidden), dtype=np.float32)


# --------------------------------------------------------------------------- #
# GatedDeltaNet state update (the linear-attention layers: 64 heads, 128 x 128)
# --------------------------------------------------------------------------- #
def gdn_inputs(seed: int, n_heads: int, d: int, n_tokens: int, layer: int = 0) -> Dict[str, np.ndarray]:
    """Inputs of the state update, fp32: state [heads][d][d] ~ N(0, 0.05);
    q, k [tokens][heads][d] ~ N(0, 1) then unit L2 norm per head (q also scaled
    by d^-1/2), as the model feeds them; v [tokens][heads][d] ~ N(0, 1);
    alpha [tokens][heads] ~ U(0.9, 1) (a gate's decay close to one); beta ~ U(0, 1)."""
    r = _rng(seed, 11, layer)
    state = r.normal(0.0, 0.05, (n_heads, d, d)).astype(np.float32)
    q = r.standard_normal((n_tokens, n_heads, d)).astype(np.float32)
    k = r.standard_normal((n_tokens, n_heads, d)).astype(np.float32)
    q = (q / np.linalg.norm(q, axis=-1, keepdims=True) / np.sqrt(d)).astype(np.float32)
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    v = r.standard_normal((n_tokens, n_heads, d)).astype(np.float32)
    alpha = r.uniform(0.9, 1.0, (n_tokens, n_heads)).astype(np.float32)
    beta = r.uniform(0.0, 1.0, (n_tokens, n_heads)).astype(np.float32)
    return {"state": state, "q": q, "k": k, "v": v, "alpha": alpha, "beta": beta}
