"""Device-resident layer weights for the C ABI (marshalling only).

Holds the torch tensors that own a layer's device memory and the matching
``moe_layer_t`` descriptor.  Experts are either packed on the device from
canonical tensors (``moe_pack_expert``) or generated on the device from a seed
(``moe_generate_layer``); no quantisation arithmetic happens here.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from . import (make_layer, moe_expert_bytes, moe_generate_layer, moe_pack_expert, moe_layer_t)


def _u16(a: np.ndarray, device) -> torch.Tensor:
    """bf16 bit patterns (uint16) as an int16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(device)


class LayerWeights:
    """norm weight, router, shared gate (bf16 bits) + packed experts on one device."""

    def __init__(self, dims, dense: Dict[str, np.ndarray], device="cuda"):
        self.dims = dims
        self.device = torch.device(device)
        self.expert_bytes = moe_expert_bytes(dims)
        if self.expert_bytes == 0:
            raise ValueError("unsupported dims")
        self.norm_weight = _u16(dense["norm_weight"], self.device)
        self.router_weight = _u16(dense["router_weight"], self.device)
        self.shared_gate = _u16(dense["shared_gate"], self.device)
        self.experts = torch.empty(dims.n_experts * self.expert_bytes, dtype=torch.uint8, device=self.device)
        self.shared = torch.empty(self.expert_bytes, dtype=torch.uint8, device=self.device)

    def expert_view(self, e: int) -> torch.Tensor:
        """Packed bytes of routed expert e (e == n_experts: the shared expert)."""
        if e == self.dims.n_experts:
            return self.shared
        return self.experts[e * self.expert_bytes:(e + 1) * self.expert_bytes]

    def pack(self, e: int, canon: Dict[str, List[np.ndarray]], stream=None) -> None:
        """Pack one expert from canonical host tensors (copied to the device first)."""
        codes = [torch.from_numpy(np.ascontiguousarray(c, np.uint8)).to(self.device) for c in canon["codes"]]
        scale = [_u16(s, self.device) for s in canon["scale"]]
        bias = [_u16(b, self.device) for b in canon["bias"]]
        # staging tensors come from torch's stream-ordered allocator on the
        # current stream, so freeing them after the enqueue is safe
        moe_pack_expert(self.dims, codes, scale, bias, self.expert_view(e), stream)

    def generate(self, seed: int, layer: int, stream=None) -> None:
        moe_generate_layer(self.dims, seed, layer, self.experts, self.shared, stream)

    def descriptor(self) -> moe_layer_t:
        return make_layer(self.norm_weight, self.router_weight, self.shared_gate, self.experts, self.shared)


def layer_from_canonical(dims, dense, experts: Sequence[Dict[str, List[np.ndarray]]], device="cuda") -> LayerWeights:
    """E+1 canonical experts (last = shared) packed on the device."""
    lw = LayerWeights(dims, dense, device)
    for e, ex in enumerate(experts):
        lw.pack(e, ex)
    return lw


def layer_generated(dims, dense, seed: int, layer: int, device="cuda") -> LayerWeights:
    lw = LayerWeights(dims, dense, device)
    lw.generate(seed, layer)
    return lw
