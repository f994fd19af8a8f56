"""Expert-cache policy of tiered residency, as a plain LRU -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares no code with the GPU library.

What it models.  The pages keep every expert on SSD and read the K selected
experts of a layer after routing, relying on the operating system's page cache
(least-recently-used replacement) to keep recently read experts in memory, at
about 71% hits on their workload ("48GB内存运行397B模型：Flash-Moe的极端量化与SSD
流式加载实践", section "SSD流式加载：绕过统一内存瓶颈"; mxp.tw reading notes,
section on the SSD streaming design, where the page cache's LRU is named as
the key).  Tiered residency moves the same idea one level up: HBM holds
``capacity`` experts, the backing store is host memory, and the cache unit is
one whole expert of one layer, keyed by (layer, expert).

Reading taken where the pages leave it open: the accesses of one call are made
in token order, and within a token in rank order (the order of its top-K
list); an expert selected twice in one call is a miss at most once.

Parity status: pinned (tests/test_tier_oracle.py) by textbook page-reference
strings with known LRU fault counts, by the stack-distance characterisation
of LRU (brute force) and by the inclusion property.
"""
from __future__ import annotations

from collections import OrderedDict
from typing import Iterable, List, Sequence, Tuple


def lru_run(accesses: Iterable[int], capacity: int, state: "OrderedDict | None" = None
            ) -> Tuple[List[bool], "OrderedDict"]:
    """Replay ``accesses`` through an LRU cache of ``capacity`` entries.

    Returns (hit per access, the cache afterwards ordered least to most
    recently used).  ``state`` continues a previous run (it is updated).
    """
    if capacity < 1:
        raise ValueError("capacity must be at least 1")
    cache = OrderedDict() if state is None else state
    hits = []
    for key in accesses:
        if key in cache:
            cache.move_to_end(key)
            hits.append(True)
        else:
            if len(cache) >= capacity:
                cache.popitem(last=False)  # the least recently used entry
            cache[key] = True
            hits.append(False)
    return hits, cache


def layer_accesses(layer: int, route_idx: Sequence[Sequence[int]], n_experts: int) -> List[int]:
    """Cache keys one layer call touches: token order, then rank order."""
    return [layer * n_experts + int(e) for row in route_idx for e in row]
