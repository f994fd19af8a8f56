"""The library's cache bookkeeping (csrc/moe_tier.h, host C++) against the LRU
oracle: the header is compiled with g++ into a small test shim (no HIP), then
driven with access sequences; the hits and the cached set must equal those of
oracle/lru.py, and the slot map must stay a bijection between cached keys and
occupied slots."""
import ctypes
import os
import random
import subprocess

import numpy as np
import pytest

from oracle.lru import lru_run

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_dequant_expert_router_amd", "csrc")

SHIM = r"""
#include "moe_tier.h"
extern "C" {
size_t shim_ints(int ns, int nk) { return moe::SlotLru::ints(ns, nk); }
// runs n accesses; hit[i], slot[i] per access; lru state in mem; returns head
int shim_run(int ns, int nk, int32_t *mem, int init, const int32_t *keys, int n, int32_t *hit, int32_t *slot,
             int32_t *ends) {
    moe::SlotLru l;
    if (init) {
        l.init(ns, nk, mem);
    } else {
        l.n_slots = ns; l.n_keys = nk; l.key = mem; l.prev = mem + ns; l.next = mem + 2 * ns;
        l.slot_of = mem + 3 * ns; l.head = ends[0]; l.tail = ends[1];
    }
    for (int i = 0; i < n; ++i) {
        bool h;
        slot[i] = l.acquire(keys[i], &h);
        hit[i] = h;
    }
    ends[0] = l.head;
    ends[1] = l.tail;
    return 0;
}
}
"""


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    d = tmp_path_factory.mktemp("tier_shim")
    src = d / "shim.cpp"
    src.write_text(SHIM)
    so = d / "libshim.so"
    subprocess.check_call(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-I", CSRC, str(src), "-o", str(so)])
    lib = ctypes.CDLL(str(so))
    lib.shim_ints.restype = ctypes.c_size_t
    lib.shim_ints.argtypes = [ctypes.c_int, ctypes.c_int]
    return lib


class Lru:
    def __init__(self, lib, ns, nk):
        self.lib, self.ns, self.nk = lib, ns, nk
        self.mem = np.zeros(lib.shim_ints(ns, nk), np.int32)
        self.ends = np.zeros(2, np.int32)
        self.started = False

    def run(self, keys):
        keys = np.asarray(keys, np.int32)
        hit = np.zeros(len(keys), np.int32)
        slot = np.zeros(len(keys), np.int32)
        p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
        self.lib.shim_run(self.ns, self.nk, p(self.mem), 0 if self.started else 1, p(keys), len(keys), p(hit),
                          p(slot), p(self.ends))
        self.started = True
        return hit.astype(bool).tolist(), slot.tolist()

    def check_maps(self):
        ns = self.ns
        key, prev, nxt, slot_of = (self.mem[:ns], self.mem[ns:2 * ns], self.mem[2 * ns:3 * ns], self.mem[3 * ns:])
        for k in range(self.nk):
            if slot_of[k] >= 0:
                assert key[slot_of[k]] == k
        for s in range(ns):
            if key[s] >= 0:
                assert slot_of[key[s]] == s
        # the list visits every slot once, head to tail, with consistent back links
        order, s, last = [], int(self.ends[0]), -1
        while s >= 0:
            assert prev[s] == last
            order.append(s)
            last, s = s, int(nxt[s])
        assert last == self.ends[1] and sorted(order) == list(range(ns))
        return [int(key[s]) for s in reversed(order) if key[s] >= 0]  # least recently used first


def test_textbook_string(shim):
    seq = [7, 0, 1, 2, 0, 3, 0, 4, 2, 3, 0, 3, 2, 1, 2, 0, 1, 7, 0, 1]
    lru = Lru(shim, 3, 8)
    hits, slots = lru.run(seq)
    assert hits.count(False) == 12
    assert lru.check_maps() == [7, 0, 1]
    assert slots[:3] == [2, 1, 0]  # empty slots are taken before any is reused


@pytest.mark.parametrize("seed", range(8))
def test_against_oracle(shim, seed):
    rng = random.Random(seed)
    nk = rng.choice([4, 16, 64, 300])
    ns = rng.randrange(1, nk + 3)
    lru = Lru(shim, ns, nk)
    state = None
    # several calls continuing one state, with a skewed key popularity
    for call in range(6):
        seq = [min(int(rng.expovariate(3.0 / nk)), nk - 1) for _ in range(rng.randrange(1, 60))]
        want, state = lru_run(seq, ns, state)
        got, slots = lru.run(seq)
        assert got == want, (seed, call)
        assert lru.check_maps() == list(state)
        # a slot handed out on a hit is the slot the key already had
        seen = {}
        for k, h, s in zip(seq, got, slots):
            if h and k in seen:
                assert seen[k] == s
            seen[k] = s


def test_one_slot(shim):
    lru = Lru(shim, 1, 5)
    hits, slots = lru.run([3, 3, 4, 3])
    assert hits == [False, True, False, False] and slots == [0, 0, 0, 0]
    assert lru.check_maps() == [3]
