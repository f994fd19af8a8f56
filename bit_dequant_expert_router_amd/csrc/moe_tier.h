// moe_tier.h -- bookkeeping of tiered expert residency: which device slot
// holds which (layer, expert), replaced least-recently-used.  Host code only
// (no HIP), in memory the caller provides.
//
// The pages leave the cache to the operating system's page cache, whose
// replacement is least-recently-used ("48GB内存运行397B模型：Flash-Moe的极端量化
// 与SSD流式加载实践", section "SSD流式加载：绕过统一内存瓶颈"; mxp.tw reading
// notes on the SSD streaming design).  Here the cache unit is one packed
// expert of one layer and the key is layer * n_experts + expert.
#ifndef MOE_TIER_H
#define MOE_TIER_H

#include <stddef.h>
#include <stdint.h>

namespace moe {

// An intrusive doubly linked list over the slots, most recently used at the
// head, and a key -> slot map.  Every operation is O(1).
struct SlotLru {
    int32_t n_slots = 0, n_keys = 0;
    int32_t head = -1, tail = -1;
    int32_t *key = nullptr;      // [n_slots] key the slot holds, -1 = empty
    int32_t *prev = nullptr;     // [n_slots] neighbour towards the head, -1 at the head
    int32_t *next = nullptr;     // [n_slots] neighbour towards the tail, -1 at the tail
    int32_t *slot_of = nullptr;  // [n_keys]  slot holding the key, -1 = not cached

    static size_t ints(int32_t ns, int32_t nk) { return 3 * (size_t)ns + (size_t)nk; }

    // Every slot empty.  Empty slots start at the tail side and are taken
    // before any slot is reused.  mem: ints(ns, nk) int32s.
    void init(int32_t ns, int32_t nk, int32_t *mem) {
        n_slots = ns;
        n_keys = nk;
        key = mem;
        prev = key + ns;
        next = prev + ns;
        slot_of = next + ns;
        for (int32_t i = 0; i < ns; ++i) {
            key[i] = -1;
            prev[i] = i - 1;
            next[i] = i + 1 < ns ? i + 1 : -1;
        }
        head = 0;
        tail = ns - 1;
        for (int32_t k = 0; k < nk; ++k) slot_of[k] = -1;
    }

    // Make slot s the most recently used.
    void touch(int32_t s) {
        if (s == head) return;
        const int32_t p = prev[s], n = next[s];  // p >= 0: s is not the head
        next[p] = n;
        if (n >= 0) prev[n] = p;
        else tail = p;
        prev[s] = -1;
        next[s] = head;
        prev[head] = s;
        head = s;
    }

    // The slot for key k, made most recently used.  *hit: k was cached.  On a
    // miss the least recently used slot is handed to k and its former key, if
    // any, is dropped; the caller fills the slot.
    int32_t acquire(int32_t k, bool *hit) {
        int32_t s = slot_of[k];
        *hit = s >= 0;
        if (s < 0) {
            s = tail;
            if (key[s] >= 0) slot_of[key[s]] = -1;
            key[s] = k;
            slot_of[k] = s;
        }
        touch(s);
        return s;
    }
};

}  // namespace moe

#endif  // MOE_TIER_H
