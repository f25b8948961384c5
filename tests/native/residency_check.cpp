// residency_check.cpp -- CPU unit test of the LRU-K residency policy with
// per-tenant shares (compiled with g++ by tests/test_host_cpu.py; no HIP).
#include <cstdio>

#include "../../include/lora.h"
#include "../../rank_adapter_gemm_token_amd/csrc/residency.hpp"

static int failures = 0;
#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                               \
        }                                                             \
    } while (0)

using lora::Residency;

int main() {
    // 4 slots, slot 3 not usable (held outside the manager); k = 2.
    Residency r(4, 2);
    for (int s = 0; s < 3; ++s) r.set_usable(s, true);
    Residency::Decision d;

    // Misses fill the free usable slots in order.
    for (uint64_t id = 1; id <= 3; ++id) {
        CHECK(r.acquire(id, 0, &d) == LORA_OK);
        CHECK(!d.hit && !d.evict && d.slot == static_cast<int>(id - 1));
    }
    CHECK(r.misses == 3 && r.resident(0) == 3);
    // Every slot referenced: nothing may be evicted, nothing changes.
    CHECK(r.acquire(4, 0, &d) == LORA_ESLOT_BUSY);
    CHECK(r.misses == 3 && r.evictions == 0 && r.slot_of(4) == -1);
    // Hit: one more reference.
    CHECK(r.acquire(2, 0, &d) == LORA_OK && d.hit && d.slot == 1);
    CHECK(r.refs(1) == 2 && r.hits == 1);
    CHECK(r.acquire(2, 7, &d) == LORA_EINVAL);  // resident for another tenant
    CHECK(r.release(2) == LORA_OK && r.release(2) == LORA_OK);
    CHECK(r.release(2) == LORA_EINVAL);  // no holder left
    CHECK(r.release(99) == LORA_EINVAL);
    CHECK(r.release(1) == LORA_OK && r.release(3) == LORA_OK);

    // LRU-K (k = 2): id 1 has one access, ids 2 and 3 have two -> 1 goes first
    // although 1 is not the least recently used by its last access.
    CHECK(r.acquire(3, 0, &d) == LORA_OK && d.hit);  // 3: accesses t3, t5
    CHECK(r.release(3) == LORA_OK);
    CHECK(r.acquire(1, 0, &d) == LORA_OK && d.hit);  // 1: accesses t1, t6 (the latest)
    CHECK(r.release(1) == LORA_OK);
    // Now 1 (t1, t6), 2 (t2, t4), 3 (t3, t5): the 2nd most recent access is
    // oldest for 1 -> victim 1, although its last access is the latest.
    CHECK(r.acquire(4, 0, &d) == LORA_OK);
    CHECK(!d.hit && d.evict && d.victim == 1 && d.slot == 0 && r.evictions == 1);
    CHECK(r.slot_of(1) == -1 && r.slot_of(4) == 0);
    // 4 (t7) has one access (infinite k-distance) but is referenced: not a
    // victim.  Among 2 (t2, t4) and 3 (t3, t5): 2.
    CHECK(r.acquire(5, 0, &d) == LORA_OK && d.evict && d.victim == 2 && d.slot == 1);
    CHECK(r.release(4) == LORA_OK);
    // Unreferenced 4 (t7) and 5 (t8) have a single access each: both go
    // before 3 (two accesses); the older last access, 4, first.
    CHECK(r.release(5) == LORA_OK);
    CHECK(r.acquire(6, 0, &d) == LORA_OK && d.evict && d.victim == 4 && d.slot == 0);
    CHECK(r.release(6) == LORA_OK);

    // Shares.  Tenant 1 may hold one slot: the first miss evicts any
    // tenant's unreferenced slot; the second may only take its own.
    CHECK(r.set_share(-1, 1) == LORA_EINVAL && r.set_share(1, -1) == LORA_EINVAL);
    CHECK(r.set_share(1, 1) == LORA_OK);
    CHECK(r.acquire(10, 1, &d) == LORA_OK && d.evict && d.victim_tenant == 0);
    const int s10 = d.slot;
    CHECK(r.resident(1) == 1);
    CHECK(r.acquire(11, 1, &d) == LORA_ESLOT_BUSY);  // own slot still referenced
    CHECK(r.release(10) == LORA_OK);
    CHECK(r.acquire(11, 1, &d) == LORA_OK && d.evict && d.victim == 10 && d.slot == s10);
    CHECK(r.resident(1) == 1);
    CHECK(r.set_share(2, 0) == LORA_OK);
    CHECK(r.acquire(20, 2, &d) == LORA_ESLOT_BUSY);  // a share of zero slots
    CHECK(r.acquire(21, -1, &d) == LORA_EINVAL);

    // A failed load: the slot is left empty and is the next free one.
    CHECK(r.release(11) == LORA_OK);
    CHECK(r.acquire(30, 0, &d) == LORA_OK);
    const int s30 = d.slot;
    r.abandon(s30);
    CHECK(r.slot_of(30) == -1 && r.refs(s30) == 0);
    CHECK(r.acquire(31, 0, &d) == LORA_OK && !d.evict && d.slot == s30);

    // The slot outside the manager is never used.
    for (uint64_t id = 40; id < 60; ++id) {
        if (r.acquire(id, 0, &d) == LORA_OK) {
            CHECK(d.slot != 3);
            r.release(id);
        }
    }
    if (failures == 0) std::printf("residency: all checks passed\n");
    return failures == 0 ? 0 : 1;
}
