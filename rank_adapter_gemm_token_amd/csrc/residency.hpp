// residency.hpp -- which adapters stay resident in a pool's slots when slots
// run out: LRU-K eviction among unreferenced slots, within per-tenant
// resident shares.
//
// "LLM 多 LoRA 推理服务工程 2026", four-layer runtime, storage-pool paragraph:
// moves between the hot (HBM) tier and the tiers below follow LRU-K over the
// recent accesses.  "Multi-LoRA 在线服务隔离", memory-accounting section: at
// the watermark, evict the version that has no live reference and was used
// least recently, never weights a request still holds, and give each tenant
// a resident share so one tenant cannot push every other adapter out.
//
// Pure C++ (no HIP), so it is unit-tested on the CPU; the pool wrapper in
// api.cpp unloads the victims and starts the loads it decides.
#pragma once

#include <cstddef>
#include <cstdint>
#include <deque>
#include <map>
#include <unordered_map>
#include <vector>

namespace lora {

class Residency {
public:
    // n_slots slots, all unusable until set_usable; k >= 1 accesses of history.
    Residency(int n_slots, int k);

    // Slots the manager may fill and evict (those free when it took the pool).
    void set_usable(int slot, bool usable);

    // Cap on the slots a tenant's adapters may hold at once (no cap if unset).
    // LORA_OK, LORA_EINVAL (tenant < 0 or max_slots < 0).
    int set_share(int32_t tenant, int max_slots);

    struct Decision {
        int slot = -1;
        bool hit = false;           // resident already: nothing to load
        bool evict = false;         // the slot holds `victim`, to be unloaded first
        uint64_t victim = 0;
        int32_t victim_tenant = -1;
    };

    // Adapter `id` of `tenant` for one more holder.  A resident adapter is a
    // hit (one more reference).  Otherwise the slot to load it into: a free
    // usable slot if the tenant is within its share, else the LRU-K victim
    // among unreferenced slots -- the tenant's own when it is at its share.
    // The miss is recorded as resident with one reference.
    // LORA_OK, LORA_EINVAL (tenant < 0, or id resident for another tenant),
    // LORA_ESLOT_BUSY (no slot may be taken; nothing changes).
    int acquire(uint64_t id, int32_t tenant, Decision *d);

    // Undo a miss whose load failed: the slot is left empty.
    void abandon(int slot);

    // One holder fewer.  LORA_OK, LORA_EINVAL (not resident or no holder).
    int release(uint64_t id);

    int slot_of(uint64_t id) const;    // -1 when not resident
    int refs(int slot) const;
    int resident(int32_t tenant) const;
    int occupied() const;  // slots holding an adapter
    int n_slots() const { return static_cast<int>(slots_.size()); }

    uint64_t hits = 0, misses = 0, evictions = 0;

private:
    struct Entry {
        bool usable = false;
        bool full = false;
        uint64_t id = 0;
        int32_t tenant = -1;
        int refs = 0;
        std::deque<uint64_t> hist;  // the last k access times, oldest first
    };
    void touch(Entry &e);
    std::vector<Entry> slots_;
    std::unordered_map<uint64_t, int> where_;
    std::map<int32_t, int> share_;
    std::map<int32_t, int> count_;
    int k_;
    uint64_t clock_ = 0;
};

}  // namespace lora
