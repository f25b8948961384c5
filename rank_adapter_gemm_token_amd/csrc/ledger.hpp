// ledger.hpp -- host-side slot states and per-tenant byte ledger of one pool.
//
// Pure C++ (no HIP), so it is unit-tested on the CPU.  Semantics follow
// xpshop.cn article 492, section 三 (a tenant's memory quota is a hard
// boundary: an over-quota mount is refused and never evicts anyone; unload
// drains first) and "Multi-LoRA 在线服务隔离", memory-accounting section
// (reserve the bytes before loading; never unload weights still in use).
//
// Slot life cycle:  FREE --begin_register--> LOADING --commit--> ACTIVE
//                   LOADING --abort--> FREE (bytes returned)
//                   ACTIVE --begin_unregister--> DRAINING --finish--> FREE
#pragma once

#include <cstddef>
#include <cstdint>
#include <map>
#include <vector>

namespace lora {

enum class SlotState : int { Free = 0, Loading = 1, Active = 2, Draining = 3 };

struct SlotRecord {
    SlotState state = SlotState::Free;
    int32_t tenant = -1;
    int rank = 0;
    float alpha = 0.0f;
    uint64_t bytes = 0;
};

class SlotBook {
public:
    SlotBook(int n_slots, int max_rank, uint64_t slot_bytes);

    // Returns LORA_OK or LORA_EINVAL (tenant < 0).
    int set_quota(int32_t tenant, uint64_t bytes);

    // Checks, then reserves the slot's bytes against the tenant's quota and
    // moves the slot to LOADING.  Returns LORA_OK, LORA_EINVAL, LORA_ESLOT_BUSY,
    // LORA_ERANK, LORA_EALPHA or LORA_EQUOTA; on error nothing changes.
    int begin_register(int slot, int32_t tenant, int rank, float alpha);
    void commit_register(int slot);  // LOADING -> ACTIVE
    void abort_register(int slot);   // LOADING -> FREE, bytes returned

    // ACTIVE -> DRAINING.  Returns LORA_OK, LORA_EINVAL or LORA_ESLOT_EMPTY.
    int begin_unregister(int slot);
    void finish_unregister(int slot);  // DRAINING -> FREE, bytes returned
    void cancel_unregister(int slot);  // DRAINING -> ACTIVE

    uint64_t tenant_used(int32_t tenant) const;
    uint64_t tenant_quota(int32_t tenant) const;
    uint64_t resident_bytes() const { return resident_; }
    int count(SlotState s) const;
    const SlotRecord &slot(int i) const { return slots_[static_cast<size_t>(i)]; }
    int n_slots() const { return static_cast<int>(slots_.size()); }
    uint64_t slot_bytes() const { return slot_bytes_; }

private:
    struct Account {
        uint64_t quota = 0;
        uint64_t used = 0;
    };
    std::vector<SlotRecord> slots_;
    std::map<int32_t, Account> tenants_;
    int max_rank_;
    uint64_t slot_bytes_;
    uint64_t resident_ = 0;
};

}  // namespace lora
