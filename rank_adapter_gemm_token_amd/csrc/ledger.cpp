// ledger.cpp -- slot states and per-tenant byte ledger (pure C++).
#include "ledger.hpp"

#include <cmath>

#include "../../include/lora.h"

namespace lora {

SlotBook::SlotBook(int n_slots, int max_rank, uint64_t slot_bytes)
    : slots_(static_cast<size_t>(n_slots > 0 ? n_slots : 0)),
      max_rank_(max_rank),
      slot_bytes_(slot_bytes) {}

int SlotBook::set_quota(int32_t tenant, uint64_t bytes) {
    if (tenant < 0) return LORA_EINVAL;
    tenants_[tenant].quota = bytes;
    return LORA_OK;
}

int SlotBook::begin_register(int slot, int32_t tenant, int rank, float alpha) {
    if (slot < 0 || slot >= n_slots() || tenant < 0) return LORA_EINVAL;
    SlotRecord &s = slots_[static_cast<size_t>(slot)];
    if (s.state != SlotState::Free) return LORA_ESLOT_BUSY;
    if (rank < 1 || rank > max_rank_) return LORA_ERANK;
    if (!std::isfinite(alpha)) return LORA_EALPHA;
    auto it = tenants_.find(tenant);
    // An unset quota is zero: default deny.
    const uint64_t quota = (it == tenants_.end()) ? 0 : it->second.quota;
    const uint64_t used = (it == tenants_.end()) ? 0 : it->second.used;
    if (used > quota || slot_bytes_ > quota - used) return LORA_EQUOTA;
    Account &a = tenants_[tenant];
    a.used += slot_bytes_;
    resident_ += slot_bytes_;
    s.state = SlotState::Loading;
    s.tenant = tenant;
    s.rank = rank;
    s.alpha = alpha;
    s.bytes = slot_bytes_;
    return LORA_OK;
}

void SlotBook::commit_register(int slot) {
    SlotRecord &s = slots_[static_cast<size_t>(slot)];
    if (s.state == SlotState::Loading) s.state = SlotState::Active;
}

void SlotBook::abort_register(int slot) {
    SlotRecord &s = slots_[static_cast<size_t>(slot)];
    if (s.state != SlotState::Loading) return;
    Account &a = tenants_[s.tenant];
    a.used -= s.bytes;
    resident_ -= s.bytes;
    s = SlotRecord();
}

int SlotBook::begin_unregister(int slot) {
    if (slot < 0 || slot >= n_slots()) return LORA_EINVAL;
    SlotRecord &s = slots_[static_cast<size_t>(slot)];
    if (s.state != SlotState::Active) return LORA_ESLOT_EMPTY;
    s.state = SlotState::Draining;
    return LORA_OK;
}

void SlotBook::finish_unregister(int slot) {
    SlotRecord &s = slots_[static_cast<size_t>(slot)];
    if (s.state != SlotState::Draining) return;
    Account &a = tenants_[s.tenant];
    a.used -= s.bytes;
    resident_ -= s.bytes;
    s = SlotRecord();
}

void SlotBook::cancel_unregister(int slot) {
    SlotRecord &s = slots_[static_cast<size_t>(slot)];
    if (s.state == SlotState::Draining) s.state = SlotState::Active;
}

uint64_t SlotBook::tenant_used(int32_t tenant) const {
    auto it = tenants_.find(tenant);
    return it == tenants_.end() ? 0 : it->second.used;
}

uint64_t SlotBook::tenant_quota(int32_t tenant) const {
    auto it = tenants_.find(tenant);
    return it == tenants_.end() ? 0 : it->second.quota;
}

int SlotBook::count(SlotState st) const {
    int n = 0;
    for (const SlotRecord &s : slots_) n += (s.state == st) ? 1 : 0;
    return n;
}

}  // namespace lora
