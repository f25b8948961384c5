// residency.cpp -- LRU-K residency with per-tenant shares (pure C++).
#include "residency.hpp"

#include "../../include/lora.h"

namespace lora {

Residency::Residency(int n_slots, int k)
    : slots_(static_cast<size_t>(n_slots > 0 ? n_slots : 0)), k_(k < 1 ? 1 : k) {}

void Residency::set_usable(int slot, bool usable) {
    if (slot >= 0 && slot < n_slots()) slots_[static_cast<size_t>(slot)].usable = usable;
}

int Residency::set_share(int32_t tenant, int max_slots) {
    if (tenant < 0 || max_slots < 0) return LORA_EINVAL;
    share_[tenant] = max_slots;
    return LORA_OK;
}

void Residency::touch(Entry &e) {
    e.hist.push_back(++clock_);
    while (static_cast<int>(e.hist.size()) > k_) e.hist.pop_front();
}

int Residency::acquire(uint64_t id, int32_t tenant, Decision *d) {
    if (tenant < 0 || d == nullptr) return LORA_EINVAL;
    *d = Decision{};
    auto w = where_.find(id);
    if (w != where_.end()) {
        Entry &e = slots_[static_cast<size_t>(w->second)];
        if (e.tenant != tenant) return LORA_EINVAL;
        ++e.refs;
        touch(e);
        ++hits;
        d->slot = w->second;
        d->hit = true;
        return LORA_OK;
    }
    const auto sh = share_.find(tenant);
    const auto ct = count_.find(tenant);
    const int held = (ct == count_.end()) ? 0 : ct->second;
    const bool at_share = (sh != share_.end()) && held >= sh->second;
    if (at_share && held == 0) return LORA_ESLOT_BUSY;  // a share of zero slots
    int pick = -1;
    if (!at_share) {
        for (int s = 0; s < n_slots(); ++s) {
            const Entry &e = slots_[static_cast<size_t>(s)];
            if (e.usable && !e.full) {
                pick = s;
                break;
            }
        }
    }
    if (pick < 0) {
        // LRU-K victim: the largest backward k-distance, i.e. the oldest k-th
        // most recent access; fewer than k accesses counts as infinitely old.
        // Ties: the least recent last access.  Only unreferenced slots, and
        // only the tenant's own when it is at its share.
        bool have = false;
        uint64_t best_k = 0, best_last = 0;
        for (int s = 0; s < n_slots(); ++s) {
            const Entry &e = slots_[static_cast<size_t>(s)];
            if (!e.usable || !e.full || e.refs > 0) continue;
            if (at_share && e.tenant != tenant) continue;
            const uint64_t kth = (static_cast<int>(e.hist.size()) < k_) ? 0 : e.hist.front();
            const uint64_t last = e.hist.empty() ? 0 : e.hist.back();
            if (!have || kth < best_k || (kth == best_k && last < best_last)) {
                have = true;
                best_k = kth;
                best_last = last;
                pick = s;
            }
        }
        if (pick < 0) return LORA_ESLOT_BUSY;
        Entry &v = slots_[static_cast<size_t>(pick)];
        d->evict = true;
        d->victim = v.id;
        d->victim_tenant = v.tenant;
        where_.erase(v.id);
        --count_[v.tenant];
        ++evictions;
    }
    Entry &e = slots_[static_cast<size_t>(pick)];
    e.full = true;
    e.id = id;
    e.tenant = tenant;
    e.refs = 1;
    e.hist.clear();
    touch(e);
    where_[id] = pick;
    ++count_[tenant];
    ++misses;
    d->slot = pick;
    return LORA_OK;
}

void Residency::abandon(int slot) {
    if (slot < 0 || slot >= n_slots()) return;
    Entry &e = slots_[static_cast<size_t>(slot)];
    if (!e.full) return;
    where_.erase(e.id);
    --count_[e.tenant];
    e = Entry{e.usable};
}

int Residency::release(uint64_t id) {
    auto w = where_.find(id);
    if (w == where_.end()) return LORA_EINVAL;
    Entry &e = slots_[static_cast<size_t>(w->second)];
    if (e.refs <= 0) return LORA_EINVAL;
    --e.refs;
    return LORA_OK;
}

int Residency::slot_of(uint64_t id) const {
    auto w = where_.find(id);
    return w == where_.end() ? -1 : w->second;
}

int Residency::refs(int slot) const {
    return (slot < 0 || slot >= n_slots()) ? 0 : slots_[static_cast<size_t>(slot)].refs;
}

int Residency::occupied() const {
    int n = 0;
    for (const Entry &e : slots_) n += e.full ? 1 : 0;
    return n;
}

int Residency::resident(int32_t tenant) const {
    auto c = count_.find(tenant);
    return c == count_.end() ? 0 : c->second;
}

}  // namespace lora
