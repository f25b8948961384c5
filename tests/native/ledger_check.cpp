// ledger_check.cpp -- CPU unit test of the pool's slot book and tenant ledger
// (compiled with g++ by tests/test_host_cpu.py; no HIP).
#include <cmath>
#include <cstdio>
#include <cstdlib>

#include "../../include/lora.h"
#include "../../rank_adapter_gemm_token_amd/csrc/ledger.hpp"

static int failures = 0;
#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                               \
        }                                                             \
    } while (0)

using lora::SlotBook;
using lora::SlotState;

int main() {
    const uint64_t SB = 1000;  // bytes per slot
    SlotBook b(4, 16, SB);

    // Default deny: a tenant without a quota cannot register.
    CHECK(b.begin_register(0, 7, 8, 16.0f) == LORA_EQUOTA);
    CHECK(b.slot(0).state == SlotState::Free);
    CHECK(b.tenant_used(7) == 0);

    CHECK(b.set_quota(-1, 10) == LORA_EINVAL);
    CHECK(b.set_quota(7, 2 * SB) == LORA_OK);
    CHECK(b.set_quota(9, 5 * SB) == LORA_OK);

    // Argument checks, nothing reserved on error.
    CHECK(b.begin_register(-1, 7, 8, 16.0f) == LORA_EINVAL);
    CHECK(b.begin_register(4, 7, 8, 16.0f) == LORA_EINVAL);
    CHECK(b.begin_register(0, -3, 8, 16.0f) == LORA_EINVAL);
    CHECK(b.begin_register(0, 7, 0, 16.0f) == LORA_ERANK);
    CHECK(b.begin_register(0, 7, 17, 16.0f) == LORA_ERANK);
    CHECK(b.begin_register(0, 7, 8, NAN) == LORA_EALPHA);
    CHECK(b.begin_register(0, 7, 8, INFINITY) == LORA_EALPHA);
    CHECK(b.tenant_used(7) == 0 && b.resident_bytes() == 0);

    // Reserve before copy; commit; busy slot.
    CHECK(b.begin_register(0, 7, 8, 16.0f) == LORA_OK);
    CHECK(b.slot(0).state == SlotState::Loading);
    CHECK(b.tenant_used(7) == SB);
    CHECK(b.begin_register(0, 9, 8, 16.0f) == LORA_ESLOT_BUSY);
    b.commit_register(0);
    CHECK(b.slot(0).state == SlotState::Active);
    CHECK(b.begin_register(0, 9, 8, 16.0f) == LORA_ESLOT_BUSY);

    // Hard quota: tenant 7 fits exactly two slots; the third is refused and
    // nothing of tenant 9 is touched (never evict another tenant).
    CHECK(b.begin_register(2, 9, 4, 8.0f) == LORA_OK);
    b.commit_register(2);
    CHECK(b.begin_register(1, 7, 16, 32.0f) == LORA_OK);
    b.commit_register(1);
    CHECK(b.tenant_used(7) == 2 * SB);
    CHECK(b.begin_register(3, 7, 8, 16.0f) == LORA_EQUOTA);
    CHECK(b.slot(3).state == SlotState::Free);
    CHECK(b.slot(2).state == SlotState::Active && b.tenant_used(9) == SB);
    CHECK(b.resident_bytes() == 3 * SB);

    // Aborted load returns the bytes.
    CHECK(b.begin_register(3, 9, 8, 16.0f) == LORA_OK);
    CHECK(b.tenant_used(9) == 2 * SB);
    b.abort_register(3);
    CHECK(b.slot(3).state == SlotState::Free && b.tenant_used(9) == SB);

    // Drain: ACTIVE -> DRAINING -> FREE; bytes come back only at the end.
    CHECK(b.begin_unregister(3) == LORA_ESLOT_EMPTY);
    CHECK(b.begin_unregister(9) == LORA_EINVAL);
    CHECK(b.begin_unregister(1) == LORA_OK);
    CHECK(b.slot(1).state == SlotState::Draining);
    CHECK(b.tenant_used(7) == 2 * SB);
    CHECK(b.begin_register(1, 9, 8, 16.0f) == LORA_ESLOT_BUSY);  // never reuse a draining slot
    CHECK(b.begin_unregister(1) == LORA_ESLOT_EMPTY);
    b.finish_unregister(1);
    CHECK(b.slot(1).state == SlotState::Free && b.tenant_used(7) == SB);

    // A cancelled drain keeps the adapter.
    CHECK(b.begin_unregister(0) == LORA_OK);
    b.cancel_unregister(0);
    CHECK(b.slot(0).state == SlotState::Active && b.tenant_used(7) == SB);

    // Lowering a quota below use evicts nothing but refuses new registers.
    CHECK(b.set_quota(7, 0) == LORA_OK);
    CHECK(b.slot(0).state == SlotState::Active && b.tenant_used(7) == SB);
    CHECK(b.begin_register(1, 7, 8, 16.0f) == LORA_EQUOTA);

    // Accounting is exact: resident = sum of charged slot bytes.
    CHECK(b.resident_bytes() == b.tenant_used(7) + b.tenant_used(9));
    CHECK(b.count(SlotState::Active) == 2);

    std::printf("%s (%d failures)\n", failures ? "FAILED" : "OK", failures);
    return failures ? 1 : 0;
}
