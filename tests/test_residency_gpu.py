"""Slot residency (lora_residency_*) on the GPU, through the C ABI: adapters
acquired by id land in the pool's free slots, evictions pick unreferenced
slots by LRU-K within tenant shares, and a slot reused for another adapter
computes that adapter's term (compared with the oracle)."""
import numpy as np
import pytest
import torch

from gpu_helpers import BIG_QUOTA, Pool, assert_close, dev, reference
from rank_adapter_gemm_token_amd import lora

pytestmark = pytest.mark.gpu

D_IN, D_OUT, R, T = 128, 128, 16, 24


def _adapter(seed, rank=8):
    rng = np.random.default_rng(seed)
    A = torch.from_numpy(rng.standard_normal((rank, D_IN)) / np.sqrt(D_IN)).to(torch.float16)
    B = torch.from_numpy(rng.standard_normal((D_OUT, rank)) * 0.1).to(torch.float16)
    return A, B, rank, 2.0 * rank


def _check_slot(p, slot, ad, seed):
    """Tokens naming `slot` get adapter `ad`'s term (oracle comparison)."""
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((T, D_IN))).to(torch.float16)
    W = torch.from_numpy(rng.standard_normal((D_OUT, D_IN)) / np.sqrt(D_IN)).to(torch.float16)
    idx = torch.full((T,), slot, dtype=torch.int32)
    idx[::5] = -1
    A, B, rank, alpha = ad
    p.adapters = {slot: (A, B, rank, alpha)}
    y = p.apply(dev(x), dev(W), dev(idx))
    torch.cuda.synchronize()
    y_ref, inv = reference(p, x, W, idx)
    assert_close(y.cpu(), y_ref, inv, "f16")


def test_acquire_evict_and_reuse():
    p = Pool(D_IN, D_OUT, R, 4, T, "f16", 0, 4)
    ld = lora.lora_loader_create(R * (D_IN + D_OUT) * 2)
    res = None
    try:
        # Slot 3 is registered outside the manager and is never touched.
        lora.lora_set_tenant_quota(p.h, 0, BIG_QUOTA)
        lora.lora_set_tenant_quota(p.h, 1, BIG_QUOTA)
        A3, B3, r3, a3 = _adapter(3)
        lora.lora_register(p.h, 3, 0, dev(A3), dev(B3), r3, a3)
        res = lora.lora_residency_create(p.h, ld, 2)
        ads = {i: _adapter(100 + i) for i in range(6)}
        slots = {}
        for i in range(3):
            s, t = lora.lora_residency_acquire(res, 1000 + i, 0, *ads[i])
            assert t != 0 and s != 3
            lora.lora_load_wait(ld, t)
            slots[i] = s
        assert sorted(slots.values()) == [0, 1, 2]
        for i in range(3):
            _check_slot(p, slots[i], ads[i], seed=i)
        # All three referenced: a fourth adapter finds no slot.
        with pytest.raises(lora.LoraError) as ei:
            lora.lora_residency_acquire(res, 1003, 0, *ads[3])
        assert ei.value.status == lora.LORA_ESLOT_BUSY
        # A hit returns the same slot and its ticket.
        s, t = lora.lora_residency_acquire(res, 1001, 0, None, None, 8, 16.0)
        assert s == slots[1]
        lora.lora_load_wait(ld, t)
        lora.lora_residency_release(res, 1001)
        # Release 1000 and 1002; 1002 used again (two accesses) -> LRU-K evicts
        # 1000 (one access) for the next miss.
        lora.lora_residency_release(res, 1000)
        lora.lora_residency_release(res, 1002)
        s, t = lora.lora_residency_acquire(res, 1002, 0, None, None, 8, 16.0)
        lora.lora_residency_release(res, 1002)
        s, t = lora.lora_residency_acquire(res, 1003, 0, *ads[3])
        assert s == slots[0]
        lora.lora_load_wait(ld, t)
        _check_slot(p, s, ads[3], seed=7)  # the reused slot holds the new adapter
        _check_slot(p, 3, (A3, B3, r3, a3), seed=8)  # the outside slot is intact
        st = lora.lora_residency_stats_read(res)
        assert st["misses"] == 4 and st["evictions"] == 1 and st["hits"] == 2
        assert st["resident"] == 3 and st["managed"] == 3
        # Tenant 1 with a share of one slot: its first adapter evicts an
        # unreferenced one of tenant 0, its second only its own.
        lora.lora_residency_set_share(res, 1, 1)
        s1, t1 = lora.lora_residency_acquire(res, 2000, 1, *ads[4])
        lora.lora_load_wait(ld, t1)
        with pytest.raises(lora.LoraError) as ei:
            lora.lora_residency_acquire(res, 2001, 1, *ads[5])
        assert ei.value.status == lora.LORA_ESLOT_BUSY
        lora.lora_residency_release(res, 2000)
        s2, t2 = lora.lora_residency_acquire(res, 2001, 1, *ads[5])
        assert s2 == s1
        lora.lora_load_wait(ld, t2)
        _check_slot(p, s2, ads[5], seed=9)
        assert lora.lora_tenant_bytes(p.h, 1) == lora.lora_pool_stats(p.h)["slot_bytes"]
    finally:
        if res is not None:
            lora.lora_residency_destroy(res)
        lora.lora_loader_destroy(ld)
        p.close()
