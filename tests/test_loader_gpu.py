"""The async host-to-slot loader (lora_loader_*, lora_load_*) on the GPU,
through the C ABI.

A slot loaded from host memory must hold exactly what lora_register puts
there from device memory: outputs of lora_apply on the two pools are equal
bit for bit (and lora_apply itself is compared with the oracle in
test_apply_gpu.py).  Also: double-buffer reuse over many loads, the LOADING
state until commit, and the register-time errors."""
import time

import numpy as np
import pytest
import torch

from gpu_helpers import BIG_QUOTA, Pool, assert_close, dev, reference
from rank_adapter_gemm_token_amd import lora
from test_apply_gpu import _small_case

pytestmark = pytest.mark.gpu


def _loaded_pool(ld, dtype, d_in, d_out, R, S, T, ads, policy=0):
    """A pool whose adapters arrive through the loader (host tensors)."""
    p = Pool(d_in, d_out, R, S, T, dtype, policy, 4)
    tickets = []
    for a in ads:
        lora.lora_set_tenant_quota(p.h, a.tenant, BIG_QUOTA)
        tickets.append(lora.lora_load_async(ld, p.h, a.slot, a.tenant, a.A.cpu().contiguous(),
                                            a.B.cpu().contiguous(), a.rank, a.alpha))
        p.adapters[a.slot] = (a.A.cpu(), a.B.cpu(), a.rank, a.alpha)
    return p, tickets


@pytest.mark.parametrize("dtype,T,d_in,d_out,S,R", [("f16", 37, 128, 192, 5, 8), ("bf16", 300, 256, 256, 7, 64),
                                                    ("f32", 20, 64, 64, 4, 16)])
def test_loaded_slots_equal_registered_slots(dtype, T, d_in, d_out, S, R):
    x, W, ads, idx = _small_case(dtype, T, d_in, d_out, S, R, seed=T + 3)
    esz = 4 if dtype == "f32" else 2
    ld = lora.lora_loader_create(R * (d_in + d_out) * esz)
    pr = Pool(d_in, d_out, R, S, T, dtype, 0, 4)
    pl = None
    try:
        pr.register_all(ads)
        pl, tickets = _loaded_pool(ld, dtype, d_in, d_out, R, S, T, ads)
        for t in tickets:
            lora.lora_load_wait(ld, t)
        assert lora.lora_pool_stats(pl.h)["active_slots"] == S
        yr = pr.apply(dev(x), dev(W), dev(idx))
        yl = pl.apply(dev(x), dev(W), dev(idx))
        torch.cuda.synchronize()
        g, w = yl.cpu(), yr.cpu()
        assert torch.equal(torch.isnan(g), torch.isnan(w))
        assert torch.equal(torch.nan_to_num(g, nan=0.0), torch.nan_to_num(w, nan=0.0))
        y_ref, inv = reference(pl, x, W, idx)
        assert_close(g, y_ref, inv, dtype)
        assert lora.lora_tenant_bytes(pl.h, ads[0].tenant) == lora.lora_pool_stats(pl.h)["slot_bytes"]
    finally:
        lora.lora_loader_destroy(ld)
        pr.close()
        if pl is not None:
            pl.close()


def test_many_loads_reuse_the_staging_buffers():
    # 3 pools x 6 slots = 18 loads through 2 staging buffers; tickets waited
    # in reverse order (earlier ones were committed when their buffer was
    # reused).
    T, d_in, d_out, S, R = 48, 128, 128, 6, 16
    ld = lora.lora_loader_create(R * (d_in + d_out) * 2)
    pools, regs, cases, all_t = [], [], [], []
    try:
        for k in range(3):
            x, W, ads, idx = _small_case("f16", T, d_in, d_out, S, R, seed=100 + k)
            p, ts = _loaded_pool(ld, "f16", d_in, d_out, R, S, T, ads)
            pools.append(p)
            all_t += ts
            r = Pool(d_in, d_out, R, S, T, "f16", 0, 4)
            r.register_all(ads)
            regs.append(r)
            cases.append((x, W, idx))
        for t in reversed(all_t):
            lora.lora_load_wait(ld, t)
        for t in all_t:
            assert lora.lora_load_poll(ld, t)
        for p, r, (x, W, idx) in zip(pools, regs, cases):
            a = p.apply(dev(x), dev(W), dev(idx)).cpu()
            b = r.apply(dev(x), dev(W), dev(idx)).cpu()
            assert torch.equal(torch.nan_to_num(a, nan=0.0), torch.nan_to_num(b, nan=0.0))
    finally:
        lora.lora_loader_destroy(ld)
        for p in pools + regs:
            p.close()


def test_loading_slot_is_not_routable_until_committed():
    T, d_in, d_out, S, R = 16, 64, 64, 3, 8
    x, W, ads, idx = _small_case("f16", T, d_in, d_out, S, R, seed=7)
    ld = lora.lora_loader_create(R * (d_in + d_out) * 2)
    p = Pool(d_in, d_out, R, S, T, "f16", 0, 4)
    try:
        lora.lora_set_tenant_quota(p.h, 0, BIG_QUOTA)
        a = ads[0]
        t = lora.lora_load_async(ld, p.h, 0, 0, a.A.contiguous(), a.B.contiguous(), a.rank, a.alpha)
        # Not committed yet: LOADING, not active; a token naming it is invalid.
        assert lora.lora_pool_stats(p.h)["active_slots"] == 0
        only0 = torch.zeros(T, dtype=torch.int32)
        p.poll_errors()
        y = p.apply(dev(x), dev(W), dev(only0))
        torch.cuda.synchronize()
        assert bool(torch.isnan(y.cpu()).all())
        assert p.poll_errors() == T
        # A second load into the LOADING slot is refused.
        with pytest.raises(lora.LoraError) as ei:
            lora.lora_load_async(ld, p.h, 0, 0, a.A.contiguous(), a.B.contiguous(), a.rank, a.alpha)
        assert ei.value.status == lora.LORA_ESLOT_BUSY
        # Poll until done (bounded), then the slot routes.
        deadline = time.time() + 10.0
        while not lora.lora_load_poll(ld, t):
            assert time.time() < deadline
            time.sleep(0.001)
        assert lora.lora_pool_stats(p.h)["active_slots"] == 1
        p.adapters[0] = (a.A.cpu(), a.B.cpu(), a.rank, a.alpha)
        y = p.apply(dev(x), dev(W), dev(only0))
        torch.cuda.synchronize()
        y_ref, inv = reference(p, x, W, only0)
        assert_close(y.cpu(), y_ref, inv, "f16")
        # Unregister works on a loaded slot.
        p.unregister(0)
        assert lora.lora_pool_stats(p.h)["active_slots"] == 0
    finally:
        lora.lora_loader_destroy(ld)
        p.close()


def test_loader_errors_change_nothing():
    d_in, d_out, S, R = 64, 64, 3, 8
    ld = lora.lora_loader_create(8 * (d_in + d_out) * 2)
    small = lora.lora_loader_create(64)
    p = Pool(d_in, d_out, R, S, 4, "f16", 0, 4)
    try:
        A = torch.randn(8, d_in).to(torch.float16)
        B = torch.randn(d_out, 8).to(torch.float16)
        A9 = torch.randn(9, d_in).to(torch.float16)
        B9 = torch.randn(d_out, 9).to(torch.float16)
        slot_bytes = lora.lora_pool_stats(p.h)["slot_bytes"]
        lora.lora_set_tenant_quota(p.h, 5, slot_bytes - 1)
        for args, status in [((0, 5, A, B, 8, 16.0), lora.LORA_EQUOTA),      # over quota
                             ((0, 6, A, B, 8, 16.0), lora.LORA_EQUOTA),      # no quota set: default deny
                             ((0, 5, A9, B9, 9, 18.0), lora.LORA_ERANK),     # rank > max_rank
                             ((0, 5, A, B, 8, float("inf")), lora.LORA_EALPHA),
                             ((3, 5, A, B, 8, 16.0), lora.LORA_EINVAL)]:     # slot out of range
            with pytest.raises(lora.LoraError) as ei:
                lora.lora_load_async(ld, p.h, *args)
            assert ei.value.status == status
        with pytest.raises(lora.LoraError) as ei:                           # larger than the loader
            lora.lora_load_async(small, p.h, 0, 5, A, B, 8, 16.0)
        assert ei.value.status == lora.LORA_EINVAL
        st = lora.lora_pool_stats(p.h)
        assert st["active_slots"] == 0 and st["resident_bytes"] == 0
        assert lora.lora_tenant_bytes(p.h, 5) == 0
        # With quota, the same slot loads.
        lora.lora_set_tenant_quota(p.h, 5, slot_bytes)
        t = lora.lora_load_async(ld, p.h, 0, 5, A, B, 8, 16.0)
        lora.lora_load_wait(ld, t)
        lora.lora_load_wait(ld, t)  # committed already: OK
        assert lora.lora_pool_stats(p.h)["active_slots"] == 1
        with pytest.raises(lora.LoraError) as ei:
            lora.lora_load_wait(ld, t + 100)  # unknown ticket
        assert ei.value.status == lora.LORA_EINVAL
    finally:
        lora.lora_loader_destroy(ld)
        lora.lora_loader_destroy(small)
        p.close()
